// Host side of libgqa: the C ABI declared in include/gqa.h, argument
// validation and the merge launch.  The attention kernels' launch and the
// per-call choice of kernel form are in launch.hpp (instantiated per head
// dim in dispatch_d*.hip).
//
// Validation follows the AstrAI commit log's binding checks (q-head/kv-head
// divisibility, head-dim contiguity, split-KV scratch layout validated before
// launch) and its NULL-means-absent convention for optional pointers.  Every
// check runs before anything is enqueued; the library never allocates,
// synchronises or reads device memory from the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>

#include "gqa.h"
#include "host_common.hpp"
#include "merge.hpp"

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace gqa_host {

gqa_status_t fail(gqa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

gqa_status_t check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return GQA_OK;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::mutex mu;
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

GQA_EXTERN_DISPATCH(32)
GQA_EXTERN_DISPATCH(64)
GQA_EXTERN_DISPATCH(128)
GQA_EXTERN_DISPATCH(256)
extern template gqa_status_t dispatch_wide<false, false>(gqa::AttnArgs, int64_t, hipStream_t);
extern template gqa_status_t dispatch_wide<false, true>(gqa::AttnArgs, int64_t, hipStream_t);
extern template gqa_status_t dispatch_wide<true, false>(gqa::AttnArgs, int64_t, hipStream_t);
extern template gqa_status_t dispatch_wide<true, true>(gqa::AttnArgs, int64_t, hipStream_t);

}  // namespace gqa_host

// Scratch of gqa_attention_decode_splitkv_noalloc: the split-KV partial
// states live here instead of in a caller workspace.  Each GPU the library
// runs on holds its own copy until the process ends.  Host code never passes
// the name itself to a kernel (on the host it is a stand-in, not a device
// address): the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

namespace {

using gqa_host::cdiv;
using gqa_host::check_launch;
using gqa_host::dispatch_rows;
using gqa_host::dispatch_wide;
using gqa_host::fail;

gqa_status_t ok() {
  g_err[0] = '\0';
  return GQA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// (b, h, s) element strides of a bf16 tensor must keep 16-byte rows aligned.
gqa_status_t check_strides(const char* name, const int64_t* st, int n) {
  if (!st) return fail(GQA_ERR_INVALID_ARGUMENT, "%s strides are NULL", name);
  for (int i = 0; i < n; ++i) {
    if (st[i] < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "%s stride %d is negative", name, i);
    if (st[i] % 8 != 0)
      return fail(GQA_ERR_UNSUPPORTED, "%s stride %d (%lld) is not a multiple of 8 elements",
                  name, i, (long long)st[i]);
  }
  return GQA_OK;
}

gqa_status_t check_ptr(const char* name, const void* p) {
  if (!p) return fail(GQA_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(GQA_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  return GQA_OK;
}

gqa_status_t check_scale(float scale) {
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(GQA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  return GQA_OK;
}

bool head_dim_ok(int32_t d) { return d == 32 || d == 64 || d == 128 || d == 256 || d == 512; }

gqa_status_t check_heads(int32_t Hq, int32_t Hkv, int32_t d) {
  if (Hq < 1 || Hkv < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "Hq and Hkv must be >= 1");
  if (Hq % Hkv != 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
  if (!head_dim_ok(d)) return fail(GQA_ERR_UNSUPPORTED, "head dim %d (supported: 32, 64, 128, 256, 512)", d);
  return GQA_OK;
}

size_t workspace_bytes_for(int64_t rows, int64_t n_split, int64_t d) {
  const int64_t raw = rows * n_split * (d + 2) * 4;
  return (size_t)((raw + 255) / 256 * 256);
}

#define GQA_TRY(...)                     \
  do {                                   \
    gqa_status_t st_ = (__VA_ARGS__);    \
    if (st_ != GQA_OK) return st_;       \
  } while (0)

// ---------------------------------------------------------------- launching

template <bool PAGED, bool PARTIAL>
gqa_status_t dispatch(gqa::AttnArgs args, int d, int64_t rows, hipStream_t stream) {
  switch (d) {
    case 32: return dispatch_rows<32, PAGED, PARTIAL>(args, rows, stream);
    case 64: return dispatch_rows<64, PAGED, PARTIAL>(args, rows, stream);
    case 128: return dispatch_rows<128, PAGED, PARTIAL>(args, rows, stream);
    case 256: return dispatch_rows<256, PAGED, PARTIAL>(args, rows, stream);
    default: return dispatch_wide<PAGED, PARTIAL>(args, rows, stream);
  }
}

gqa_status_t launch_merge(const void* workspace, void* o, const int64_t* os, int32_t B,
                          int32_t Hq, int32_t Sq, int32_t d, int32_t n_split, const float* sink,
                          hipStream_t stream, bool sparse = false) {
  const int64_t rows = (int64_t)B * Hq * Sq;
  if (rows == 0) return GQA_OK;
  const float2* ml = reinterpret_cast<const float2*>(workspace);
  const float* ot = reinterpret_cast<const float*>(reinterpret_cast<const char*>(workspace) +
                                                   (size_t)rows * n_split * 8);
  // d = 128 merges with fewer rows than 8 per CU (decode) keep one row per
  // wave; larger ones and the other head dims take the packed form
  const bool one_row = d == 128 && rows < 8 * (int64_t)gqa_host::device_cus();
  using gqa::kMergePackedLpr;
  const int rpb = d == 32    ? gqa::MergeCfg<32, kMergePackedLpr<32>>::ROWS_PER_BLOCK
                  : d == 64  ? gqa::MergeCfg<64, kMergePackedLpr<64>>::ROWS_PER_BLOCK
                  : d == 128 ? (one_row ? gqa::MergeCfg<128, 64>::ROWS_PER_BLOCK
                                        : gqa::MergeCfg<128, kMergePackedLpr<128>>::ROWS_PER_BLOCK)
                  : d == 256 ? gqa::MergeCfg<256, kMergePackedLpr<256>>::ROWS_PER_BLOCK
                             : gqa::MergeCfg<512, kMergePackedLpr<512>>::ROWS_PER_BLOCK;
  const int64_t nblocks = cdiv(rows, rpb);
  if (nblocks * 256 > 0xffffffffLL)  // work-items of one dispatch: 32 bits
    return fail(GQA_ERR_UNSUPPORTED, "merge grid too large (%lld rows)", (long long)rows);
  (void)hipGetLastError();
  auto pick = [&](auto sp) {
    constexpr bool S = decltype(sp)::value;
    return d == 32    ? gqa::merge_kernel<32, S, kMergePackedLpr<32>>
           : d == 64  ? gqa::merge_kernel<64, S, kMergePackedLpr<64>>
           : d == 128 ? (one_row ? gqa::merge_kernel<128, S, 64>
                                 : gqa::merge_kernel<128, S, kMergePackedLpr<128>>)
           : d == 256 ? gqa::merge_kernel<256, S, kMergePackedLpr<256>>
                      : gqa::merge_kernel<512, S, kMergePackedLpr<512>>;
  };
  auto kern = sparse ? pick(std::true_type{}) : pick(std::false_type{});
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(256), 0, stream, ml, ot,
                     reinterpret_cast<uint16_t*>(o), os[0], os[1], os[2], sink, Hq, Sq, n_split,
                     rows);
  return check_launch("merge kernel");
}

gqa::AttnArgs dense_args(const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                         const void* v, const int64_t* vs, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t Sq, int32_t Skv, const int32_t* kv_len, float scale,
                         int32_t causal) {
  gqa::AttnArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k);
  a.v = reinterpret_cast<const uint16_t*>(v);
  a.q_sb = qs[0]; a.q_sh = qs[1]; a.q_ss = qs[2];
  a.k_sb = ks[0]; a.k_sh = ks[1]; a.k_ss = ks[2];
  a.v_sb = vs[0]; a.v_sh = vs[1]; a.v_ss = vs[2];
  a.kv_len = kv_len;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv; a.Sq = Sq; a.Skv = Skv;
  a.causal = causal;
  a.tile = 0;
  a.n_split = 1;
  a.scale_log2 = scale * gqa::kLog2e;
  return a;
}

// Shared checks of the dense entry points.
// K/V tiles are read through buffer resources whose per-lane offsets and
// size are 32-bit byte counts spanning up to 63 key rows past the tile's
// first (the prefill kernel's 64-key tiles): 63 * stride * 2 + 512 bytes
// stays below 2^32 for every stride below 2^25 elements.
constexpr int64_t kMaxKeyStride = (int64_t)1 << 25;
gqa_status_t check_key_stride(const char* name, int64_t st) {
  if (st >= kMaxKeyStride)
    return fail(GQA_ERR_UNSUPPORTED, "%s key-row stride (%lld) must be below 2^25 elements", name,
                (long long)st);
  return GQA_OK;
}

gqa_status_t check_dense(const void* q, const int64_t* qs, const void* k, const int64_t* ks,
                         const void* v, const int64_t* vs, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t Sq, int32_t Skv, int32_t d, float scale, int32_t causal) {
  if (B < 0 || Sq < 0 || Skv < 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "B, Sq and Skv must be >= 0");
  GQA_TRY(check_heads(Hq, Hkv, d));
  GQA_TRY(check_scale(scale));
  if (causal != 0 && causal != 1) return fail(GQA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  if ((int64_t)B * Sq == 0) return GQA_OK;  // empty: nothing is read or written
  GQA_TRY(check_ptr("q", q));
  GQA_TRY(check_ptr("k", k));
  GQA_TRY(check_ptr("v", v));
  GQA_TRY(check_strides("q", qs, 3));
  GQA_TRY(check_strides("k", ks, 3));
  GQA_TRY(check_strides("v", vs, 3));
  GQA_TRY(check_key_stride("k", ks[2]));
  GQA_TRY(check_key_stride("v", vs[2]));
  return GQA_OK;
}

gqa_status_t check_tile(int32_t tile, bool required) {
  if (tile < 0 || tile % 64 != 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "tile_s_kv (%d) must be 0 or a positive multiple of 64", tile);
  if (required && tile == 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "tile_s_kv must be a positive multiple of 64");
  return GQA_OK;
}

gqa_status_t check_workspace(const void* ws, size_t have, size_t need) {
  if (need == 0) return GQA_OK;
  if (!ws) return fail(GQA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned16(ws)) return fail(GQA_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  if (have < need)
    return fail(GQA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return GQA_OK;
}

// The partial phase (validated arguments).
gqa_status_t run_partial(gqa::AttnArgs a, int32_t d, int32_t tile, void* ws, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const int64_t n_split = a.Skv > 0 ? cdiv(a.Skv, tile) : 1;
  a.tile = tile;
  a.n_split = (int32_t)n_split;
  a.ws_ml = reinterpret_cast<float2*>(ws);
  a.ws_o = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (size_t)rows * n_split * 8);
  return dispatch<false, true>(a, d, (int64_t)a.Sq * a.G, stream);
}

}  // namespace

extern "C" {

int32_t gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char* gqa_last_error(void) { return g_err; }

gqa_status_t gqa_attention_workspace_size(int64_t B, int64_t Hq, int64_t Sq, int64_t Skv,
                                          int64_t d, int32_t tile_s_kv, size_t* bytes) {
  if (!bytes) return fail(GQA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (B < 0 || Hq < 0 || Sq < 0 || Skv < 0 || d < 0 || tile_s_kv < 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "negative size");
  if (tile_s_kv == 0) {
    *bytes = 0;
    return ok();
  }
  const int64_t n_split = Skv > 0 ? cdiv(Skv, tile_s_kv) : 1;
  *bytes = workspace_bytes_for(B * Hq * Sq, n_split, d);
  return ok();
}

gqa_status_t gqa_attention_prefill(const void* q, const int64_t q_stride[3], const void* k,
                                   const int64_t k_stride[3], const void* v,
                                   const int64_t v_stride[3], void* o, const int64_t o_stride[3],
                                   int32_t B, int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Skv,
                                   int32_t d, const int32_t* kv_len, float scale,
                                   const float* sink, int32_t causal, int32_t tile_s_kv,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  GQA_TRY(check_dense(q, q_stride, k, k_stride, v, v_stride, B, Hq, Hkv, Sq, Skv, d, scale, causal));
  GQA_TRY(check_tile(tile_s_kv, false));
  const int64_t rows = (int64_t)B * Hq * Sq;
  if (rows == 0) return ok();
  GQA_TRY(check_ptr("o", o));
  GQA_TRY(check_strides("o", o_stride, 3));
  size_t need = 0;
  if (tile_s_kv > 0)
    need = workspace_bytes_for(rows, Skv > 0 ? cdiv(Skv, tile_s_kv) : 1, d);
  GQA_TRY(check_workspace(workspace, workspace_bytes, need));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  gqa::AttnArgs a = dense_args(q, q_stride, k, k_stride, v, v_stride, B, Hq, Hkv, Sq, Skv,
                               kv_len, scale, causal);
  if (tile_s_kv == 0) {
    a.o = reinterpret_cast<uint16_t*>(o);
    a.o_sb = o_stride[0]; a.o_sh = o_stride[1]; a.o_ss = o_stride[2];
    a.sink = sink;
    GQA_TRY(dispatch<false, false>(a, d, (int64_t)Sq * a.G, st));
    return ok();
  }
  // Causal groups of more than 64 rows have many empty states (splits past a
  // q-tile's diagonal): the partial kernel leaves their O~ unwritten and the
  // sparse merge reads only the states that hold keys.  Elsewhere every state
  // is written (an empty one as zeros) and the merge issues all its loads in
  // one round: short-q/long-kv (B 16, Hkv 4, 16384 keys, splits of 4096)
  // 113-119 -> 109-112 us for the step.
  const bool sparse = (int64_t)Sq * a.G > 64 && causal;
  a.skip_empty_o = sparse;
  GQA_TRY(run_partial(a, d, tile_s_kv, workspace, st));
  GQA_TRY(launch_merge(workspace, o, o_stride, B, Hq, Sq, d, a.Skv > 0 ? (int32_t)cdiv(Skv, tile_s_kv) : 1,
                       sink, st, sparse));
  return ok();
}

gqa_status_t gqa_attention_decode_splitkv(const void* q, const int64_t q_stride[3], const void* k,
                                          const int64_t k_stride[3], const void* v,
                                          const int64_t v_stride[3], void* o,
                                          const int64_t o_stride[3], int32_t B, int32_t Hq,
                                          int32_t Hkv, int32_t Skv, int32_t d,
                                          const int32_t* kv_len, float scale, const float* sink,
                                          int32_t tile_s_kv, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  GQA_TRY(check_tile(tile_s_kv, true));
  return gqa_attention_prefill(q, q_stride, k, k_stride, v, v_stride, o, o_stride, B, Hq, Hkv, 1,
                               Skv, d, kv_len, scale, sink, 0, tile_s_kv, workspace,
                               workspace_bytes, stream);
}

gqa_status_t gqa_attention_decode_tile(int32_t B, int32_t Hkv, int32_t Skv, int32_t* tile_s_kv) {
  if (!tile_s_kv) return fail(GQA_ERR_INVALID_ARGUMENT, "tile_s_kv is NULL");
  if (B < 1 || Hkv < 1 || Skv < 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "B and Hkv must be >= 1 and Skv >= 0");
  const int64_t cus = gqa_host::device_cus();
  int32_t tile = 128;
  while (tile < 8192 && (int64_t)B * Hkv * cdiv(Skv, tile) > cus) tile *= 2;
  *tile_s_kv = tile;
  return ok();
}

gqa_status_t gqa_attention_decode_splitkv_fused(
    const void* q, const int64_t q_stride[3], const void* k, const int64_t k_stride[3],
    const void* v, const int64_t v_stride[3], void* o, const int64_t o_stride[3], int32_t B,
    int32_t Hq, int32_t Hkv, int32_t Skv, int32_t d, const int32_t* kv_len, float scale,
    const float* sink, int32_t tile_s_kv, void* workspace, size_t workspace_bytes,
    int32_t* tickets, int64_t n_tickets, void* stream) {
  GQA_TRY(check_dense(q, q_stride, k, k_stride, v, v_stride, B, Hq, Hkv, 1, Skv, d, scale, 0));
  GQA_TRY(check_tile(tile_s_kv, true));
  if (Hq / Hkv > 32)
    return fail(GQA_ERR_UNSUPPORTED, "in-kernel merge handles groups of up to 32 heads (G = %d)",
                Hq / Hkv);
  if (d == 512) return fail(GQA_ERR_UNSUPPORTED, "in-kernel merge handles head dims up to 256");
  const int64_t rows = (int64_t)B * Hq;
  if (rows == 0) return ok();
  GQA_TRY(check_ptr("o", o));
  GQA_TRY(check_strides("o", o_stride, 3));
  if (!tickets) return fail(GQA_ERR_INVALID_ARGUMENT, "tickets is NULL");
  if (n_tickets < rows)
    return fail(GQA_ERR_WORKSPACE, "tickets holds %lld entries, needs B * Hq = %lld",
                (long long)n_tickets, (long long)rows);
  GQA_TRY(check_workspace(workspace, workspace_bytes,
                          workspace_bytes_for(rows, Skv > 0 ? cdiv(Skv, tile_s_kv) : 1, d)));
  gqa::AttnArgs a = dense_args(q, q_stride, k, k_stride, v, v_stride, B, Hq, Hkv, 1, Skv, kv_len,
                               scale, 0);
  a.o = reinterpret_cast<uint16_t*>(o);
  a.o_sb = o_stride[0]; a.o_sh = o_stride[1]; a.o_ss = o_stride[2];
  a.sink = sink;
  a.tickets = tickets;
  GQA_TRY(run_partial(a, d, tile_s_kv, workspace, reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

gqa_status_t gqa_attention_decode_splitkv_noalloc(
    const void* q, const int64_t q_stride[3], const void* k, const int64_t k_stride[3],
    const void* v, const int64_t v_stride[3], void* o, const int64_t o_stride[3], int32_t B,
    int32_t Hq, int32_t Hkv, int32_t Skv, int32_t d, const int32_t* kv_len, float scale,
    const float* sink, int32_t tile_s_kv, void* stream) {
  // every host-side check first, so that no size or argument error touches
  // a device
  GQA_TRY(check_tile(tile_s_kv, true));
  GQA_TRY(check_dense(q, q_stride, k, k_stride, v, v_stride, B, Hq, Hkv, 1, Skv, d, scale, 0));
  const int64_t rows = (int64_t)B * Hq;
  if (rows == 0) return ok();
  GQA_TRY(check_ptr("o", o));
  GQA_TRY(check_strides("o", o_stride, 3));
  const size_t need = workspace_bytes_for(rows, Skv > 0 ? cdiv(Skv, tile_s_kv) : 1, d);
  if (need > (size_t)GQA_NOALLOC_SCRATCH_BYTES)
    return fail(GQA_ERR_WORKSPACE,
                "no-alloc decode needs %zu bytes of partial states; the library's scratch holds "
                "%zu (fewer rows or larger splits fit)",
                need, (size_t)GQA_NOALLOC_SCRATCH_BYTES);
  // the scratch's device address, looked up once per device with that
  // device current; later calls reuse it
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(GQA_ERR_UNSUPPORTED, "device %d (up to 64 supported)", dev);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(GQA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      addr[dev] = p;
    }
    ws = addr[dev];
  }
  return gqa_attention_decode_splitkv(q, q_stride, k, k_stride, v, v_stride, o, o_stride, B, Hq,
                                      Hkv, Skv, d, kv_len, scale, sink, tile_s_kv, ws,
                                      (size_t)GQA_NOALLOC_SCRATCH_BYTES, stream);
}

gqa_status_t gqa_attention_splitkv_partial(const void* q, const int64_t q_stride[3],
                                           const void* k, const int64_t k_stride[3],
                                           const void* v, const int64_t v_stride[3], int32_t B,
                                           int32_t Hq, int32_t Hkv, int32_t Sq, int32_t Skv,
                                           int32_t d, const int32_t* kv_len, float scale,
                                           int32_t causal, int32_t tile_s_kv, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  GQA_TRY(check_dense(q, q_stride, k, k_stride, v, v_stride, B, Hq, Hkv, Sq, Skv, d, scale, causal));
  GQA_TRY(check_tile(tile_s_kv, true));
  const int64_t rows = (int64_t)B * Hq * Sq;
  if (rows == 0) return ok();
  const size_t need = workspace_bytes_for(rows, Skv > 0 ? cdiv(Skv, tile_s_kv) : 1, d);
  GQA_TRY(check_workspace(workspace, workspace_bytes, need));
  gqa::AttnArgs a = dense_args(q, q_stride, k, k_stride, v, v_stride, B, Hq, Hkv, Sq, Skv,
                               kv_len, scale, causal);
  GQA_TRY(run_partial(a, d, tile_s_kv, workspace, reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

gqa_status_t gqa_attention_splitkv_merge(const void* workspace, size_t workspace_bytes, void* o,
                                         const int64_t o_stride[3], int32_t B, int32_t Hq,
                                         int32_t Sq, int32_t d, int32_t n_split,
                                         const float* sink, void* stream) {
  if (B < 0 || Sq < 0) return fail(GQA_ERR_INVALID_ARGUMENT, "B and Sq must be >= 0");
  if (Hq < 1 || n_split < 1) return fail(GQA_ERR_INVALID_ARGUMENT, "Hq and n_split must be >= 1");
  if (!head_dim_ok(d)) return fail(GQA_ERR_UNSUPPORTED, "head dim %d (supported: 32, 64, 128, 256, 512)", d);
  const int64_t rows = (int64_t)B * Hq * Sq;
  if (rows == 0) return ok();
  GQA_TRY(check_ptr("o", o));
  GQA_TRY(check_strides("o", o_stride, 3));
  GQA_TRY(check_workspace(workspace, workspace_bytes, workspace_bytes_for(rows, n_split, d)));
  GQA_TRY(launch_merge(workspace, o, o_stride, B, Hq, Sq, d, n_split, sink,
                       reinterpret_cast<hipStream_t>(stream)));
  return ok();
}

}  // extern "C"

namespace {

// gqa_attention_paged and gqa_attention_paged_append (k_new == nullptr: no append)
gqa_status_t paged_impl(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                        const int32_t* cu_seqlens_q, const void* k_cache, const void* v_cache,
                        int64_t kv_stride_page, int64_t kv_stride_row, int64_t kv_stride_h,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        const int32_t* kv_len, const void* k_new, const void* v_new,
                        int64_t new_stride_t, int64_t new_stride_h, void* o, int64_t o_stride_t,
                        int64_t o_stride_h, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                        int32_t page_size, int32_t total_q, int32_t max_q_len, float scale,
                        const float* sink, int32_t causal, int32_t tile_s_kv, void* workspace,
                        size_t workspace_bytes, void* stream, bool append) {
  if (B < 0 || total_q < 0 || max_q_len < 0 || max_pages_per_seq < 0)
    return fail(GQA_ERR_INVALID_ARGUMENT, "B, total_q, max_q_len and max_pages_per_seq must be >= 0");
  GQA_TRY(check_heads(Hq, Hkv, d));
  if (page_size != 64) return fail(GQA_ERR_UNSUPPORTED, "page_size %d (supported: 64)", page_size);
  GQA_TRY(check_scale(scale));
  if (causal != 0 && causal != 1) return fail(GQA_ERR_INVALID_ARGUMENT, "causal must be 0 or 1");
  GQA_TRY(check_tile(tile_s_kv, false));
  if (append && d == 512) return fail(GQA_ERR_UNSUPPORTED, "append handles head dims up to 256");
  if (append && (int64_t)max_q_len * (Hq / Hkv) > 32)
    return fail(GQA_ERR_UNSUPPORTED,
                "append handles up to 32 query rows per kv head (max_q_len %d x group %d)",
                max_q_len, Hq / Hkv);
  if (B == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (append) {
    GQA_TRY(check_ptr("k_new", k_new));
    GQA_TRY(check_ptr("v_new", v_new));
    const int64_t ns[2] = {new_stride_t, new_stride_h};
    GQA_TRY(check_strides("k_new/v_new", ns, 2));
    GQA_TRY(check_key_stride("k_new/v_new", new_stride_t));
  }
  GQA_TRY(check_ptr("q", q));
  GQA_TRY(check_ptr("o", o));
  GQA_TRY(check_ptr("k_cache", k_cache));
  GQA_TRY(check_ptr("v_cache", v_cache));
  if (!cu_seqlens_q) return fail(GQA_ERR_INVALID_ARGUMENT, "cu_seqlens_q is NULL");
  if (!page_table) return fail(GQA_ERR_INVALID_ARGUMENT, "page_table is NULL");
  if (!kv_len) return fail(GQA_ERR_INVALID_ARGUMENT, "kv_len is NULL (required for paged)");
  const int64_t qs[2] = {q_stride_t, q_stride_h};
  const int64_t os[2] = {o_stride_t, o_stride_h};
  const int64_t kvs[3] = {kv_stride_page, kv_stride_row, kv_stride_h};
  GQA_TRY(check_strides("q", qs, 2));
  GQA_TRY(check_strides("o", os, 2));
  GQA_TRY(check_strides("kv", kvs, 3));
  GQA_TRY(check_key_stride("kv", kv_stride_row));
  if ((int64_t)max_pages_per_seq * page_size > 0x7fffffffLL)
    return fail(GQA_ERR_UNSUPPORTED, "max_pages_per_seq too large");
  const int32_t Skv = max_pages_per_seq * page_size;
  const int64_t n_split = tile_s_kv > 0 ? (Skv > 0 ? cdiv(Skv, tile_s_kv) : 1) : 1;
  if (tile_s_kv > 0)
    GQA_TRY(check_workspace(workspace, workspace_bytes,
                            workspace_bytes_for((int64_t)Hq * total_q, n_split, d)));

  gqa::AttnArgs a{};
  a.q = reinterpret_cast<const uint16_t*>(q);
  a.k = reinterpret_cast<const uint16_t*>(k_cache);
  a.v = reinterpret_cast<const uint16_t*>(v_cache);
  a.o = reinterpret_cast<uint16_t*>(o);
  a.q_ss = q_stride_t; a.q_sh = q_stride_h;
  a.o_ss = o_stride_t; a.o_sh = o_stride_h;
  a.k_sh = kv_stride_h; a.v_sh = kv_stride_h;
  a.kv_sp = kv_stride_page; a.kv_sr = kv_stride_row;
  a.kv_len = kv_len;
  a.cu_seqlens_q = cu_seqlens_q;
  a.page_table = page_table;
  a.max_pages = max_pages_per_seq;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.Sq = max_q_len;
  a.Skv = Skv;
  a.total_q = total_q;
  a.causal = causal;
  a.scale_log2 = scale * gqa::kLog2e;
  if (append) {
    a.k_new = reinterpret_cast<const uint16_t*>(k_new);
    a.v_new = reinterpret_cast<const uint16_t*>(v_new);
    a.new_st = new_stride_t;
    a.new_sh = new_stride_h;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int64_t rows = (int64_t)max_q_len * a.G;
  if (tile_s_kv == 0) {
    a.tile = 0;
    a.n_split = 1;
    a.sink = sink;
    GQA_TRY(dispatch<true, false>(a, d, rows, st));
    return ok();
  }
  a.tile = tile_s_kv;
  a.n_split = (int32_t)n_split;
  a.ws_ml = reinterpret_cast<float2*>(workspace);
  a.ws_o = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) +
                                    (size_t)Hq * total_q * n_split * 8);
  // ragged sequences leave many states empty (the splits past a sequence's
  // keys): their O~ stays unwritten, and the merge of groups of more than 64
  // rows reads only the states that hold keys
  a.skip_empty_o = 1;
  GQA_TRY(dispatch<true, true>(a, d, rows, st));
  // partial rows are h * total_q + t: the merge sees B = 1, Sq = total_q
  const int64_t mo[3] = {0, o_stride_h, o_stride_t};
  GQA_TRY(launch_merge(workspace, o, mo, 1, Hq, total_q, d, (int32_t)n_split, sink, st,
                       rows > 64));
  return ok();
}

}  // namespace

extern "C" {

gqa_status_t gqa_attention_paged(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                                 const int32_t* cu_seqlens_q, const void* k_cache,
                                 const void* v_cache, int64_t kv_stride_page,
                                 int64_t kv_stride_row, int64_t kv_stride_h,
                                 const int32_t* page_table, int32_t max_pages_per_seq,
                                 const int32_t* kv_len, void* o, int64_t o_stride_t,
                                 int64_t o_stride_h, int32_t B, int32_t Hq, int32_t Hkv, int32_t d,
                                 int32_t page_size, int32_t total_q, int32_t max_q_len,
                                 float scale, const float* sink, int32_t causal,
                                 int32_t tile_s_kv, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return paged_impl(q, q_stride_t, q_stride_h, cu_seqlens_q, k_cache, v_cache, kv_stride_page,
                    kv_stride_row, kv_stride_h, page_table, max_pages_per_seq, kv_len, nullptr,
                    nullptr, 0, 0, o, o_stride_t, o_stride_h, B, Hq, Hkv, d, page_size, total_q,
                    max_q_len, scale, sink, causal, tile_s_kv, workspace, workspace_bytes, stream,
                    false);
}

gqa_status_t gqa_attention_paged_append(
    const void* q, int64_t q_stride_t, int64_t q_stride_h, const int32_t* cu_seqlens_q,
    void* k_cache, void* v_cache, int64_t kv_stride_page, int64_t kv_stride_row,
    int64_t kv_stride_h, const int32_t* page_table, int32_t max_pages_per_seq,
    const int32_t* kv_len, const void* k_new, const void* v_new, int64_t new_stride_t,
    int64_t new_stride_h, void* o, int64_t o_stride_t, int64_t o_stride_h, int32_t B, int32_t Hq,
    int32_t Hkv, int32_t d, int32_t page_size, int32_t total_q, int32_t max_q_len, float scale,
    const float* sink, int32_t causal, int32_t tile_s_kv, void* workspace,
    size_t workspace_bytes, void* stream) {
  return paged_impl(q, q_stride_t, q_stride_h, cu_seqlens_q, k_cache, v_cache, kv_stride_page,
                    kv_stride_row, kv_stride_h, page_table, max_pages_per_seq, kv_len, k_new,
                    v_new, new_stride_t, new_stride_h, o, o_stride_t, o_stride_h, B, Hq, Hkv, d,
                    page_size, total_q, max_q_len, scale, sink, causal, tile_s_kv, workspace,
                    workspace_bytes, stream, true);
}

}  // extern "C"
