// Shared device definitions of libgqa's gfx950 (CDNA4) kernels: the kernel
// argument block, bf16/MFMA vector types and small wave helpers.
//
// Operation (nvfp4-megamoe-kernel commit log, dsv4/kernels/attention: the
// multi-tile FA2 commit -- running max and sum carried across KV tiles with P
// left un-normalised, O divided by the running sum once at the end):
//   per query row: m <- max(m, max_j s_j); alpha = e^(m_old - m);
//   l <- alpha l + sum_j e^(s_j - m); O <- alpha O + sum_j e^(s_j - m) v_j.
// Here every exponent is base 2 with log2(e) folded into the score scale,
// which is the same algebra.
//
// Work decomposition (AstrAI commit log, the commit that packs HB = min(G,
// warps) query heads per block so each K/V tile streams once per block):
// one workgroup per (batch b, kv head g, q-tile, kv split).  The workgroup's
// query rows are the flattened (position p, head-in-group hh) pairs
// rho = p * G + hh of one kv group, so all G query heads that share kv head g
// consume the same K/V tile from LDS.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, 64-lane waves).  Each wave owns
// 32 query rows (the MFMA N dimension) and computes S^T = K Q^T with K as the
// A operand, so a lane holds one query row's scores for 16 keys per 32-key
// block -- the row max/sum reductions stay in-lane plus one exchange with
// lane ^ 32.  P^T then feeds O^T = V^T P^T as the B operand straight from the
// accumulator registers: the K rows are read in a permuted order (bits 2 and
// 3 of the row index swapped) so that accumulator registers 8t..8t+7 of a
// lane hold 8 consecutive keys, which is what the B operand of the next MFMA
// needs.  V is stored transposed in LDS (Vt[d][key]) so the A operand of the
// P.V product is one 16-byte LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// (1.0, 1.0) in bf16: v_dot2 against it sums a packed pair in fp32
constexpr bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  // element strides; dense: (b, h, s); paged Q/O: (unused, h, t)
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  const int32_t* kv_len;   // [B] or nullptr (= Skv)
  const float* sink;       // [Hq] scaled-domain logits or nullptr
  float2* ws_ml;           // partial mode: {m, l} per (row, split)
  float* ws_o;             // partial mode: O~ per (row, split, d)
  const int32_t* cu_seqlens_q;  // paged: [B + 1]
  const int32_t* page_table;    // paged: [B, max_pages]
  int64_t kv_sp, kv_sr;         // paged: page and in-page row strides (head stride in k_sh)
  int32_t max_pages;
  int32_t B, Hq, Hkv, G, Sq, Skv;
  int32_t causal;
  int32_t tile;       // keys per split (0 = the whole range)
  int32_t n_split;
  int32_t spw;        // consecutive splits per workgroup (stream kernel; 1 elsewhere)
  int32_t n_qtiles;   // q-tiles per (b, g)
  int32_t total_q;    // paged: packed query rows (partial-state row = h * total_q + t)
  float scale_log2;   // scale * log2(e), > 0
  // paged append (stream kernel): the K/V of the query tokens, packed like Q
  // ([total_q, Hkv, d] by (t, h) strides), or nullptr.  Token i of sequence b
  // holds key row kv_len_b - q_len_b + i, which the kernel attends from here
  // and writes into its cache page.
  const uint16_t* k_new;
  const uint16_t* v_new;
  int64_t new_st, new_sh;
  // in-kernel merge (stream kernel, partial mode): one ticket per (b, kv
  // head, q-tile), zero on entry and left zero; nullptr = merge kernel
  int32_t* tickets;
  // partial mode, shared-tile kernel: an empty state's O~ (all zeros) is left
  // unwritten; set only where the library's own merge, which gives such a
  // state weight 0 without reading it, follows
  int32_t skip_empty_o;
};

// Raw buffer resource (CDNA: stride 0, no swizzle, third dword 0x00020000).
// Loads at offsets at or past `bytes` return zeros without touching memory.
using BufRes = __amdgpu_buffer_rsrc_t;
__device__ __forceinline__ BufRes make_bufres(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// Cache policy of the K/V loads.  Where no other workgroup reads a
// workgroup's K/V tiles (one q-tile per (b, kv head, split)), the loads carry
// the non-temporal hint: streamed once, they run faster with it (split-KV
// decode partial kernel, 537 MB: 95.7 -> 80.5 us).  Tiles that several
// q-tiles share keep the default policy: their re-reads hit the L2, and the
// hint cost causal prefill 1.02 -> 1.09 ms.
constexpr int kCpDefault = 0;
constexpr int kCpNonTemporal = 2;  // nt
template <int CP = kCpDefault>
__device__ __forceinline__ u32x4 buf_load16v(BufRes r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP);
}
template <int CP = kCpDefault>
__device__ __forceinline__ uint4 buf_load16(BufRes r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// per-lane offset `off` plus a wave-uniform offset `soff` (held in an SGPR)
template <int CP = kCpDefault>
__device__ __forceinline__ uint4 buf_load16(BufRes r, uint32_t off, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, CP);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ int swap_bits23(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;  // round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float xor32_max(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}
__device__ __forceinline__ float xor32_sum(float x) { return x + __shfl_xor(x, 32, 64); }

// XOR swizzle of the 16-byte slots of a row-major V tile row `key` (DC slots
// per row).  Measured on gfx950: ds_read_b64_tr_b16 is served per 32-lane
// half-wave from 64 four-byte banks, so the four (prefill) or eight (stream)
// key rows one half-wave gathers from must land on disjoint slot groups;
// this swizzle makes both gather shapes, and the b128 row writes,
// bank-conflict free.  Rows of 256 bytes or more (DC >= 16) all start on bank
// 0, so keys 0-7 take eight different 32-byte slot pairs; a 128-byte row
// shares the bank window with its neighbour (key bit 0 picks the half), and
// four 64-byte rows fill a window by themselves.  The value always has bit 0
// clear, which keeps each 32-byte pair together, and stays below DC.
template <int DC>
__device__ __forceinline__ int vslot_swz(int key) {
  static_assert(DC == 4 || DC == 8 || DC == 16 || DC == 32 || DC == 64,
                "head dim 32, 64, 128, 256 or 512");
  if constexpr (DC >= 16)
    return ((key & 3) << 2) | (((key >> 2) & 1) << 1);
  else if constexpr (DC == 8)
    return (((key >> 1) & 1) << 2) | (((key >> 2) & 1) << 1);
  else
    return ((key >> 2) & 1) << 1;
}

// Workgroup barrier that orders LDS only: global loads in flight (prefetch)
// stay in flight across it, unlike __syncthreads(), whose fence also waits
// for them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// f(integral_constant<int, i>) for i = 0 .. N - 1, expanded at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// exp2 with the -inf convention used throughout: exp2(-inf) = 0.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace gqa
