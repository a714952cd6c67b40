// Kernel launch and the per-call choice of kernel form (the templates that
// instantiate the attention kernels).  Each dispatch_d<D>.hip instantiates
// dispatch_rows for one head dim, so the kernels of the four head dims
// compile in parallel; gqa_api.hip calls them through dispatch().
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "attn_prefill.hpp"
#include "attn_stream.hpp"
#include "host_common.hpp"

namespace gqa_host {

// Launch one attention kernel instantiation over the (b, g, split, q-tile)
// grid; `rows_per_tile` query rows of a kv group per workgroup.
template <class K>
gqa_status_t launch_grid(K* kern, int lds_bytes, int threads, gqa::AttnArgs args,
                         int64_t q_rows_per_bg, int rows_per_tile, hipStream_t stream,
                         int lds_max = 0) {
  // dynamic LDS above 64 KiB has to be allowed once per kernel and device;
  // the cache is keyed by both and holds every form the library builds on a
  // few devices (past its size the attribute would simply be set on every
  // launch)
  static std::mutex mu;
  static struct { const void* kern; int dev; } done[1024];
  static int ndone = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  {
    std::lock_guard<std::mutex> lock(mu);
    bool seen = false;
    for (int i = 0; i < ndone; ++i)
      seen |= done[i].kern == reinterpret_cast<const void*>(kern) && done[i].dev == dev;
    if (!seen) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         lds_max > lds_bytes ? lds_max : lds_bytes);
      if (e != hipSuccess) return fail(GQA_ERR_HIP, "hipFuncSetAttribute: %s", hipGetErrorString(e));
      if (ndone < 1024) done[ndone++] = {reinterpret_cast<const void*>(kern), dev};
    }
  }
  args.n_qtiles = (int32_t)cdiv(q_rows_per_bg, rows_per_tile);
  if (args.spw < 1) args.spw = 1;
  const int64_t nblocks = (int64_t)args.B * args.Hkv * cdiv(args.n_split, args.spw) * args.n_qtiles;
  if (nblocks <= 0) return GQA_OK;
  // the dispatch packet counts work-items in 32 bits
  if (nblocks * threads > 0xffffffffLL)
    return fail(GQA_ERR_UNSUPPORTED, "grid too large (%lld workgroups)", (long long)nblocks);
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  hipLaunchKernelGGL(kern, dim3((unsigned)nblocks), dim3(threads), lds_bytes, stream, args);
  return check_launch("attention kernel");
}

// The non-temporal form where one q-tile covers the rows of a (b, kv head,
// split).  Only the forms that can see several q-tiles are built in the
// default form too: the 2- and 4-wave forms at d = 64 and 128 take at most
// 64 and 128 rows, one q-tile.  Two key groups take one q-tile only for
// 65-128 rows at d = 128.
template <int D, int NW, bool PAGED, bool PARTIAL, int KS = 1>
gqa_status_t launch_prefill(gqa::AttnArgs args, int64_t rows, hipStream_t stream) {
  using C = gqa::PrefillCfg<D, NW, KS>;
  args.spw = 1;
  if constexpr (KS == 1 || D == 128)
    if (cdiv(rows, C::ROWS) == 1)
      return launch_grid(&gqa::attn_prefill_kernel<D, NW, PAGED, PARTIAL, KS, true>, C::DYN_LDS_BYTES,
                         C::NT, args, rows, C::ROWS, stream);
  if constexpr (NW == 8 || (NW == 4 && (D == 32 || D == 256)))
    return launch_grid(&gqa::attn_prefill_kernel<D, NW, PAGED, PARTIAL, KS, false>, C::DYN_LDS_BYTES,
                       C::NT, args, rows, C::ROWS, stream);
  return fail(GQA_ERR_UNSUPPORTED, "no prefill form for %lld rows at d = %d, %d waves",
              (long long)rows, D, NW);
}


// The non-temporal form where one q-tile covers the group's rows; only 17-32
// rows at d = 256 (one 16-column block per q-tile) take two.
template <int D, int NQB, int NW, bool PAGED, bool PARTIAL, bool KROW = false>
gqa_status_t launch_stream_nw(gqa::AttnArgs args, int64_t rows, hipStream_t stream) {
  using C = gqa::StreamCfg<D, NQB, KROW>;
  const int lds = C::lds_bytes(NW, PARTIAL ? args.spw : 0);
  const int lds_max = C::lds_bytes(NW, PARTIAL ? C::max_spw(NW) : 0);
  if (cdiv(rows, 16 * NQB) == 1)
    return launch_grid(&gqa::attn_stream_kernel<D, NQB, NW, PAGED, PARTIAL, true, KROW>, lds,
                       NW * 64, args, rows, 16 * NQB, stream, lds_max);
  if constexpr (D == 256 && NQB == 1)
    return launch_grid(&gqa::attn_stream_kernel<D, NQB, NW, PAGED, PARTIAL, false>, lds, NW * 64,
                       args, rows, 16 * NQB, stream, lds_max);
  return fail(GQA_ERR_UNSUPPORTED, "no stream form for %lld rows at d = %d", (long long)rows, D);
}

// Launch shape of the stream kernel.  Split-KV runs: each workgroup takes
// `spw` consecutive splits, as many as still leave at least one workgroup
// per CU: HBM streams faster with fewer, longer sequential runs (measured on
// the 16 x 8-head x 8-split decode: 1 split per workgroup 98-99 us, 2 or 4
// splits 95-96 us).  Two waves per workgroup once there are at least as
// many workgroups as CUs (the same decode: 2 waves per workgroup beat 4);
// four when the grid is smaller, to use more of each CU (where the four
// waves' combine slots fit in LDS: not for 32-row groups at d = 256).
template <int D, int NQB, bool PAGED, bool PARTIAL, bool KROW = false>
gqa_status_t launch_stream(gqa::AttnArgs args, int64_t rows, hipStream_t stream) {
  using C = gqa::StreamCfg<D, NQB, KROW>;
  const int64_t cus = device_cus();
  const int64_t per_split = (int64_t)args.B * args.Hkv * cdiv(rows, 16 * NQB);
  int spw = 1;
  if (PARTIAL)
    while (spw * 2 <= C::max_spw(2) && spw * 2 <= args.n_split &&
           per_split * cdiv(args.n_split, spw * 2) >= cus)
      spw *= 2;
  args.spw = spw;
  const int64_t nblocks = per_split * cdiv(args.n_split, spw);
  if constexpr (C::FOUR_WAVES)
    if (nblocks < cus) return launch_stream_nw<D, NQB, 4, PAGED, PARTIAL, KROW>(args, rows, stream);
  return launch_stream_nw<D, NQB, 2, PAGED, PARTIAL, KROW>(args, rows, stream);
}

// Kernel choice by query rows per (b, kv head) and grid size.  Groups of up
// to 32 rows (decode, short query blocks) stream keys per wave in the
// stream kernel; larger groups share K/V tiles across the waves of a
// workgroup, 32 rows per wave (the prefill kernel).  On grids that fill the
// CUs twice or more the shared-tile form takes some short groups too, and on
// grids that fit them in one round it splits a workgroup's keys between two
// wave groups (both below).  The prefill kernel's widths per head dim: a 64-key tile splits into whole
// 16-byte chunks per thread from 2 waves up at d = 32 only up to 4 waves; the
// V swizzle needs 4 or more waves at d = 256, where one workgroup per CU
// with 4 waves (one per SIMD) holds the 32-row O and Q of a wave in
// registers without spilling.
template <int D, bool PAGED, bool PARTIAL>
gqa_status_t dispatch_rows(gqa::AttnArgs args, int64_t rows, hipStream_t stream) {
  // Short groups on the shared-tile prefill form, where its grid (one
  // workgroup per (b, kv head, split)) fills the CUs at least twice: at
  // d <= 64 every group of up to 64 rows, whose 32-key stream tiles carry
  // few bytes per step; at d = 128 and 256 the groups of 17-32 rows (two
  // 16-column blocks, or at d = 256 two q-tiles reading K/V twice).
  // Measured at B 16, Hkv 8, 8192 keys, splits of 1024: decode 52 -> 48 us
  // at d = 64; 32-row groups 112-123 -> 101-102 us at d = 128 and 382 ->
  // 219 us at d = 256 (dense decode at d = 128 stays faster on the stream
  // kernel, 82 against 88 us, and so does paged decode at d = 256, 173
  // against 198 us).  Smaller grids
  // keep the stream kernel, whose launch shape adapts to them (B 1 decode
  // at d = 64: 18 us, 24 us routed).  The fused append and the in-kernel
  // merge live in the stream kernel only.
  if (rows <= 64 && !args.k_new && !args.tickets &&
      (int64_t)args.B * args.Hkv * args.n_split >= 2 * (int64_t)device_cus()) {
    if constexpr (D <= 64) {
      return launch_prefill<D, 2, PAGED, PARTIAL>(args, rows, stream);
    } else if (rows > 16 && rows <= 32) {
      if constexpr (D == 128) return launch_prefill<D, 2, PAGED, PARTIAL>(args, rows, stream);
      if constexpr (D == 256) return launch_prefill<D, 4, PAGED, PARTIAL>(args, rows, stream);
    }
  }
  // Paged groups of up to 16 rows at d = 128 whose pool is token-major (one
  // head's rows of a page 2 KB or more apart): the stream kernel with K
  // loaded as whole rows and staged through LDS.  Its operand-shaped K loads
  // (64-byte pieces of 16 rows per instruction) spread over 32 KB there.
  // Measured at B 16, Hkv 8, 8192 keys, splits of 1024: 96-97 us with
  // operand-shaped K, 91.7 us on the shared-tile form, 90-91 us with whole
  // rows; a pure load loop over the same pool reads it in 89.2 us with the
  // operand shape and 80.5 us with whole rows.  Head-major pools keep the
  // operand shape (84.6 us; whole rows 80.0 against 77.7 us in the loop).
  if constexpr (PAGED && D == 128)
    if (rows <= 16 && args.kv_sr > D)
      return launch_stream<D, 1, PAGED, PARTIAL, true>(args, rows, stream);
  if (rows <= 16) return launch_stream<D, 1, PAGED, PARTIAL>(args, rows, stream);
  if (rows <= 32) {
    // two 16-column blocks of Q do not fit beside the d = 256 tiles: two q-tiles
    if constexpr (D == 256)
      return launch_stream<D, 1, PAGED, PARTIAL>(args, rows, stream);
    else
      return launch_stream<D, 2, PAGED, PARTIAL>(args, rows, stream);
  }
  if constexpr (D == 256) {
    return launch_prefill<D, 4, PAGED, PARTIAL>(args, rows, stream);
  } else {
    if (rows <= 64) return launch_prefill<D, 2, PAGED, PARTIAL>(args, rows, stream);
    if constexpr (D == 128) {
      // 65-128 rows on a grid that fits the CUs in one round: the 8-wave
      // form with two key groups over the 128 rows halves each workgroup's
      // walk (short-q, B 16, Hkv 4, 16384 keys: one pass 350 -> 240 us,
      // splits of 4096 122-142 -> 101-111 us; with splits of 2048, 512
      // workgroups, the 4-wave form two per CU is as fast)
      if (rows <= 128 && (int64_t)args.B * args.Hkv * args.n_split <= device_cus())
        return launch_prefill<D, 8, PAGED, PARTIAL, 2>(args, rows, stream);
    }
    if (D == 32 || rows <= 128) return launch_prefill<D, 4, PAGED, PARTIAL>(args, rows, stream);
    if constexpr (D != 32) {
      // The 8-wave form holds one workgroup per CU.  A grid that fits the
      // CUs in one round leaves no later workgroups to even out the load:
      // its time is the longest key walk of a workgroup, which two key
      // groups per workgroup halve.  Their grid is twice as large, and at
      // 128 rows per tile a CU pulls twice the K/V bytes per flop, so they
      // are taken only where that grid still fits one round, or where the
      // walk is long (32 or more 64-key tiles: the longest one allowed by
      // the split size or the key count).  Measured: ragged paged one pass
      // (56 workgroups) 111 -> 70 us, with splits of 2048 72 -> 52 us, of
      // 1024 (256 workgroups, 16 tiles) 48 us kept; causal 2048^2 at
      // B = 1, Hkv = 8 (256 workgroups, 32 tiles) 62 -> 53 us; causal
      // 4096^2 there (512 workgroups) 137 -> 160 us with two groups, kept.
      using C1 = gqa::PrefillCfg<D, 8>;
      const int64_t per = (int64_t)args.B * args.Hkv * args.n_split;
      const int64_t n1 = per * cdiv(rows, C1::ROWS);
      const int64_t n2 = per * cdiv(rows, gqa::PrefillCfg<D, 8, 2>::ROWS);
      const int64_t keys = args.tile > 0 ? std::min<int64_t>(args.tile, args.Skv) : args.Skv;
      const int64_t cus = device_cus();
      if (n1 <= cus && (n2 <= cus || cdiv(keys, C1::BK) >= 32))
        return launch_prefill<D, 8, PAGED, PARTIAL, 2>(args, rows, stream);
      return launch_prefill<D, 8, PAGED, PARTIAL>(args, rows, stream);
    }
  }
  return GQA_OK;  // not reached
}

}  // namespace gqa_host
