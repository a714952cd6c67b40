// Shared-tile GQA forward kernel: query groups of more than 32 rows per
// (b, kv head), and shorter groups on grids large enough (launch.hpp).  One
// workgroup per (b, kv head g, q-tile of 32 * NW / KS rows, kv split); its
// waves share each 64-key K/V tile through LDS, so a tile
// is fetched once per workgroup for every query head of the group (AstrAI
// commit log, the commit that packs HB = min(G, warps) query heads per
// block).  Each wave owns 32 query rows.  The 8-wave form (d = 64, 128)
// runs one workgroup per CU, two waves per SIMD with up to 256 VGPRs each;
// d = 256 runs 4 waves, one per SIMD, its double-buffered tiles taking
// 130 KiB of LDS.  The 8-wave form can also split a workgroup's keys between
// two groups of 4 waves (KS = 2, PrefillCfg) where the grid is small.
//
// MFMA mapping, v_mfma_f32_32x32x16_bf16 (32 query rows are the N
// dimension):
//   S^T = K Q^T  : A = K rows from LDS, read in a permuted row order (bits 2
//                  and 3 of the row index swapped) so that accumulator
//                  registers 8t..8t+7 of a lane hold 8 consecutive keys;
//                  B = Q in registers.  A lane holds one query row's scores,
//                  so row max/sum reductions are in-lane plus one exchange
//                  with lane ^ 32 (v_permlane32_swap).
//   O^T += V^T P^T: B = P straight from the S^T accumulators (bf16), A = V^T
//                  gathered from the row-major V tile with two
//                  ds_read_b64_tr_b16 per MFMA (within each 16-lane group,
//                  destination lane i, element e comes from source lane
//                  4e + i/4, element i%4).
// K tiles are stored row-major with a padded pitch (D + 8 elements), V tiles
// row-major unpadded with 16-byte slots XOR-swizzled per row (vslot_swz), so
// the row writes, the K operand reads and the transposing V reads are all
// bank-conflict free (checked with the LDS bank-conflict counter).
//
// The 8-wave form with one key group (d = 64, 128: causal and long prefill)
// runs the two waves of each SIMD in ping-pong: each wave alternates an
// MFMA-only phase (S of tile t, then P.V of tile t - 1) and a vector phase
// (softmax of tile t, staging), the two waves of a SIMD half a tile apart,
// with a workgroup barrier at every phase boundary (block "Ping-pong" below).
// The other forms run each 64-key tile as four phases over its two 32-key
// halves, so the softmax (vector ALU) of one half has the other half's MFMAs
// to hide behind inside the wave:
//   1. S_0 = K_0 Q^T
//   2. S_1 = K_1 Q^T          || softmax of S_0
//   3. O += V_0^T P_0^T       || softmax of S_1
//   4. O += V_1^T P_1^T, stage the next tile
// Scheduling group barriers set the interleave; tiles that need masking run
// a separate copy of the step, so no phase has a branch inside it.
//
// Online softmax in base 2 with a lazily moved reference: a row's reference
// m only moves when the max of a half tile exceeds it by more than 8 (log2
// units), so the O / l rescale is skipped almost always; P = 2^(s - m) <=
// 2^8 then.  The algebra is unchanged -- (m, l, O) stay consistent -- and the
// final division by l happens once (nvfp4-megamoe-kernel commit log,
// multi-tile FA2 and normalise-once commits).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace gqa {

// KS = 2 splits the workgroup's key range between two groups of NW / 2
// waves over the same rows (alternate tiles, each group with its own pair of
// LDS stages); the groups combine their (m, l, O) in LDS at the end.  It
// halves the longest key walk of a workgroup where the grid is too small for
// the load to even out across CUs.
template <int D, int NW, int KS = 1>
struct PrefillCfg {
  static_assert(KS == 1 || KS == 2, "key groups per workgroup");
  static constexpr int BK = 64;              // keys per tile
  static constexpr int DC = D / 8;           // 16-byte chunks per row
  static constexpr int NT = NW * 64;
  static constexpr int NWH = NW / KS;        // waves per key group
  static constexpr int NTH = NWH * 64;       // threads per key group (they stage its tiles)
  static constexpr int ROWS = 32 * NWH;      // query rows per workgroup
  static constexpr int KP = D + 8;           // K row pitch (elements): padded, not swizzled
  static constexpr int KTILE = BK * KP;      // elements of one K tile
  static constexpr int TILE = BK * D;        // elements of one V tile
  static constexpr int STAGE = KTILE + TILE; // K then V
  static constexpr int LDS_BYTES = KS * 2 * STAGE * 2;
  // The cross-tile pipelined form (4 waves, one key group, d = 256) keeps
  // its two stages in static LDS arrays, filled by LDS DMA: no dynamic LDS.
  static constexpr bool XP = NW == 4 && KS == 1 && D == 256;
  static constexpr int DYN_LDS_BYTES = XP ? 0 : LDS_BYTES;
  // the launch bound's minimum waves per SIMD (it caps the registers a wave
  // may take): 2 where two sets of stages fit in 160 KiB of LDS, else 1
  // (d = 256, or two key groups at d = 128).  An 8-wave workgroup is 2 waves
  // per SIMD either way, one workgroup per CU.
  static constexpr int MIN_WAVES_PER_SIMD = 2 * LDS_BYTES <= 160 * 1024 ? 2 : 1;
  static constexpr int CPT = BK * DC / NTH;  // chunks per thread per tensor
  static_assert(CPT >= 1 && BK * DC % NTH == 0 && NTH % DC == 0, "tile split");
  static_assert((NTH / DC) % 8 == 0, "chunk rows keep the V swizzle");
  // the combine parks one group's accumulators (D / 2 floats per lane), m,
  // m_true and l
  static_assert(KS == 1 || NWH * 64 * (D / 2 + 4) * 4 <= LDS_BYTES, "combine fits the stages");
};

constexpr float kLazyRescale = 8.f;  // log2 units
// paged grids order their work by sequence length up to this many sequences
constexpr int kRankedMaxB = 256;

// Row maxima use the NaN-propagating maximum (v_maximum3_f32 on gfx950):
// fmaxf would first quiet each input with an extra instruction.  The scores
// are never NaN (padding rows read as zero and masked keys are -inf).
__device__ __forceinline__ float vmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The r-th sequence by decreasing kv_len (ties by index): a bijection of
// 0 .. B-1, computed with one lane per sequence.  Wave-uniform result.
__device__ __forceinline__ int seq_by_rank(const int32_t* kv_len, int B, int r, int lane) {
  const __attribute__((address_space(4))) int32_t* kl =
      (const __attribute__((address_space(4))) int32_t*)kv_len;
  for (int base = 0; base < B; base += 64) {
    const int l = base + lane;
    const int wl = l < B ? kv_len[l] : 0;
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int wj = kl[j];  // uniform: a scalar load
      rank += (wj > wl) || (wj == wl && j < l);
    }
    const uint64_t hit = __ballot(l < B && rank == r);
    if (hit) return base + (int)__builtin_ctzll(hit);
  }
  return r;  // not reached: ranks are a permutation of 0 .. B-1
}

// NT: a single q-tile per (b, kv head, split), so no other workgroup reads
// this one's K/V tiles, which are then loaded with the non-temporal hint.
template <int D, int NW, bool PAGED, bool PARTIAL, int KS, bool NT>
__global__ void __launch_bounds__(NW * 64, (PrefillCfg<D, NW, KS>::MIN_WAVES_PER_SIMD))
attn_prefill_kernel(const AttnArgs a) {
  using C = PrefillCfg<D, NW, KS>;
  constexpr int CP = NT ? kCpNonTemporal : kCpDefault;
  constexpr int NTH = C::NTH;
  constexpr int BK = C::BK;
  constexpr int DC = C::DC;
  constexpr int CPT = C::CPT;
  constexpr int NCK = D / 16;  // 16-wide d steps of K Q^T
  constexpr int NDB = D / 32;  // 32-row d blocks of O^T
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int kh = KS == 1 ? 0 : wv / C::NWH;                  // key group
  const int wq = KS == 1 ? wv : wv % C::NWH;                 // 32-row block
  const int col = lane & 31;
  const int hl = lane >> 5;

  const int L = blockIdx.x;
  int b, g, split, qt;
  if (PAGED && a.B <= kRankedMaxB) {
    // Ragged sequences: the longest first, all of a sequence's work units
    // together (late q-tiles first), so the heaviest workgroups start in the
    // first wave of the grid and the light ones fill in behind them.
    const int per_seq = a.Hkv * a.n_split * a.n_qtiles;
    const int rem = L % per_seq;
    b = seq_by_rank(a.kv_len, a.B, L / per_seq, lane);
    g = rem % a.Hkv;
    split = (rem / a.Hkv) % a.n_split;
    qt = a.n_qtiles - 1 - rem / (a.Hkv * a.n_split);
  } else {
    const int nbg = a.B * a.Hkv;
    const int bg = L % nbg;
    const int rest = L / nbg;
    split = rest % a.n_split;
    qt = a.n_qtiles - 1 - rest / a.n_split;  // late (heavy causal) q-tiles first
    b = bg / a.Hkv;
    g = bg % a.Hkv;
  }
  const int G = a.G;

  int q_len, q_row0 = 0;
  if constexpr (PAGED) {
    q_row0 = a.cu_seqlens_q[b];
    q_len = a.cu_seqlens_q[b + 1] - q_row0;
  } else {
    q_len = a.Sq;
  }
  int n = a.Skv;
  if (a.kv_len) n = min(max(a.kv_len[b], 0), a.Skv);
  const int rows_total = q_len * G;
  const int row0 = qt * C::ROWS;
  if (row0 >= rows_total) return;

  int kbeg = 0, kend = n;
  if (a.tile > 0) {
    kbeg = split * a.tile;
    kend = min(n, kbeg + a.tile);
  }
  if (a.causal) {
    const int p_last = (min(row0 + C::ROWS, rows_total) - 1) / G;
    kend = min(kend, min(max(n - q_len + p_last + 1, 0), n));
  }
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  // this key group's tiles are kh, kh + KS, ...; every group runs nsteps
  // steps (one barrier each), idling through the ones it has no tile for
  const int ntl = ntiles > kh ? (ntiles - kh + KS - 1) / KS : 0;
  const int nsteps = (ntiles + KS - 1) / KS;

  // ---- this lane's query row and masking bounds
  const int wrow0 = row0 + 32 * wq;
  int wlo = kend;  // below wlo no row of the wave is masked
  if (a.causal) wlo = min(kend, min(max(n - q_len + wrow0 / G + 1, 0), n));
  if (wrow0 >= rows_total) wlo = kbeg;
  // tiles [0, nfull_all) need no mask for any row of this wave; nfull of
  // them are this group's
  const int nfull_all = min(ntiles, max(0, (wlo - kbeg) / BK));
  const int nfull = nfull_all > kh ? (nfull_all - kh + KS - 1) / KS : 0;
  const int rho = wrow0 + col;
  const bool rvalid = rho < rows_total;
  const int pq = rvalid ? rho / G : 0;
  const int hq = g * G + (rvalid ? rho - pq * G : 0);
  int lim = kend;
  if (a.causal) lim = min(kend, min(max(n - q_len + pq + 1, 0), n));
  bf16x8 qf[NCK];  // Q operand: row `col`, d = 16 c + 8 hl + e
  {
    const uint16_t* qp;
    if constexpr (PAGED)
      qp = a.q + (int64_t)(q_row0 + pq) * a.q_ss + (int64_t)hq * a.q_sh;
    else
      qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)pq * a.q_ss;
#pragma unroll
    for (int c = 0; c < NCK; ++c)
      qf[c] = rvalid ? *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hl) : bf16x8{};
  }
  float sl2 = -INFINITY;  // sink in log2 units (final mode)
  if constexpr (!PARTIAL)
    if (a.sink && rvalid) sl2 = a.sink[hq] * kLog2e;
  float mref = sl2;   // reference the running sums are taken against
  float mtrue = sl2;  // true running max (for the partial epilogue)
  float l = 0.f;      // this lane's share of the running sum
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  // ---- K/V staging.  A 64-key tile is one page of the paged layout; it is
  // loaded through one buffer resource per tensor that starts at the tile
  // and ends at its last row before kv_len, so rows past kv_len read as
  // zeros without touching memory (and are masked).  The threads of a key
  // group stage its tiles: chunk i of group thread t is row t / DC +
  // i NTH / DC at a per-thread constant offset.
  struct Stage {
    u32x4 k[CPT];
    u32x4 v[CPT];
  };
  const uint32_t kss2 = (uint32_t)(PAGED ? a.kv_sr : a.k_ss) * 2u;
  const uint32_t vss2 = (uint32_t)(PAGED ? a.kv_sr : a.v_ss) * 2u;
  const int gt = KS == 1 ? tid : tid % NTH;  // thread within the key group
  const int srow = gt / DC, sch = gt % DC;
  uint32_t koff[CPT], voff[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    koff[i] = (uint32_t)(srow + i * (NTH / DC)) * kss2 + 16u * sch;
    voff[i] = (uint32_t)(srow + i * (NTH / DC)) * vss2 + 16u * sch;
  }
  const uint16_t* khead = a.k + (PAGED ? (int64_t)g * a.k_sh
                                       : (int64_t)b * a.k_sb + (int64_t)g * a.k_sh);
  const uint16_t* vhead = a.v + (PAGED ? (int64_t)g * a.v_sh
                                       : (int64_t)b * a.v_sb + (int64_t)g * a.v_sh);
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)a.page_table;
  struct TileRes {
    BufRes k, v;
  };
  // `live` false: the prefetch past the last tile (it re-addresses that
  // tile); its resources are empty, so the loads return zeros without
  // touching memory, and the tile is never used.
  auto tile_res = [&](int j0, bool live) {
    int64_t off;
    if constexpr (PAGED)
      off = (int64_t)ptab[(int64_t)b * a.max_pages + (j0 >> 6)] * a.kv_sp;
    else
      off = (int64_t)j0 * a.k_ss;
    const uint32_t valid = (uint32_t)min(BK, n - j0);  // >= 1: tiles start below kend <= n
    return TileRes{make_bufres(khead + off, live ? (valid - 1u) * kss2 + (uint32_t)D * 2u : 0u),
                   make_bufres(vhead + (PAGED ? off : (int64_t)j0 * a.v_ss),
                               live ? (valid - 1u) * vss2 + (uint32_t)D * 2u : 0u)};
  };
  auto load_k = [&](const TileRes& r, Stage& st) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) st.k[i] = buf_load16v<CP>(r.k, koff[i]);
  };
  auto load_v = [&](const TileRes& r, Stage& st) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) st.v[i] = buf_load16v<CP>(r.v, voff[i]);
  };
  auto load_tile = [&](int j0, Stage& st, bool live) {
    const TileRes r = tile_res(j0, live);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      st.k[i] = buf_load16v<CP>(r.k, koff[i]);
      st.v[i] = buf_load16v<CP>(r.v, voff[i]);
    }
  };
  // the rows of a thread's chunks differ by multiples of 8: one swizzle
  const int kst = srow * C::KP + 8 * sch;
  const int vst = srow * D + 8 * (sch ^ vslot_swz<DC>(srow));
  uint16_t* const sg = smem + kh * 2 * C::STAGE;  // this group's two stages
  auto store_tile = [&](int stage, const Stage& st) {
    uint16_t* Ks = sg + stage * C::STAGE;
    uint16_t* Vs = Ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      *reinterpret_cast<u32x4*>(Ks + kst + i * (NTH / DC) * C::KP) = st.k[i];
      *reinterpret_cast<u32x4*>(Vs + vst + i * (NTH / DC) * D) = st.v[i];
    }
  };
  auto store_k = [&](int stage, const Stage& st) {
    uint16_t* Ks = sg + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *reinterpret_cast<u32x4*>(Ks + kst + i * (NTH / DC) * C::KP) = st.k[i];
  };
  auto store_v = [&](int stage, const Stage& st) {
    uint16_t* Vs = sg + stage * C::STAGE + C::KTILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      *reinterpret_cast<u32x4*>(Vs + vst + i * (NTH / DC) * D) = st.v[i];
  };
  // first key of this group's it-th tile
  auto tile_key = [&](int it) { return kbeg + (it * KS + kh) * BK; };

  Stage nx;
  if constexpr (!C::XP) {
    if (ntl > 0) {
      load_tile(tile_key(0), nx, true);
      store_tile(0, nx);
    }
    lds_barrier();
  }

  const int krow_a = swap_bits23(col);  // K row (within a 32-key half) this lane feeds to MFMA
  const int g16 = lane >> 4;
  const int r16 = lane & 15;
  // K operand of d step c, key half h
  auto kread = [&](const uint16_t* Ks, int c, int h) {
    return *reinterpret_cast<const bf16x8*>(Ks + (32 * h + krow_a) * C::KP + 16 * c + 8 * hl);
  };
  // V^T operand of d block db, keys 16 t .. 16 t + 15 (two transposing
  // reads).  The slot swizzle of key 16 t + 8 hl + 4 half + r16 / 4 depends
  // only on the lane and `half` (key bits 0-2), so a lane needs 2 x NDB base
  // offsets and the 16-key step t is an immediate.
  // The swizzle changes slot bits 1-3 only, so d blocks db and db + 4 (slot
  // + 16) differ by a constant: bases for the first four blocks suffice.
  constexpr int NVB = NDB < 4 ? NDB : 4;
  int vbase[2][NVB];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int db = 0; db < NVB; ++db) {
      const int cc = 32 * db + 16 * (g16 & 1) + 4 * (r16 & 3);
      const int key = 8 * hl + 4 * half + (r16 >> 2);
      vbase[half][db] = key * D + 8 * ((cc >> 3) ^ vslot_swz<DC>(key)) + (cc & 7);
    }
  auto vread = [&](const uint16_t* Vs, int t, int db) {
    i16x4 va[2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
      va[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(Vs + vbase[half][db % NVB] +
                                                     128 * (db / NVB) + 16 * t * D));
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(va[0], va[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T of key half h (register j = key j0 + 32 h + 16 (j >> 3) + 8 hl + (j & 7)),
  // with the K operands of the next d steps in flight
  auto qk = [&](const uint16_t* Ks, int h, auto interleave) {
    constexpr bool IL = decltype(interleave)::value;
    constexpr int PD = 2;
    bf16x8 kb[PD + 1];
#pragma unroll
    for (int c = 0; c < PD; ++c) kb[c] = kread(Ks, c, h);
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      if (c + PD < NCK) kb[(c + PD) % (PD + 1)] = kread(Ks, c + PD, h);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[c % (PD + 1)], qf[c], s, 0, 0, 0);
      if constexpr (IL) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x0002, 8, 0);  // VALU
      }
    }
    return s;
  };
  // S^T of both key halves with their MFMAs alternating, so each
  // accumulator's consecutive MFMAs are apart (a wave's MFMA that reads the
  // previous one's result waits for it); operands stream a few MFMAs ahead
  // The MFMA-only phases keep their operand reads PD MFMAs ahead in program
  // order (a scheduling barrier after each step): left free, the scheduler
  // sinks each read next to its MFMA to save registers, and every MFMA then
  // waits out a whole LDS latency.
  auto qk2 = [&](const uint16_t* Ks, f32x16& s0, f32x16& s1) {
    constexpr int PD = 3;
    bf16x8 kb[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) kb[i] = kread(Ks, i >> 1, i & 1);
    s0 = f32x16{};
    s1 = f32x16{};
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NCK; ++i) {
      if (i & 1)
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[i % (PD + 1)], qf[i >> 1], s1, 0, 0, 0);
      else
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[i % (PD + 1)], qf[i >> 1], s0, 0, 0, 0);
      if (i + PD < 2 * NCK) kb[(i + PD) % (PD + 1)] = kread(Ks, (i + PD) >> 1, (i + PD) & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T += V^T P^T for both key halves, the same way (reads PD MFMAs ahead)
  auto pv2 = [&](const uint16_t* Vs, const bf16x8 (&pb0)[2], const bf16x8 (&pb1)[2]) {
    constexpr int NS = 4 * NDB;  // MFMA steps (half, t, db)
    constexpr int PD = 3;
    bf16x8 vb[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) vb[i] = vread(Vs, i / NDB, i % NDB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const bf16x8& pb = (i / NDB) & 1 ? ((i / NDB) >> 1 ? pb1[1] : pb0[1])
                                        : ((i / NDB) >> 1 ? pb1[0] : pb0[0]);
      acc[i % NDB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % (PD + 1)], pb, acc[i % NDB], 0, 0, 0);
      if (i + PD < NS) vb[(i + PD) % (PD + 1)] = vread(Vs, (i + PD) / NDB, (i + PD) % NDB);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T += V^T P^T for keys 32 h .. 32 h + 31, next V operands in flight
  auto pv = [&](const uint16_t* Vs, int h, const bf16x8 (&pb)[2], auto interleave) {
    constexpr bool IL = decltype(interleave)::value;
    constexpr int NS = 2 * NDB;  // MFMA steps (t, db)
    constexpr int PD = 2;
    bf16x8 vb[PD + 1];
#pragma unroll
    for (int i = 0; i < PD; ++i) vb[i] = vread(Vs, 2 * h + i / NDB, i % NDB);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + PD < NS) vb[(i + PD) % (PD + 1)] = vread(Vs, 2 * h + (i + PD) / NDB, (i + PD) % NDB);
      acc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb[i % (PD + 1)], pb[i / NDB],
                                                             acc[i % NDB], 0, 0, 0);
      if constexpr (IL) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);  // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x0002, 8, 0);  // VALU
      }
    }
  };
  // Softmax of key half h, branch-free: mask (MASK tiles only), half max,
  // lazy reference move (returns the O rescale factor, 1 when the reference
  // stays), P rounded to bf16 and the row sum over the same rounded values.
  auto softmax = [&](auto mask_tag, int j0, int h, f32x16& s, bf16x8 (&pb)[2]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
      const int rem = lim - j0 - 32 * h - 8 * hl;  // first masked offset of this lane
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (16 * (j >> 3) + (j & 7) >= rem) s[j] = -INFINITY;
    }
    float m = s[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) m = vmax(m, s[j]);
    const float mx = half_swap_max(m) * a.scale_log2;
    mtrue = fmaxf(mtrue, mx);
    const bool move = mx > mref + kLazyRescale;
    const float alpha = move ? ex2(mref - mx) : 1.f;  // 0 when mref = -inf
    mref = move ? mx : mref;
    const float mu = (mref == -INFINITY) ? 0.f : mref;
    // each pair of weights is rounded once (one v_cvt_pk_bf16_f32) and that
    // packed word feeds both the row sum and the P operand
    float ls = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 x = {ex2(__builtin_fmaf(s[8 * t + 2 * e], a.scale_log2, -mu)),
                         ex2(__builtin_fmaf(s[8 * t + 2 * e + 1], a.scale_log2, -mu))};
        const bf16x2 pp = __builtin_convertvector(x, bf16x2);
        ls = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls, false);
        w[e] = __builtin_bit_cast(uint32_t, pp);
      }
      pb[t] = __builtin_bit_cast(bf16x8, w);
    }
    l = l * alpha + ls;
    return alpha;
  };
  // Softmax of a whole 64-key tile (both halves against one reference):
  // one max, one lazy reference decision, P rounded to bf16 and the row sum
  // over the same rounded values.  Returns the O rescale factor.
  auto softmax2 = [&](auto mask_tag, int j0, f32x16& s0, f32x16& s1, bf16x8 (&p0)[2],
                      bf16x8 (&p1)[2]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    if constexpr (MASK) {
      // key offset o of the tile is masked iff o >= rem; the sign of
      // rem - 1 - o gives an all-ones word for those, merged bitwise (no
      // compare results to hold in scalar registers across the tile)
      const int rem1 = lim - j0 - 8 * hl - 1;
      constexpr uint32_t kNegInf = 0xff800000u;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t m0 = (uint32_t)((rem1 - (16 * (j >> 3) + (j & 7))) >> 31);
        const uint32_t m1 = (uint32_t)((rem1 - (32 + 16 * (j >> 3) + (j & 7))) >> 31);
        s0[j] = __uint_as_float((m0 & kNegInf) | (~m0 & __float_as_uint(s0[j])));
        s1[j] = __uint_as_float((m1 & kNegInf) | (~m1 & __float_as_uint(s1[j])));
      }
    }
    float m = vmax(s0[0], s1[0]);
#pragma unroll
    for (int j = 1; j < 16; ++j) m = vmax(vmax(m, s0[j]), s1[j]);
    const float mx = half_swap_max(m) * a.scale_log2;
    mtrue = fmaxf(mtrue, mx);
    const bool move = mx > mref + kLazyRescale;
    const float alpha = move ? ex2(mref - mx) : 1.f;  // 0 when mref = -inf
    mref = move ? mx : mref;
    const float mu = (mref == -INFINITY) ? 0.f : mref;
    float ls = 0.f;
    auto expo = [&](const f32x16& sv, bf16x8 (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x2 x = {ex2(__builtin_fmaf(sv[8 * t + 2 * e], a.scale_log2, -mu)),
                           ex2(__builtin_fmaf(sv[8 * t + 2 * e + 1], a.scale_log2, -mu))};
          const bf16x2 pp = __builtin_convertvector(x, bf16x2);
          ls = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls, false);
          w[e] = __builtin_bit_cast(uint32_t, pp);
        }
        pb[t] = __builtin_bit_cast(bf16x8, w);
      }
    };
    expo(s0, p0);
    expo(s1, p1);
    l = l * alpha + ls;
    return alpha;
  };
  // Keeps a half's P inside the phase that computes it: without this the
  // compiler sinks the exponentials past the rescale branch into the next
  // phase, and the overlap with the other half's MFMAs is lost.  (P is
  // finished vector-ALU output, not a load: nothing waits here.)
  auto pin = [](const bf16x8 (&pb)[2]) { asm volatile("" ::"v"(pb[0]), "v"(pb[1])); };
  auto rescale = [&](float alpha) {
    if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] *= alpha;
    }
  };

  // Whole-phase operand fetches (EARLY): each phase's LDS operands are
  // requested before the previous phase's MFMAs, so none of its MFMAs waits
  // on LDS latency.  Needs 2 x D / 4 more VGPRs: the 8-wave form at d <= 128
  // has them, with two key groups (twice the staging registers) only at
  // d = 64, and the 2- and 4-wave forms at d <= 64.  At d = 128 those forms
  // spill with it.
  constexpr bool EARLY =
      (NW == 8 && D <= 128 && (KS == 1 || D <= 64)) || (NW <= 4 && D <= 64);
  auto kfetch = [&](const uint16_t* Ks, int h, bf16x8 (&k)[NCK]) {
#pragma unroll
    for (int c = 0; c < NCK; ++c) k[c] = kread(Ks, c, h);
  };
  auto vfetch = [&](const uint16_t* Vs, int h, bf16x8 (&v)[2 * NDB]) {
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) v[i] = vread(Vs, 2 * h + i / NDB, i % NDB);
  };
  auto qk_reg = [&](const bf16x8 (&k)[NCK], auto interleave) {
    constexpr bool IL = decltype(interleave)::value;
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NCK; ++c) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[c], qf[c], s, 0, 0, 0);
      if constexpr (IL) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);  // LDS reads (next phase)
        __builtin_amdgcn_sched_group_barrier(0x0002, 8, 0);  // VALU
      }
    }
    return s;
  };
  // interleave: 1 = vector work and next-phase LDS reads between the MFMAs,
  // 2 = the next tile's LDS writes between the MFMAs
  auto pv_reg = [&](const bf16x8 (&v)[2 * NDB], const bf16x8 (&pb)[2], auto interleave) {
    constexpr int IL = decltype(interleave)::value;
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
      acc[i % NDB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[i], pb[i / NDB], acc[i % NDB], 0, 0, 0);
      if constexpr (IL == 1) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);  // LDS reads (next phase)
        __builtin_amdgcn_sched_group_barrier(0x0002, 8, 0);  // VALU
      } else if constexpr (IL == 2) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0200, 1, 0);  // LDS write
      }
    }
  };

  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;
  // `par` is the tile's LDS stage (it & 1) as a constant, so every LDS
  // address of the step is a base register plus an immediate
  auto step_early = [&](auto mask_tag, int it, auto par) {
    constexpr int PAR = decltype(par)::value;
    const int j0 = tile_key(it);
    load_tile(tile_key(min(it + 1, ntl - 1)), nx, it + 1 < ntl);
    const uint16_t* Ks = sg + PAR * C::STAGE;
    const uint16_t* Vs = Ks + C::KTILE;
    bf16x8 k0[NCK], k1[NCK], v0[2 * NDB], v1[2 * NDB], p0[2], p1[2];
    kfetch(Ks, 0, k0);
    kfetch(Ks, 1, k1);
    __builtin_amdgcn_sched_barrier(0);
    // 1. S_0
    f32x16 s0 = qk_reg(k0, False{});
    __builtin_amdgcn_sched_barrier(0);
    // 2. S_1 || softmax of S_0; V_0 operands requested
    vfetch(Vs, 0, v0);
    f32x16 s1 = qk_reg(k1, True{});
    const float alpha0 = softmax(mask_tag, j0, 0, s0, p0);
    pin(p0);
    __builtin_amdgcn_sched_barrier(0);
    rescale(alpha0);
    // 3. O += V_0 P_0 || softmax of S_1; V_1 operands requested
    vfetch(Vs, 1, v1);
    pv_reg(v0, p0, std::integral_constant<int, 1>{});
    const float alpha1 = softmax(mask_tag, j0, 1, s1, p1);
    pin(p1);
    __builtin_amdgcn_sched_barrier(0);
    rescale(alpha1);
    // 4. stage the next tile into the idle buffer (no wave reads it before
    // the barrier below), then O += V_1 P_1: the LDS writes overlap the MFMAs
    store_tile(1 - PAR, nx);
    pv_reg(v1, p1, std::integral_constant<int, 2>{});
    lds_barrier();
  };
  auto step = [&](auto mask_tag, int it) {
    const int j0 = tile_key(it);
    // Unconditional prefetch of the next tile (past the end an empty one):
    // no branch separates the loads from the compute.
    // Its K is loaded now and stored into the idle stage after the K^T Q
    // phases; its V is loaded then and stored at the end, so only one
    // tensor's chunks are held in registers at a time.
    const TileRes nr = tile_res(tile_key(min(it + 1, ntl - 1)), it + 1 < ntl);
    load_k(nr, nx);
    const uint16_t* Ks = sg + (it & 1) * C::STAGE;
    const uint16_t* Vs = Ks + C::KTILE;
    bf16x8 p0[2], p1[2];
    // 1. S_0
    f32x16 s0 = qk(Ks, 0, False{});
    __builtin_amdgcn_sched_barrier(0);
    // 2. S_1 || softmax of S_0
    f32x16 s1 = qk(Ks, 1, True{});
    const float alpha0 = softmax(mask_tag, j0, 0, s0, p0);
    pin(p0);
    __builtin_amdgcn_sched_barrier(0);
    rescale(alpha0);
    store_k((it + 1) & 1, nx);
    load_v(nr, nx);
    __builtin_amdgcn_sched_barrier(0);
    // 3. O += V_0 P_0 || softmax of S_1
    pv(Vs, 0, p0, True{});
    const float alpha1 = softmax(mask_tag, j0, 1, s1, p1);
    pin(p1);
    __builtin_amdgcn_sched_barrier(0);
    rescale(alpha1);
    // 4. O += V_1 P_1, stage the next tile's V
    pv(Vs, 1, p1, False{});
    store_v((it + 1) & 1, nx);
    lds_barrier();
  };

  // ---- Ping-pong of the two waves of each SIMD (8 waves, one key group,
  // d <= 128).  A wave issues in order, and an MFMA holds its wave until the
  // matrix pipe takes it.  Measured on gfx950 (loops, one workgroup per CU):
  // with one wave per SIMD, about two vector instructions after each MFMA
  // run in its shadow and each further one adds ~4.5 cycles (an exponential
  // ~8); vector work of ANOTHER wave on the SIMD costs the MFMA wave nothing,
  // but while that wave keeps MFMAs queued the other issues only about one
  // vector instruction per MFMA.  So each wave alternates two pure phases,
  // and the barrier that ends a phase lets the lagging vector phase finish:
  //   M(t): S = K_t Q^T (both halves), then O += V_{t-1}^T P_{t-1}^T  (MFMA
  //         and LDS operand reads only)
  //   V(t): softmax of S_t -> P_t and the O rescale, then this thread's
  //         share of the next tiles' staging (LDS writes, global loads)
  // and waves 4-7 run one phase behind waves 0-3; wave w and wave w + 4 share
  // a SIMD, so one is always in M while the other is in V.  A barrier ends
  // every phase ("slot"); both halves pass 2 ntl + 1 of them (the lagging
  // half starts with a slot of staging only, the leading half ends with a
  // barrier after its last M).
  //
  // Tile t's K is read in slots 2t (leading half) and 2t + 1 (lagging), its
  // V in slots 2t + 2 and 2t + 3.  The V phase of tile u stores K(u+1) and
  // V(u) (leading, slot 2u + 1) or K(u+2) and V(u+1) (lagging, slot 2u + 2)
  // into the stages of those tiles, each after the previous occupant's last
  // reader and before the first reader; it then requests the shares its next
  // V phase stores, two slots ahead.  Past the last tile the loads go through
  // empty resources (zeros) and land in stage areas no wave reads again.
  constexpr bool PP = EARLY && NW == 8 && KS == 1;
  if constexpr (PP) {
    const int lagh = (wv >> 2) & 1;  // wave-uniform: 1 = the lagging half
    u32x4 rk[CPT], rv[CPT];          // staged shares: one K tile, one V tile
    auto share_res = [&](int T, bool isk) __attribute__((always_inline)) {
      const int j0 = tile_key(max(0, min(T, ntl - 1)));  // in the page table even past the end
      int64_t off;
      if constexpr (PAGED)
        off = (int64_t)ptab[(int64_t)b * a.max_pages + (j0 >> 6)] * a.kv_sp;
      else
        off = (int64_t)j0 * (isk ? a.k_ss : a.v_ss);
      const uint32_t rs2 = isk ? kss2 : vss2;
      const uint32_t valid = (uint32_t)min(BK, n - j0);
      return make_bufres((isk ? khead : vhead) + off,
                         T < ntl ? (valid - 1u) * rs2 + (uint32_t)D * 2u : 0u);
    };
    auto stage_load = [&](int tk, int tv) __attribute__((always_inline)) {
      const BufRes kr = share_res(tk, true);
      const BufRes vr = share_res(tv, false);
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        rk[i] = buf_load16v<CP>(kr, koff[i]);
        rv[i] = buf_load16v<CP>(vr, voff[i]);
      }
    };
    auto stage_store = [&](int tk, int tv) __attribute__((always_inline)) {
      uint16_t* Kd = sg + (tk & 1) * C::STAGE + kst;
      uint16_t* Vd = sg + (tv & 1) * C::STAGE + C::KTILE + vst;
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        *reinterpret_cast<u32x4*>(Kd + i * (NTH / DC) * C::KP) = rk[i];
        *reinterpret_cast<u32x4*>(Vd + i * (NTH / DC) * D) = rv[i];
      }
    };
    f32x16 ps0, ps1;     // S of the tile between its M and V phases
    bf16x8 pp0[2], pp1[2];  // P of the tile between its V phase and the next M
    auto m_qk = [&](auto par) __attribute__((always_inline)) {
      qk2(sg + decltype(par)::value * C::STAGE, ps0, ps1);
    };
    auto m_pv = [&](auto par) __attribute__((always_inline)) {
      pv2(sg + decltype(par)::value * C::STAGE + C::KTILE, pp0, pp1);
    };
    auto v_phase = [&](auto mask_tag, int u) __attribute__((always_inline)) {
      rescale(softmax2(mask_tag, tile_key(u), ps0, ps1, pp0, pp1));
      stage_store(u + 1 + lagh, u + lagh);
      stage_load(u + 2 + lagh, u + 1 + lagh);
    };
    // tile u's V phase, then M(u + 1): the next tile's QK^T and tile u's
    // P.V.  After the last tile the QK^T runs on whatever the idle stage
    // holds and its S is never used (one branch-free step: two copies of the
    // phase cost more registers than the 16 MFMAs once per workgroup).
    auto pp_step = [&](auto mask_tag, int u, auto par) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par)::value;
      v_phase(mask_tag, u);
      lds_barrier();
      m_qk(std::integral_constant<int, 1 - PAR>{});
      m_pv(std::integral_constant<int, PAR>{});
      if (!(lagh && u == ntl - 1)) lds_barrier();  // the lagging half has one fewer here
    };
    if (ntl > 0) {
      stage_load(1, 0);
      if (lagh) {  // slot 0: the lagging half's staging only
        stage_store(1, 0);
        stage_load(2, 1);
        lds_barrier();
      }
      m_qk(std::integral_constant<int, 0>{});  // M(0): no P.V yet
      lds_barrier();
      using P0 = std::integral_constant<int, 0>;
      using P1 = std::integral_constant<int, 1>;
      int u = 0;
      for (; u + 1 < nfull; u += 2) {
        pp_step(False{}, u, P0{});
        pp_step(False{}, u + 1, P1{});
      }
      if (u < nfull) {  // odd number of unmasked tiles
        pp_step(False{}, u, P0{});
        ++u;
        if (u < ntl) {
          pp_step(True{}, u, P1{});
          ++u;
        }
      }
      for (; u + 1 < ntl; u += 2) {
        pp_step(True{}, u, P0{});
        pp_step(True{}, u + 1, P1{});
      }
      if (u < ntl) pp_step(True{}, u, P0{});
    }
  }

  // ---- Cross-tile pipelining inside each wave (4 waves, one key group,
  // d = 256).  One wave per SIMD, so its MFMAs can only overlap vector work
  // of the same wave: an MFMA holds the wave until the busy matrix pipe takes
  // it, but about two independent vector instructions after each MFMA run in
  // its shadow, and each further one adds ~4.5 cycles (~8 for an exponential;
  // measured on gfx950 with this MFMA stream in a loop).  A 64-key tile at
  // d = 256 carries 64 MFMAs per wave against ~130 softmax instructions, so
  // each wave runs the softmax of tile t between its own MFMAs of
  // independent work, one MFMA step at a time in a fixed order, and one
  // barrier per tile orders the stages:
  //   steps 0 .. NA-1:   O += V_{t-1}^T P_{t-1}^T, with the mask, row max and
  //                      lazy reference move of tile t, then its weights
  //   steps NA .. NST-1: S_{t+1} = K_{t+1} Q^T, with the rest of the weights
  //   then the (rare) O rescale by tile t's factor -- after the P.V of tile
  //   t - 1, before that of tile t -- and the barrier.
  // Both reads of an iteration come from stage (t + 1) & 1 (K of tile t + 1,
  // V of tile t - 1).  At its start the four waves request K of tile t + 2
  // and V of tile t into stage t & 1, whose last readers ran before the
  // previous barrier, by LDS DMA: 64 lanes x 16 bytes straight into one
  // 1 KiB block of the stage per instruction, with no staging registers (64
  // per lane at d = 256) and no LDS writes in the waves.  The barrier at the
  // iteration's end waits for them.  The stages are separate static arrays,
  // so the compiler can tell the DMA targets from the stage the MFMA
  // operands are read from and does not wait for the DMA there.  The first
  // P.V has P = 0 over stage 1's V, zero-filled at the start; the last QK^T
  // runs on an empty K tile and its S is unused.  Measured on causal
  // prefill (B 2, Hq 32, Hkv 8, 8192 keys): 2.61 ms with the four-phase step
  // and register staging, 2.11 ms with this one.
  constexpr bool XP = C::XP;
  if constexpr (XP) {
    __shared__ __attribute__((aligned(16))) uint16_t xk0[C::KTILE], xk1[C::KTILE];
    __shared__ __attribute__((aligned(16))) uint16_t xv0[C::TILE], xv1[C::TILE];
    using LdsPtr = __attribute__((address_space(3))) void*;
    static_assert(D == 256 && NW == 4, "the layouts below are for d = 256, 4 waves");
    // K: row pairs.  One 1 KiB DMA block is a pair of 512-byte rows; pairs sit
    // PAIR elements apart (32 bytes of pad), and the odd row of a pair holds
    // the two 16-byte halves of each 32-byte chunk swapped.  The K operand
    // reads (16 bytes per lane, 16 lanes over 16 rows) then hit 16 distinct
    // 16-byte bank slots: a pair's rows differ in the half, pairs by the pad.
    // V: rows of D elements, slot p of row r holding chunk p ^ vslot_swz(r).
    // Wave w issues blocks i = w, w + 4, ...: a lane's row within the block
    // and its chunk are the same in all of them (the V swizzle repeats every
    // 8 rows), so one per-lane offset per tensor plus the block's row step.
    // Rows past kv_len lie outside the tile's buffer and read as zeros.
    constexpr int PAIR = 2 * D + 16;  // elements per row pair with its pad
    static_assert(C::KTILE == 32 * PAIR, "K tile of 32 row pairs");
    const int hi = lane >> 5;  // the block's odd row
    const uint32_t dko = (uint32_t)hi * kss2 + 16u * (uint32_t)((lane & 31) ^ hi);
    const uint32_t dvo =
        (uint32_t)hi * vss2 + 16u * (uint32_t)((lane & 31) ^ vslot_swz<DC>(2 * wv + hi));
    auto dma_k = [&](const TileRes& r, uint16_t* dst) __attribute__((always_inline)) {
      BufRes rr = r.k;  // a const resource argument makes the host pass drop the kernel
      for (int i = wv; i < 32; i += 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (LdsPtr)(dst + PAIR * i), 16,
                                                 (int)(dko + 2u * (uint32_t)i * kss2), 0, 0, CP);
    };
    auto dma_v = [&](const TileRes& r, uint16_t* dst) __attribute__((always_inline)) {
      BufRes rr = r.v;
      for (int i = wv; i < 32; i += 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (LdsPtr)(dst + 512 * i), 16,
                                                 (int)(dvo + 2u * (uint32_t)i * vss2), 0, 0, CP);
    };
    // K operand of d step c, key half h, in the pair layout: a per-lane base
    // and immediates
    const int kxo = (krow_a >> 1) * PAIR + (krow_a & 1) * D + 8 * (hl ^ (krow_a & 1));
    auto kreadx = [&](const uint16_t* Ks, int c, int h) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(Ks + kxo + 16 * PAIR * h + 16 * c);
    };
    // S of the tile whose softmax runs next, P of the tile whose P.V runs
    // next: two register sets each, which swap roles with the tile's parity
    f32x16 sA0, sA1, sB0, sB1;
    bf16x8 pA0[2], pA1[2], pB0[2], pB1[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) pB0[t] = pB1[t] = bf16x8{};
    // first key of a real tile to address an empty (zero-size) load with
    auto any_key = [&](int t) __attribute__((always_inline)) {
      return tile_key(max(0, min(t, ntl - 1)));
    };
    auto xp_step = [&](auto mask_tag, int t, auto par, const f32x16& sc0, const f32x16& sc1,
                       f32x16& sn0, f32x16& sn1, const bf16x8 (&pv0)[2], const bf16x8 (&pv1)[2],
                       bf16x8 (&pc0)[2], bf16x8 (&pc1)[2]) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par)::value;
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr int PD = 3;          // operand reads run this many MFMAs ahead
      constexpr int NA = 4 * NDB;    // P.V MFMAs
      constexpr int NB = 2 * NCK;    // K Q^T MFMAs
      constexpr int NST = NA + NB;   // all MFMA steps of the iteration
      const uint16_t* Kn = PAR ? xk0 : xk1;  // K of tile t + 1
      const uint16_t* Vp = PAR ? xv0 : xv1;  // V of tile t - 1
      dma_k(tile_res(any_key(t + 2), t + 2 < ntl), PAR ? xk1 : xk0);
      dma_v(tile_res(tile_key(t), true), PAR ? xv1 : xv0);
      // operand of MFMA step g: V^T of P.V step g, then K of K Q^T step g - NA
      auto opread = [&](int g) __attribute__((always_inline)) {
        return g < NA ? vread(Vp, g / NDB, g % NDB) : kreadx(Kn, (g - NA) >> 1, (g - NA) & 1);
      };
      f32x16 c0 = sc0, c1 = sc1;
      const int rem1 = lim - tile_key(t) - 8 * hl - 1;  // masked key offsets: o > rem1
      float m = -INFINITY, mx = 0.f, alpha = 1.f, mu = 0.f, ls = 0.f;
      u32x4 w[2][2];  // packed weights: key half, 16-key group
      sn0 = f32x16{};
      sn1 = f32x16{};
      bf16x8 ob[PD + 1];
#pragma unroll
      for (int g = 0; g < PD; ++g) ob[g] = opread(g);
      __builtin_amdgcn_sched_barrier(0);
      // One MFMA per step, the read PD steps ahead, and a fixed share of the
      // softmax of tile t: steps 0-3 mask (tiles that need it) and take the
      // row max over 4 of the 16 register pairs each, step 4 the reference
      // move, then the 16 weight pairs spread over the remaining steps.
      // (expanded at compile time: a 64-step loop at d = 256 is too large
      // for the unroller, and a rolled loop indexes the register arrays)
      auto mstep = [&](auto gc) __attribute__((always_inline)) {
        constexpr int g = decltype(gc)::value;
        if constexpr (g < NA) {
          constexpr int i = g;
          const bf16x8& pb = (i / NDB) & 1 ? ((i / NDB) >> 1 ? pv1[1] : pv0[1])
                                            : ((i / NDB) >> 1 ? pv1[0] : pv0[0]);
          acc[i % NDB] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[g % (PD + 1)], pb, acc[i % NDB], 0, 0, 0);
        } else {
          constexpr int i = g - NA;
          if constexpr (i & 1)
            sn1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[g % (PD + 1)], qf[i >> 1], sn1, 0, 0, 0);
          else
            sn0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ob[g % (PD + 1)], qf[i >> 1], sn0, 0, 0, 0);
        }
        if constexpr (g + PD < NST) ob[(g + PD) % (PD + 1)] = opread(g + PD);
        if constexpr (g < 4) {
#pragma unroll
          for (int j = 4 * g; j < 4 * g + 4; ++j) {
            if constexpr (MASK) {
              // the sign of rem1 - o is an all-ones word for a masked
              // offset o, merged bitwise (no compare masks to hold)
              constexpr uint32_t kNegInf = 0xff800000u;
              const uint32_t m0 = (uint32_t)((rem1 - (16 * (j >> 3) + (j & 7))) >> 31);
              const uint32_t m1 = (uint32_t)((rem1 - (32 + 16 * (j >> 3) + (j & 7))) >> 31);
              c0[j] = __uint_as_float((m0 & kNegInf) | (~m0 & __float_as_uint(c0[j])));
              c1[j] = __uint_as_float((m1 & kNegInf) | (~m1 & __float_as_uint(c1[j])));
            }
            m = vmax(vmax(m, c0[j]), c1[j]);
          }
          if constexpr (g == 3) mx = half_swap_max(m) * a.scale_log2;
        } else if constexpr (g == 4) {
          mtrue = fmaxf(mtrue, mx);
          const bool move = mx > mref + kLazyRescale;
          alpha = move ? ex2(mref - mx) : 1.f;  // 0 when mref = -inf
          mref = move ? mx : mref;
          mu = (mref == -INFINITY) ? 0.f : mref;
        } else {
          // weight pair k (two adjacent keys of one row) at step 5 + k (NST - 5) / 16:
          // rounded once to bf16x2, which feeds both the row sum and P
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            if (5 + k * (NST - 5) / 16 != g) continue;
            const int hf = k >> 3, grp = (k >> 2) & 1, e = k & 3;
            const f32x16& sv = hf ? c1 : c0;
            const f32x2 x = {ex2(__builtin_fmaf(sv[8 * grp + 2 * e], a.scale_log2, -mu)),
                             ex2(__builtin_fmaf(sv[8 * grp + 2 * e + 1], a.scale_log2, -mu))};
            const bf16x2 pp = __builtin_convertvector(x, bf16x2);
            ls = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls, false);
            w[hf][grp][e] = __builtin_bit_cast(uint32_t, pp);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      };
      static_for<NST>(mstep);
#pragma unroll
      for (int grp = 0; grp < 2; ++grp) {
        pc0[grp] = __builtin_bit_cast(bf16x8, w[0][grp]);
        pc1[grp] = __builtin_bit_cast(bf16x8, w[1][grp]);
      }
      l = l * alpha + ls;
      // keeps the softmax in the MFMA steps above: left free, the compiler
      // sinks the exponentials past the rescale branch, out of the shadows
      pin(pc0);
      pin(pc1);
      asm volatile("" ::"v"(l));
      rescale(alpha);
      lds_barrier();  // also waits for this wave's DMA
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // tile t of parity 0 takes S from set A and P of tile t - 1 from set B
    auto xp0 = [&](auto mask_tag, int t) __attribute__((always_inline)) {
      xp_step(mask_tag, t, P0{}, sA0, sA1, sB0, sB1, pB0, pB1, pA0, pA1);
    };
    auto xp1 = [&](auto mask_tag, int t) __attribute__((always_inline)) {
      xp_step(mask_tag, t, P1{}, sB0, sB1, sA0, sA1, pA0, pA1, pB0, pB1);
    };
    if (ntl > 0) {
      // stage 0: tile 0; stage 1: K of tile 1, V zeros (0 x inf would be NaN)
      {
        const TileRes r0 = tile_res(tile_key(0), true);
        dma_k(r0, xk0);
        dma_v(r0, xv0);
        dma_k(tile_res(any_key(1), ntl > 1), xk1);
      }
#pragma unroll
      for (int i = 0; i < C::TILE / (8 * C::NT); ++i)
        *reinterpret_cast<u32x4*>(xv1 + 8 * (tid + i * C::NT)) = u32x4{};
      lds_barrier();
      // S of tile 0
      sA0 = f32x16{};
      sA1 = f32x16{};
#pragma unroll
      for (int c = 0; c < NCK; ++c) {
        sA0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreadx(xk0, c, 0), qf[c], sA0, 0, 0, 0);
        sA1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreadx(xk0, c, 1), qf[c], sA1, 0, 0, 0);
      }
      lds_barrier();       // read by every wave before iteration 0 refills stage 0
      int u = 0;
      for (; u + 1 < nfull; u += 2) {
        xp0(False{}, u);
        xp1(False{}, u + 1);
      }
      if (u < nfull) {  // odd number of unmasked tiles
        xp0(False{}, u);
        ++u;
        if (u < ntl) {
          xp1(True{}, u);
          ++u;
        }
      }
      for (; u + 1 < ntl; u += 2) {
        xp0(True{}, u);
        xp1(True{}, u + 1);
      }
      if (u < ntl) xp0(True{}, u);
      // O += V^T P^T of the last tile
      if ((ntl - 1) & 1)
        pv2(xv1, pB0, pB1);
      else
        pv2(xv0, pA0, pA1);
    }
  }

  int it = 0;
  if constexpr (PP || XP) {
    // done above
  } else if constexpr (EARLY) {
    // Tiles two at a time (stages 0 and 1), unmasked tiles first, then the
    // masked ones; a leftover single tile runs on its own stage.  (The
    // forms without the early fetch keep a runtime stage: unrolled, they
    // would spill.)
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    for (; it + 1 < nfull; it += 2) {
      step_early(False{}, it, P0{});
      step_early(False{}, it + 1, P1{});
    }
    if (it < nfull) {  // odd number of unmasked tiles
      step_early(False{}, it, P0{});
      ++it;
      if (it < ntl) {
        step_early(True{}, it, P1{});
        ++it;
      }
    }
    for (; it + 1 < ntl; it += 2) {
      step_early(True{}, it, P0{});
      step_early(True{}, it + 1, P1{});
    }
    if (it < ntl) step_early(True{}, it, P0{});
  } else {
    for (; it < nfull; ++it) step(False{}, it);
    for (; it < ntl; ++it) step(True{}, it);
  }
  if constexpr (KS > 1) {
    for (int i = ntl; i < nsteps; ++i) lds_barrier();  // steps this group has no tile for
    // Combine the key groups (the same associative (m, l, O) merge as
    // between splits): group 1 parks its O, reference, true max and sum
    // share in the stages, which no wave reads after the last barrier;
    // group 0 takes both to the larger reference.  Lane-major float4
    // slots: the same lane of the same row block reads what it needs.
    constexpr int XF = 64 * NDB * 16;  // accumulator floats of a row block
    float* xo = reinterpret_cast<float*>(smem) + wq * XF;
    float4* xm = reinterpret_cast<float4*>(reinterpret_cast<float*>(smem) + C::NWH * XF) + wq * 64;
    if (kh == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(xo + ((db * 4 + q4) * 64 + lane) * 4) =
              make_float4(acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                          acc[db][4 * q4 + 3]);
      xm[lane] = make_float4(mref, mtrue, l, 0.f);
    }
    lds_barrier();
    if (kh == 1) return;
    const float4 st1 = xm[lane];
    const float mc = fmaxf(mref, st1.x);
    const float f0 = mref == -INFINITY ? 0.f : ex2(mref - mc);
    const float f1 = st1.x == -INFINITY ? 0.f : ex2(st1.x - mc);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 o1 = *reinterpret_cast<const float4*>(xo + ((db * 4 + q4) * 64 + lane) * 4);
        acc[db][4 * q4] = acc[db][4 * q4] * f0 + o1.x * f1;
        acc[db][4 * q4 + 1] = acc[db][4 * q4 + 1] * f0 + o1.y * f1;
        acc[db][4 * q4 + 2] = acc[db][4 * q4 + 2] * f0 + o1.z * f1;
        acc[db][4 * q4 + 3] = acc[db][4 * q4 + 3] * f0 + o1.w * f1;
      }
    l = l * f0 + st1.z * f1;
    mref = mc;
    mtrue = fmaxf(mtrue, st1.y);
  }

  // ---- epilogue; accumulator register j of d-block db holds
  //      d = 32 db + 8 (j >> 2) + 4 hl + (j & 3) of query row `col`
  float lt = half_swap_sum(l);
  if constexpr (PARTIAL) {
    // report the state against the true max (as the partial format states)
    const float f = (mtrue == -INFINITY) ? 0.f : ex2(mref - mtrue);
    lt *= f;
    if (!rvalid) return;
    int64_t row;
    if constexpr (PAGED)
      row = (int64_t)hq * a.total_q + q_row0 + pq;
    else
      row = ((int64_t)b * a.Hq + hq) * a.Sq + pq;
    const int64_t idx = row * a.n_split + split;
    if (hl == 0) a.ws_ml[idx] = make_float2(mtrue == -INFINITY ? -INFINITY : mtrue * kLn2, lt);
    if (a.skip_empty_o && mtrue == -INFINITY) return;  // no visible key in this split
    float* op = a.ws_o + idx * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(op + 32 * db + 8 * q4 + 4 * hl) =
            make_float4(acc[db][4 * q4] * f, acc[db][4 * q4 + 1] * f, acc[db][4 * q4 + 2] * f,
                        acc[db][4 * q4 + 3] * f);
  } else {
    if (sl2 != -INFINITY) lt += ex2(sl2 - mref);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (!rvalid) return;
    uint16_t* op;
    if constexpr (PAGED)
      op = a.o + (int64_t)(q_row0 + pq) * a.o_ss + (int64_t)hq * a.o_sh;
    else
      op = a.o + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + (int64_t)pq * a.o_ss;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * q4 + 4 * hl) =
            make_uint2(pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                       pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv));
  }
}

}  // namespace gqa
