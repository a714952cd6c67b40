// Stream GQA forward kernel for query groups of at most 16 * NQB rows per
// (b, kv head): single-token decode and short query blocks.
//
// Each workgroup owns one (b, kv head g, q-tile) and a run of `spw`
// consecutive kv splits.  Its NW waves cut the run's keys into 32-key tiles
// taken round-robin, and each wave streams its tiles on its own.  A wave
// keeps the next tile's K and V (two tiles in the d = 128 decode form) in
// flight in registers while it computes on the current one; where one
// q-tile covers the group, no other workgroup reads those tiles and the
// loads carry the non-temporal hint (NT).  When a wave's next tile belongs to a later split, the
// waves' running states (m, l, O) are combined through LDS (the associative
// (m, l, O) merge of the kernbench2 2-D mesh all-reduce-mlo commit) and
// written as that split's partial (or as the final normalised output when
// there is no split); the prefetched tile stays in flight meanwhile.  Longer
// runs per workgroup stream HBM faster than one split each (fewer, longer
// sequential streams), while the partials keep the split size.
//
// Two options ride on the same kernel: the paged append (the query tokens'
// own K/V come from k_new / v_new and are written into their pages; block
// after the key loop) and the in-kernel split merge (tickets; block after
// the partial write-out).
//
// MFMA mapping, v_mfma_f32_16x16x32_bf16 (16 query columns per block, so a
// 4-row GQA group wastes 12 columns instead of 28 with the 32-wide form):
//   S^T[key][q] = K Q^T : A = K straight from global memory (lane = key row
//                         c16, 8 d per lane group), B = Q in registers (in
//                         LDS at d = 256).
//   O^T[d][q] += V^T P^T: B = P from the S^T accumulators of the lane (two
//                         16-key blocks -> 8 keys), A = V^T read from a
//                         wave-private row-major LDS tile with
//                         ds_read_b64_tr_b16 (within each 16-lane group,
//                         destination lane i, element e comes from source
//                         lane 4e + i/4, element i%4 -- so each source lane
//                         points at 4 d of one key row and every lane gets 4
//                         keys of one d).
//   16-byte V slots in LDS are XOR-swizzled per row (vslot_swz), which makes
//   both the b128 row writes and the transposing reads bank-conflict free.
//   KROW (paged pools stored token-major, d = 128): K is loaded like V, as
//   whole rows (four 256-byte rows per instruction rather than 64-byte
//   pieces of 16 rows spread over the 2 KB row stride), written to a
//   wave-private LDS tile with rows padded by 32 bytes and read back in the
//   A layout above; it reaches the MFMAs bit for bit as the direct form's.
#pragma once

#include "common.hpp"

namespace gqa {

template <int D, int NQB, bool KROW = false>
struct StreamCfg {
  static constexpr int BK = 32;             // keys per tile
  static constexpr int NC = D / 32;         // 32-wide d steps of Q.K
  static constexpr int NDB = D / 16;        // 16-row d blocks of O^T
  static constexpr int DC = D / 8;          // 16-byte chunks per row
  static constexpr int VPL = BK * DC / 64;  // V chunks per lane per tile
  static constexpr int VTILE = BK * D;      // V tile elements (per wave)
  // K as whole rows (KROW): a wave-private K tile, rows padded by 32 bytes
  // so that the operand reads (16 rows, one 16-byte slot each) and the row
  // writes are bank-conflict free (a 16-byte pad left conflicts on 2% of
  // the cycles, by the LDS bank-conflict counter)
  static constexpr int KP = D + 16;
  static constexpr int KTILE = KROW ? BK * KP : 0;
  static constexpr int SLOT_F = NQB * (2 + 4 * NDB) * 64;  // combine floats per wave
  static constexpr int PSTR = D + 4;       // parked column: O (D floats), m, l, pad
  static constexpr int PEND_F = NQB * 16 * PSTR;  // parked floats per split
  // d = 256 keeps Q in LDS (row pitch D + 8: conflict-free operand reads)
  static constexpr bool Q_LDS = D > 128;
  static constexpr int QP = D + 8;
  static constexpr int QTILE = Q_LDS ? NQB * 16 * QP : 0;
  // LDS: one V tile per wave (and one K tile with KROW), one combine slot
  // per wave other than 0, (partial mode) one parked state per split of the
  // run, and Q at d = 256
  static constexpr int lds_bytes(int nw, int spw) {
    return nw * (VTILE + KTILE) * 2 + (nw - 1) * SLOT_F * 4 + spw * PEND_F * 4 + QTILE * 2;
  }
  static constexpr int LDS_LIMIT = 160 * 1024;
  // splits per workgroup: up to 8 (one 16-column block) or 4, as LDS allows
  static constexpr int max_spw(int nw) {
    int s = NQB == 1 ? 8 : 4;
    while (s > 1 && lds_bytes(nw, s) > LDS_LIMIT) s /= 2;
    return s;
  }
  // the wider (4-wave) form needs its combine slots and one parked split
  static constexpr bool FOUR_WAVES = lds_bytes(4, 1) <= LDS_LIMIT;
  static_assert(lds_bytes(2, max_spw(2)) <= LDS_LIMIT, "two-wave form fits in LDS");
};

// One wave per SIMD: the register budget then holds two in-flight tiles,
// Q, O and the softmax state without spilling (a spill reload waits behind
// the tile loads in flight), and this HBM-bound kernel streams fastest with
// few, long-running waves per CU anyway.
// NT: no other workgroup reads this one's K/V tiles (one q-tile), which
// are then loaded with the non-temporal hint.
template <int D, int NQB, int NW, bool PAGED, bool PARTIAL, bool NT, bool KROW = false>
__global__ void __launch_bounds__(NW * 64, 1)
attn_stream_kernel(const AttnArgs a) {
  using C = StreamCfg<D, NQB, KROW>;
  constexpr int CP = NT ? kCpNonTemporal : kCpDefault;
  // tiles in flight per wave while it computes on one.  Two at d = 128 with
  // one 16-column block (the decode form): the split-KV decode's partial
  // kernel went from 81.5-82.8 to 79.5-80.8 us with its non-temporal loads.
  // Elsewhere two spill (d = 256, and 32 columns at d = 128) or were not
  // measured faster.
  constexpr int DEPTH = (D == 128 && NQB == 1) ? 2 : 1;
  // At d = 256 a tile is 128 VGPRs, and Q and two whole tiles would not fit
  // the 256 arch VGPRs: the next tile's V loads are issued once the current
  // V is in LDS and its K loads once the current K has been through the
  // MFMAs, so one tile's worth of K/V is live.  That still keeps as many
  // bytes in flight per wave as a whole d = 128 tile.
  constexpr bool LATE = D > 128;
  constexpr int BK = C::BK;
  constexpr int NC = C::NC;
  constexpr int NDB = C::NDB;
  constexpr int DC = C::DC;
  constexpr int VPL = C::VPL;
  // whole-row K loads with V in `load` (the early-issue order)
  static_assert(!KROW || (!LATE && 2 * NC == VPL), "whole-row K: one K load per V load");
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int lane = threadIdx.x & 63;
  // wave index, made visibly wave-uniform so loops over a wave's tiles are
  // scalar loops (a divergent loop makes the compiler wait on in-flight loads)
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int grp = lane >> 4;

  const int L = blockIdx.x;
  const int nbg = a.B * a.Hkv;
  const int bg = L % nbg;
  const int rest = L / nbg;
  const int n_sg = (a.n_split + a.spw - 1) / a.spw;
  const int sg = rest % n_sg;
  const int qt = a.n_qtiles - 1 - rest / n_sg;
  const int s0 = sg * a.spw;                   // first split of the run
  const int nsp = min(a.spw, a.n_split - s0);  // splits in the run
  const int b = bg / a.Hkv;
  const int g = bg % a.Hkv;
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
  const int row0 = qt * (16 * NQB);
  if (row0 >= rows_total) return;
  // keys read from the cache: all n, or (append) the n - q_len before the
  // query tokens' own keys, which come from k_new / v_new after the loop
  int nl = n;
  if constexpr (PAGED)
    if (a.k_new) nl = max(n - q_len, 0);

  int kbeg = 0, kend = nl;
  if (a.tile > 0) {
    kbeg = s0 * a.tile;
    kend = min(nl, kbeg + nsp * a.tile);
  }
  if (a.causal) {
    const int p_last = (min(row0 + 16 * NQB, rows_total) - 1) / G;
    kend = min(kend, min(max(n - q_len + p_last + 1, 0), n));
  }
  const int ntiles = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  // below wlo no row of the workgroup is masked
  int wlo = kend;
  if (a.causal) wlo = min(kend, min(max(n - q_len + row0 / G + 1, 0), n));

  // ---- this lane's query columns (one per 16-column block)
  bool rvalid[NQB];
  int pq[NQB], hq[NQB], lim[NQB];
  bf16x8 qf[NQB][NC];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int rho = row0 + 16 * qb + c16;
    rvalid[qb] = rho < rows_total;
    pq[qb] = rvalid[qb] ? rho / G : 0;
    hq[qb] = g * G + (rvalid[qb] ? rho - pq[qb] * G : 0);
    lim[qb] = kend;
    if (a.causal) lim[qb] = min(kend, min(max(n - q_len + pq[qb] + 1, 0), n));
    const uint16_t* qp;
    if constexpr (PAGED)
      qp = a.q + (int64_t)(q_row0 + pq[qb]) * a.q_ss + (int64_t)hq[qb] * a.q_sh;
    else
      qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq[qb] * a.q_sh + (int64_t)pq[qb] * a.q_ss;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[qb][c] = rvalid[qb] ? *reinterpret_cast<const bf16x8*>(qp + 32 * c + 8 * grp)
                             : bf16x8{};
  }

  // d = 256: Q goes to LDS once (wave 0 writes, every wave reads it per tile)
  uint16_t* qlds = smem + NW * (C::VTILE + C::KTILE) + 2 * ((NW - 1) * C::SLOT_F) +
                   2 * (PARTIAL ? a.spw * C::PEND_F : 0);
  if constexpr (C::Q_LDS) {
    if (wv == 0) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          *reinterpret_cast<bf16x8*>(qlds + (qb * 16 + c16) * C::QP + 32 * c + 8 * grp) =
              qf[qb][c];
    }
    lds_barrier();
  }
  auto qop = [&](int qb, int c) {
    if constexpr (C::Q_LDS)
      return *reinterpret_cast<const bf16x8*>(qlds + (qb * 16 + c16) * C::QP + 32 * c + 8 * grp);
    else
      return qf[qb][c];
  };

  float m[NQB], l[NQB];
  f32x4 acc[NQB][NDB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m[qb] = -INFINITY;
    if constexpr (!PARTIAL)
      if (a.sink && rvalid[qb]) m[qb] = a.sink[hq[qb]] * kLog2e;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4{};
  }

  // one tile in registers: K in MFMA A layout, V as row chunks.  A tile's
  // 32 rows are loaded through a buffer resource whose size ends at the
  // tile's last row before kv_len (a 32-key tile never straddles a 64-key
  // page), so rows past kv_len read as zeros without touching memory, and
  // keys at or past kend are masked below (P = 0 exactly): whatever such rows
  // hold never reaches the output.  Each lane's offsets are constants; the
  // tile start and its page are wave-uniform scalar work.  Branch-free loads
  // keep the compiler's wait counts exact, which is what lets the next tile's
  // loads stay in flight during this tile's math.
  struct Tile {
    uint4 k[2][NC];
    uint4 v[VPL];
  };
  const uint32_t kss2 = (uint32_t)(PAGED ? a.kv_sr : a.k_ss) * 2u;
  const uint32_t vss2 = (uint32_t)(PAGED ? a.kv_sr : a.v_ss) * 2u;
  uint32_t koff[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) koff[kb] = (uint32_t)(16 * kb + c16) * kss2 + 16u * grp;
  const uint32_t voff = (uint32_t)(lane / DC) * vss2 + 16u * (lane % DC);
  const uint32_t vstep = (uint32_t)(64 / DC) * vss2;
  // whole-row K: chunk j of the lane is row lane / DC + j (64 / DC), 16-byte
  // slot lane % DC (the V pattern), kept in t.k[j / NC][j % NC]
  const uint32_t kroff = (uint32_t)(lane / DC) * kss2 + 16u * (lane % DC);
  const uint32_t krstep = (uint32_t)(64 / DC) * kss2;
  // page table through the constant address space: uniform reads become
  // scalar loads, which do not queue behind the tile loads in flight
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)a.page_table;
  // `live` false: a prefetch past the wave's last tile (it re-addresses that
  // tile); its resources are empty, so the loads return zeros without
  // touching memory, and the tile is never used.
  auto load = [&](int j0, Tile& t, bool live) {
    const uint16_t *kp, *vp;
    if constexpr (PAGED) {
      const int pg = ptab[(int64_t)b * a.max_pages + (j0 >> 6)];
      const int64_t off = (int64_t)pg * a.kv_sp + (int64_t)(j0 & 63) * a.kv_sr;
      kp = a.k + off + (int64_t)g * a.k_sh;
      vp = a.v + off + (int64_t)g * a.v_sh;
    } else {
      kp = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh + (int64_t)j0 * a.k_ss;
      vp = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh + (int64_t)j0 * a.v_ss;
    }
    const uint32_t valid = (uint32_t)min(BK, nl - j0);  // >= 1: tiles start below kend <= nl
    const BufRes kr = make_bufres(kp, live ? (valid - 1u) * kss2 + (uint32_t)D * 2u : 0u);
    const BufRes vr = make_bufres(vp, live ? (valid - 1u) * vss2 + (uint32_t)D * 2u : 0u);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if constexpr (KROW)
          t.k[kb][c] = buf_load16<CP>(kr, kroff + (uint32_t)(kb * NC + c) * krstep);
        else
          t.k[kb][c] = buf_load16<CP>(kr, koff[kb] + 64u * c);
      }
#pragma unroll
    for (int j = 0; j < VPL; ++j) t.v[j] = buf_load16<CP>(vr, voff + (uint32_t)j * vstep);
  };
  // the K (which = 0) or V (which = 1) half of `load`, for the late-issue order
  // (operand-shaped K only)
  auto tile_res = [&](int j0, int which, bool live) {
    const uint16_t* p;
    if constexpr (PAGED) {
      const int pg = ptab[(int64_t)b * a.max_pages + (j0 >> 6)];
      const int64_t off = (int64_t)pg * a.kv_sp + (int64_t)(j0 & 63) * a.kv_sr;
      p = which ? a.v + off + (int64_t)g * a.v_sh : a.k + off + (int64_t)g * a.k_sh;
    } else {
      p = which ? a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh + (int64_t)j0 * a.v_ss
                : a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh + (int64_t)j0 * a.k_ss;
    }
    const uint32_t valid = (uint32_t)min(BK, nl - j0);  // >= 1: tiles start below kend <= nl
    return make_bufres(p, live ? (valid - 1u) * (which ? vss2 : kss2) + (uint32_t)D * 2u : 0u);
  };
  auto load_k = [&](int j0, Tile& t, bool live) {
    const BufRes kr = tile_res(j0, 0, live);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < NC; ++c) t.k[kb][c] = buf_load16<CP>(kr, koff[kb] + 64u * c);
  };
  auto load_v = [&](int j0, Tile& t, bool live) {
    const BufRes vr = tile_res(j0, 1, live);
#pragma unroll
    for (int j = 0; j < VPL; ++j) t.v[j] = buf_load16<CP>(vr, voff, (uint32_t)j * vstep);
  };

  uint16_t* vbuf = smem + wv * C::VTILE;
  uint16_t* kbuf = smem + NW * C::VTILE + wv * C::KTILE;
  float* slots = reinterpret_cast<float*>(smem + NW * (C::VTILE + C::KTILE));
  float* pend = slots + (NW - 1) * C::SLOT_F;  // parked split states (partial mode)

  // At d = 256 the swizzle repeats every 8 key rows: V row writes need 4
  // per-lane LDS offsets and the transposing reads 8 (one per d block mod 8),
  // with the rest as immediates.  (Recomputing all 16 + 32 offsets per lane
  // costs more registers than the tiles leave.)
  constexpr int RPJ = 64 / DC;                    // V rows per 64-lane chunk step
  constexpr int WPER = RPJ >= 8 ? 1 : 8 / RPJ;    // chunk steps per swizzle period
  constexpr int RPER = NDB < 8 ? NDB : 8;
  int vwo[WPER], vro[RPER];
  if constexpr (LATE) {
#pragma unroll
    for (int jl = 0; jl < WPER; ++jl) {
      const int kl = lane / DC + RPJ * jl;
      vwo[jl] = kl * D + 8 * ((lane % DC) ^ vslot_swz<DC>(kl));
    }
    const int kl0 = 4 * grp + (c16 >> 2);
    const int sw = vslot_swz<DC>(kl0);
#pragma unroll
    for (int dl = 0; dl < RPER; ++dl)
      vro[dl] = kl0 * D + 8 * ((2 * dl + ((c16 & 3) >> 1)) ^ sw) + 4 * (c16 & 1);
  }
  // V tile -> wave-private LDS (row-major, swizzled 16-byte slots)
  auto stage_v = [&](const Tile& t) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      if constexpr (LATE) {
        *reinterpret_cast<uint4*>(vbuf + vwo[j % WPER] + (j / WPER) * 8 * D) = t.v[j];
      } else {
        const int ci = lane + 64 * j;
        const int kl = ci / DC;
        const int slot = (ci % DC) ^ vslot_swz<DC>(kl);
        *reinterpret_cast<uint4*>(vbuf + kl * D + 8 * slot) = t.v[j];
      }
    }
  };
  // whole-row K tile -> wave-private LDS (row-major, padded rows)
  const int kwo = (lane / DC) * C::KP + 8 * (lane % DC);
  const int kro = c16 * C::KP + 8 * grp;
  auto stage_k = [&](const Tile& t) {
#pragma unroll
    for (int j = 0; j < 2 * NC; ++j)
      *reinterpret_cast<uint4*>(kbuf + kwo + j * (64 / DC) * C::KP) = t.k[j / NC][j % NC];
  };
  // S^T = K Q^T for two 16-key blocks; the A operand (key row 16 kb + c16,
  // d 32 c + 8 grp .. + 7) from the registers, or read back from the K tile
  auto qk = [&](const Tile& t, f32x4 (&s)[NQB][2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb][kb] = f32x4{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          bf16x8 ka;
          if constexpr (KROW)
            ka = *reinterpret_cast<const bf16x8*>(kbuf + kro + 16 * kb * C::KP + 32 * c);
          else
            ka = __builtin_bit_cast(bf16x8, t.k[kb][c]);
          s[qb][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qop(qb, c), s[qb][kb], 0, 0, 0);
        }
      }
  };
  // mask, online softmax and O^T += V^T P^T of the tile at key j0
  auto finish = [&](int j0, f32x4 (&s)[NQB][2]) {
    // register r of block kb holds key j0 + 16 kb + 4 grp + r
    if (j0 + BK > wlo) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (j0 + 16 * kb + 4 * grp + r >= lim[qb]) s[qb][kb][r] = -INFINITY;
    }
    bf16x8 pb[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      float mx = fmaxf(fmaxf(fmaxf(s[qb][0][0], s[qb][0][1]), fmaxf(s[qb][0][2], s[qb][0][3])),
                       fmaxf(fmaxf(s[qb][1][0], s[qb][1][1]), fmaxf(s[qb][1][2], s[qb][1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m[qb], mx * a.scale_log2);
      const float mu = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = ex2(m[qb] - mu);
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const __bf16 pj = (__bf16)ex2(__builtin_fmaf(s[qb][kb][r], a.scale_log2, -mu));
          pb[qb][4 * kb + r] = pj;
          ls += (float)pj;  // the sum uses the same rounded weights as P.V
        }
      l[qb] = l[qb] * alpha + ls;
      m[qb] = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[qb][db] *= alpha;
    }
    // O^T += V^T P^T; A operand by two transposing LDS reads per d block
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      i16x4 va[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint16_t* src;
        if constexpr (LATE) {
          // slot (2 db + x) ^ sw = 16 (db / 8) + ((2 (db % 8) + x) ^ sw), sw < 16
          src = vbuf + vro[db % RPER] + 16 * half * D + 128 * (db / RPER);
        } else {
          const int kl = 16 * half + 4 * grp + (c16 >> 2);
          const int slot = (2 * db + ((c16 & 3) >> 1)) ^ vslot_swz<DC>(kl);
          src = vbuf + kl * D + 8 * slot + 4 * (c16 & 1);
        }
        va[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(src));
      }
      const bf16x8 vv = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(va[0], va[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[qb], acc[qb][db], 0, 0, 0);
    }
  };
  auto compute = [&](int j0, const Tile& t) {
    f32x4 s[NQB][2];
    qk(t, s);
    finish(j0, s);
  };

  // ---- end of a split: combine the NW waves' states through LDS (wave 0
  // keeps the result), write the split's partial or the final output, and
  // start the next split from the empty state.  Every wave calls this once
  // per split of the run, in order, so the barriers match.
  auto flush = [&](int s) __attribute__((always_inline)) {
    if constexpr (NW > 1) {
      if (s > 0) lds_barrier();  // wave 0 has read the previous split's slots
      if (wv > 0) {
        float* red = slots + (wv - 1) * C::SLOT_F;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float* r = red + qb * (2 + 4 * NDB) * 64;
          r[lane] = m[qb];
          r[64 + lane] = l[qb];
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e) r[(2 + 4 * db + e) * 64 + lane] = acc[qb][db][e];
        }
      }
      lds_barrier();
      if (wv == 0) {
#pragma unroll 1
        for (int w2 = 1; w2 < NW; ++w2) {
          const float* base = slots + (w2 - 1) * C::SLOT_F;
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float* r = base + qb * (2 + 4 * NDB) * 64;
            const float m2 = r[lane];
            const float l2 = r[64 + lane];
            const float mn = fmaxf(m[qb], m2);
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            const float wa = ex2(m[qb] - mu);
            const float wb = ex2(m2 - mu);
            l[qb] = l[qb] * wa + l2 * wb;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                acc[qb][db][e] = acc[qb][db][e] * wa + r[(2 + 4 * db + e) * 64 + lane] * wb;
            m[qb] = mn;
          }
        }
      }
    }
    // epilogue (wave 0); acc[qb][db][e] holds d = 16 db + 4 grp + e of column c16
    if (wv == 0) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float lt = l[qb];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        if (!rvalid[qb]) continue;
        const int p = pq[qb], h = hq[qb];
        if constexpr (PARTIAL) {
          // park the split's state in LDS; it is written out after the loop
          float* pc = pend + ((s * NQB + qb) * 16 + c16) * C::PSTR;
          if (grp == 0)
            *reinterpret_cast<float2*>(pc + D) =
                make_float2(m[qb] == -INFINITY ? -INFINITY : m[qb] * kLn2, lt);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<float4*>(pc + 16 * db + 4 * grp) =
                make_float4(acc[qb][db][0], acc[qb][db][1], acc[qb][db][2], acc[qb][db][3]);
        } else {
          float sl2 = -INFINITY;
          if (a.sink) sl2 = a.sink[h] * kLog2e;
          if (sl2 != -INFINITY) lt += ex2(sl2 - m[qb]);
          const float inv = lt > 0.f ? 1.f / lt : 0.f;
          uint16_t* op;
          if constexpr (PAGED)
            op = a.o + (int64_t)(q_row0 + p) * a.o_ss + (int64_t)h * a.o_sh;
          else
            op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)p * a.o_ss;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<uint2*>(op + 16 * db + 4 * grp) =
                make_uint2(pack_bf16x2(acc[qb][db][0] * inv, acc[qb][db][1] * inv),
                           pack_bf16x2(acc[qb][db][2] * inv, acc[qb][db][3] * inv));
        }
      }
    }
    if constexpr (PARTIAL) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        m[qb] = -INFINITY;
        l[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[qb][db] = f32x4{};
      }
    }
  };

  // ---- key loop: this wave takes tiles wv, wv + NW, ... of the run;
  // DEPTH + 1 register tiles in rotation.  The prefetch is unconditional
  // (past the end it addresses the wave's last tile through empty resources,
  // so nothing is read) so no branch sits between a load and the compute
  // that must not wait for it.
  // Splits are multiples of 64 keys, so no tile straddles two of them.  The
  // finished splits are flushed before the first tile of a later split, at a
  // point where that tile (and the DEPTH - 1 after it) is in flight and the
  // remaining register tile is free.
  {
    const int tps = a.tile > 0 ? a.tile / BK : 0x7fffffff;  // tiles per split
    int cur = 0;                 // split (within the run) being accumulated
    int next_tile = tps;         // first tile of split cur + 1
    auto enter = [&](int k) __attribute__((always_inline)) {
      const int t = wv + NW * k;
      while (t >= next_tile) {
        flush(cur);
        ++cur;
        next_tile += tps;
      }
    };
    const int mine = wv < ntiles ? (ntiles - wv + NW - 1) / NW : 0;
    auto tile_key = [&](int k) { return kbeg + (wv + NW * min(k, mine - 1)) * BK; };
    if (mine > 0) {
      Tile t[DEPTH + 1];
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) load(tile_key(u), t[u], u < mine);
      // The exit leaves both loops at once: a path back through the loop
      // head with a prefetched tile left unconsumed would make the compiler
      // wait for that tile on every iteration.
      for (int k = 0;; k += DEPTH + 1) {
#pragma unroll
        for (int u = 0; u <= DEPTH; ++u) {
          if (k + u >= mine) goto keys_done;
          enter(k + u);
          Tile& nx = t[(u + DEPTH) % (DEPTH + 1)];
          if constexpr (!LATE) {
            load(tile_key(k + u + DEPTH), nx, k + u + DEPTH < mine);
            // keep the prefetch ahead of the first wait on tile k + u
            __builtin_amdgcn_sched_barrier(0);
            stage_v(t[u]);
            if constexpr (KROW) stage_k(t[u]);
            compute(tile_key(k + u), t[u]);
          } else {
            // next V once this V is in LDS, next K once this K has been used
            stage_v(t[u]);
            load_v(tile_key(k + u + DEPTH), nx, k + u + DEPTH < mine);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 s[NQB][2];
            qk(t[u], s);
            __builtin_amdgcn_sched_barrier(0);
            load_k(tile_key(k + u + DEPTH), nx, k + u + DEPTH < mine);
            __builtin_amdgcn_sched_barrier(0);
            finish(tile_key(k + u), s);
          }
        }
      }
    }
  keys_done:
    if constexpr (PAGED) {
      // append: the query tokens' own keys nl .. n - 1 (at most 32) count
      // once, in the split holding key n - 1, as one more tile of wave 0,
      // loaded straight from k_new / v_new (no workgroup reads those cache
      // rows in this launch); the workgroup of q-tile 0 also writes them
      // into their cache pages.
      const int nnew = n - nl;
      const int s_new = a.tile > 0 ? (n - 1) / a.tile : 0;
      if (a.k_new && nnew > 0 && s_new >= s0 && s_new < s0 + nsp) {
        while (cur < s_new - s0) {
          flush(cur);
          ++cur;
        }
        const int64_t t0 = q_row0 + q_len - nnew;  // packed row of key nl
        const uint16_t* kn = a.k_new + t0 * a.new_st + (int64_t)g * a.new_sh;
        const uint16_t* vn = a.v_new + t0 * a.new_st + (int64_t)g * a.new_sh;
        if (wv == 0) {
          const uint32_t ns2 = (uint32_t)a.new_st * 2u;
          const BufRes kr = make_bufres(kn, (uint32_t)(nnew - 1) * ns2 + (uint32_t)D * 2u);
          const BufRes vr = make_bufres(vn, (uint32_t)(nnew - 1) * ns2 + (uint32_t)D * 2u);
          Tile tn;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              if constexpr (KROW)
                tn.k[kb][c] = buf_load16<CP>(
                    kr, (uint32_t)(lane / DC + (kb * NC + c) * (64 / DC)) * ns2 + 16u * (lane % DC));
              else
                tn.k[kb][c] =
                    buf_load16<CP>(kr, (uint32_t)(16 * kb + c16) * ns2 + 64u * c + 16u * grp);
            }
#pragma unroll
          for (int j = 0; j < VPL; ++j)
            tn.v[j] = buf_load16<CP>(vr, (uint32_t)(lane / DC + j * (64 / DC)) * ns2 +
                                         16u * (lane % DC));
          // every key of the tile goes through the mask: key nl + r is
          // visible up to the row's causal bound, and rows r >= nnew not at all
          wlo = nl;
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            lim[qb] = a.causal ? min(max(n - q_len + pq[qb] + 1, 0), n) : n;
          stage_v(tn);
          if constexpr (KROW) stage_k(tn);
          compute(nl, tn);
        }
        if (qt == 0) {
          uint16_t* kc = const_cast<uint16_t*>(a.k) + (int64_t)g * a.k_sh;
          uint16_t* vc = const_cast<uint16_t*>(a.v) + (int64_t)g * a.v_sh;
          for (int idx = threadIdx.x; idx < 2 * nnew * DC; idx += NW * 64) {
            const int which = idx >= nnew * DC;
            const int rem = idx - which * nnew * DC;
            const int r = rem / DC, ch = rem % DC;
            const int key = nl + r;
            const int64_t dst = (int64_t)a.page_table[(int64_t)b * a.max_pages + (key >> 6)] *
                                    a.kv_sp +
                                (int64_t)(key & 63) * a.kv_sr + 8 * ch;
            const int64_t src = (int64_t)r * a.new_st + 8 * ch;
            *reinterpret_cast<uint4*>((which ? vc : kc) + dst) =
                *reinterpret_cast<const uint4*>((which ? vn : kn) + src);
          }
        }
      }
    }
    while (cur < nsp) {
      flush(cur);
      ++cur;
    }
  }

  // ---- split partials: the run's parked states go out with coalesced
  // stores, two query columns per wave instruction (one at d = 256).  Global stores stay out
  // of the key loop, where the registers they read would have to be guarded
  // by waits that also hold back the prefetch.
  if constexpr (PARTIAL) {
    lds_barrier();
    constexpr int LPC = D / 4;              // lanes per column (float4 each)
    constexpr int CPI = LPC <= 32 ? 2 : 1;  // columns per wave instruction
    const int half = CPI == 2 ? lane >> 5 : 0;
    const int ln = CPI == 2 ? lane & 31 : lane;
    for (int it = CPI * wv + half; it < nsp * NQB * 16; it += CPI * NW) {
      const int s = it / (NQB * 16);
      const int qb = (it / 16) % NQB;
      const int col = it % 16;
      const int rho = row0 + 16 * qb + col;
      if (rho >= rows_total) continue;
      const int p = rho / G, h = g * G + (rho - p * G);
      int64_t row;
      if constexpr (PAGED)
        row = (int64_t)h * a.total_q + q_row0 + p;
      else
        row = ((int64_t)b * a.Hq + h) * a.Sq + p;
      const int64_t idx = row * a.n_split + s0 + s;
      const float* pc = pend + ((s * NQB + qb) * 16 + col) * C::PSTR;
      if (a.tickets) {
        // in-kernel merge: system-scope stores go through to memory, which
        // leaves the device-scope release below less to write back
        if (ln < LPC)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(a.ws_o + idx * D + 4 * ln) + e,
                               __float_as_uint(pc[4 * ln + e]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
        if (ln == 0)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(a.ws_ml + idx) + e,
                               __float_as_uint(pc[D + e]), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
      } else {
        if (ln < LPC)
          *reinterpret_cast<float4*>(a.ws_o + idx * D + 4 * ln) =
              *reinterpret_cast<const float4*>(pc + 4 * ln);
        if (ln == 0) a.ws_ml[idx] = *reinterpret_cast<const float2*>(pc + D);
      }
    }

    // ---- in-kernel merge.  The pattern is the AstrAI commit log's scale-ring
    // epilogue (after a fence, a counter elects the last block, which
    // finishes the reduction in the same launch).  Here every lane's partial
    // stores are released device-wide, each workgroup takes a ticket for its
    // (b, kv head, q-tile), and the one that draws the last of the n_sg
    // tickets acquires the others' partials, merges every split of its rows
    // (the merge kernel's arithmetic, sink included) and resets the ticket.
    // No workgroup waits on another.
    if (a.tickets) {
      // The barrier makes every wave's stores visible to thread 0, whose
      // device-scope fences then release them (and, for the last workgroup,
      // acquire the others' partials) for the whole workgroup: on gfx950 a
      // device-scope release writes back the XCD's L2, so one per workgroup.
      __syncthreads();
      int* flag = reinterpret_cast<int*>(slots);
      if (threadIdx.x == 0) {
        int32_t* tk = a.tickets + (int64_t)bg * a.n_qtiles + qt;
        __threadfence();
        const int last = atomicAdd(tk, 1) == n_sg - 1;
        if (last) {
          atomicExch(tk, 0);
          __threadfence();
        }
        *flag = last;
      }
      __syncthreads();
      if (*flag == 0) return;
      for (int it = CPI * wv + half; it < NQB * 16; it += CPI * NW) {
        const int rho = row0 + it;
        if (rho >= rows_total) continue;
        const int p = rho / G, h = g * G + (rho - p * G);
        int64_t row;
        if constexpr (PAGED)
          row = (int64_t)h * a.total_q + q_row0 + p;
        else
          row = ((int64_t)b * a.Hq + h) * a.Sq + p;
        const float2* ml = a.ws_ml + row * a.n_split;
        const float* ot = a.ws_o + row * a.n_split * D + 4 * ln;
        const float sk = a.sink ? a.sink[h] : -INFINITY;  // scaled domain, natural log
        float M = sk;
        for (int sp = 0; sp < a.n_split; ++sp) M = fmaxf(M, ml[sp].x);
        float L = sk == -INFINITY ? 0.f : __expf(sk - M);
        float4 o4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (M != -INFINITY) {
          for (int sp = 0; sp < a.n_split; ++sp) {
            const float2 st = ml[sp];
            if (st.x == -INFINITY) continue;  // empty split: weight 0
            const float w = __expf(st.x - M);
            L += st.y * w;
            if (ln < LPC) {
              const float4 ov = *reinterpret_cast<const float4*>(ot + (int64_t)sp * D);
              o4.x += w * ov.x;
              o4.y += w * ov.y;
              o4.z += w * ov.z;
              o4.w += w * ov.w;
            }
          }
        }
        const float inv = (M != -INFINITY && L > 0.f) ? 1.f / L : 0.f;
        uint16_t* op;
        if constexpr (PAGED)
          op = a.o + (int64_t)(q_row0 + p) * a.o_ss + (int64_t)h * a.o_sh;
        else
          op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)p * a.o_ss;
        if (ln < LPC)
          *reinterpret_cast<uint2*>(op + 4 * ln) =
              make_uint2(pack_bf16x2(o4.x * inv, o4.y * inv), pack_bf16x2(o4.z * inv, o4.w * inv));
      }
    }
  }
}

}  // namespace gqa
