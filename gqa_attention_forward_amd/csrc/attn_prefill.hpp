// Prefill GQA forward kernel: query groups of more than 32 rows per
// (b, kv head).  One workgroup per (b, kv head g, q-tile of 32 * NW rows,
// kv split); all NW waves share each 64-key K/V tile through LDS, so a tile
// is fetched once per workgroup for every query head of the group (AstrAI
// commit log, the commit that packs HB = min(G, warps) query heads per
// block).
//
// MFMA mapping, v_mfma_f32_32x32x16_bf16, NB blocks of 32 query rows per
// wave (the MFMA N dimension; with NB = 2 every K and V operand read from
// LDS feeds two MFMAs, and each block's softmax can overlap the other
// block's MFMAs inside one wave):
//   S^T = K Q^T  : A = K rows from LDS, read in a permuted row order (bits 2
//                  and 3 of the row index swapped) so that accumulator
//                  registers 8t..8t+7 of a lane hold 8 consecutive keys;
//                  B = Q in registers.  A lane holds one query row's scores,
//                  so row max/sum reductions are in-lane plus one exchange
//                  with lane ^ 32.
//   O^T += V^T P^T: B = P straight from the S^T accumulators (bf16), A = V^T
//                  gathered from the row-major V tile with two
//                  ds_read_b64_tr_b16 per MFMA (within each 16-lane group,
//                  destination lane i, element e comes from source lane
//                  4e + i/4, element i%4).
// K tiles are stored row-major with a padded pitch (D + 8 elements), V tiles
// row-major unpadded with 16-byte slots XOR-swizzled per row (vslot_swz), so
// the row writes, the K operand reads and the transposing V reads are all
// bank-conflict free (checked with the LDS bank-conflict counter), and K
// operand addresses are one base plus immediate offsets.
//
// Online softmax in base 2 with a lazily moved reference: a row's reference
// m only moves when the tile max exceeds it by more than 8 (log2 units), so
// the O / l rescale is skipped on most tiles; P = 2^(s - m) <= 2^8 then.
// The algebra is unchanged -- (m, l, O) stay consistent -- and the final
// division by l happens once (nvfp4-megamoe-kernel commit log, multi-tile
// FA2 and normalise-once commits).
#pragma once

#include "common.hpp"

namespace gqa {

template <int D, int NW, int NB>
struct PrefillCfg {
  static constexpr int BK = 64;              // keys per tile
  static constexpr int DC = D / 8;           // 16-byte chunks per row
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = 32 * NB * NW;  // query rows per workgroup
  static constexpr int KP = D + 8;           // K row pitch (elements): padded, not swizzled
  static constexpr int KTILE = BK * KP;      // elements of one K tile
  static constexpr int TILE = BK * D;        // elements of one V tile
  static constexpr int STAGE = KTILE + TILE; // K then V
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int CPT = BK * DC / NT;   // chunks per thread per tensor
  static_assert(CPT >= 1 && BK * DC % NT == 0, "tile split");
};

constexpr float kLazyRescale = 8.f;  // log2 units

// Two waves per SIMD with one 32-row block per wave; one wave per SIMD (and
// room for 2x the state) with two.
template <int D, int NW, int NB, bool PAGED, bool PARTIAL>
__global__ void __launch_bounds__(NW * 64, NB == 1 ? 2 : 1)
attn_prefill_kernel(const AttnArgs a) {
  using C = PrefillCfg<D, NW, NB>;
  constexpr int NT = C::NT;
  constexpr int BK = C::BK;
  constexpr int DC = C::DC;
  constexpr int CPT = C::CPT;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int col = lane & 31;
  const int hl = lane >> 5;

  const int L = blockIdx.x;
  const int nbg = a.B * a.Hkv;
  const int bg = L % nbg;
  const int rest = L / nbg;
  const int split = rest % a.n_split;
  const int qt = a.n_qtiles - 1 - rest / a.n_split;  // late (heavy causal) q-tiles first
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

  // ---- this lane's query rows (one per 32-row block) and masking bounds
  const int wrow0 = row0 + 32 * NB * wv;
  int wlo = kend;  // below wlo no row of the wave is masked
  if (a.causal) wlo = min(kend, min(max(n - q_len + wrow0 / G + 1, 0), n));
  if (wrow0 >= rows_total) wlo = kbeg;
  bool rvalid[NB];
  int pq[NB], hq[NB], lim[NB];
  bf16x8 qf[NB][D / 16];  // Q operand: row `col` of block nb, d = 16 c + 8 hl + e
  float sl2[NB], mref[NB], mtrue[NB], l[NB];
  f32x16 acc[NB][D / 32];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int rho = wrow0 + 32 * nb + col;
    rvalid[nb] = rho < rows_total;
    pq[nb] = rvalid[nb] ? rho / G : 0;
    hq[nb] = g * G + (rvalid[nb] ? rho - pq[nb] * G : 0);
    lim[nb] = kend;
    if (a.causal) lim[nb] = min(kend, min(max(n - q_len + pq[nb] + 1, 0), n));
    const uint16_t* qp;
    if constexpr (PAGED)
      qp = a.q + (int64_t)(q_row0 + pq[nb]) * a.q_ss + (int64_t)hq[nb] * a.q_sh;
    else
      qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq[nb] * a.q_sh + (int64_t)pq[nb] * a.q_ss;
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[nb][c] = rvalid[nb] ? *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hl) : bf16x8{};
    sl2[nb] = -INFINITY;  // sink in log2 units (final mode)
    if constexpr (!PARTIAL)
      if (a.sink && rvalid[nb]) sl2[nb] = a.sink[hq[nb]] * kLog2e;
    mref[nb] = sl2[nb];   // reference the running sums are taken against
    mtrue[nb] = sl2[nb];  // true running max (for the partial epilogue)
    l[nb] = 0.f;          // this lane's share of the running sum
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[nb][i] = f32x16{};
  }

  // ---- K/V staging: chunk ci = tid + i NT of a 64 x DC tile.  A 64-key
  // tile is one page of the paged layout; its rows load through a buffer
  // resource whose size ends at the tile's last row before kv_len, so rows
  // past kv_len read as zeros without touching memory (and are masked).
  // Each thread's offsets are constants; tile start and page are scalar.
  struct Stage {
    u32x4 k[CPT];
    u32x4 v[CPT];
  };
  const uint32_t kss2 = (uint32_t)(PAGED ? a.kv_sr : a.k_ss) * 2u;
  const uint32_t vss2 = (uint32_t)(PAGED ? a.kv_sr : a.v_ss) * 2u;
  const uint32_t koff0 = (uint32_t)(tid / DC) * kss2 + 16u * (tid % DC);
  const uint32_t voff0 = (uint32_t)(tid / DC) * vss2 + 16u * (tid % DC);
  static_assert(NT % DC == 0, "row step");
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)a.page_table;
  auto load_tile = [&](int j0, Stage& st) {
    const uint16_t *kp, *vp;
    if constexpr (PAGED) {
      const int pg = ptab[(int64_t)b * a.max_pages + (j0 >> 6)];
      kp = a.k + (int64_t)pg * a.kv_sp + (int64_t)g * a.k_sh;
      vp = a.v + (int64_t)pg * a.kv_sp + (int64_t)g * a.v_sh;
    } else {
      kp = a.k + (int64_t)b * a.k_sb + (int64_t)g * a.k_sh + (int64_t)j0 * a.k_ss;
      vp = a.v + (int64_t)b * a.v_sb + (int64_t)g * a.v_sh + (int64_t)j0 * a.v_ss;
    }
    const uint32_t valid = (uint32_t)min(BK, n - j0);  // >= 1: tiles start below kend <= n
    const BufRes kr = make_bufres(kp, (valid - 1u) * kss2 + (uint32_t)D * 2u);
    const BufRes vr = make_bufres(vp, (valid - 1u) * vss2 + (uint32_t)D * 2u);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      st.k[i] = buf_load16v(kr, koff0 + (uint32_t)(i * (NT / DC)) * kss2);
      st.v[i] = buf_load16v(vr, voff0 + (uint32_t)(i * (NT / DC)) * vss2);
    }
  };
  auto store_tile = [&](int stage, const Stage& st) {
    uint16_t* Ks = smem + stage * C::STAGE;
    uint16_t* Vs = Ks + C::KTILE;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ci = tid + i * NT;
      const int row = ci / DC, ch = ci % DC;
      *reinterpret_cast<u32x4*>(Ks + row * C::KP + 8 * ch) = st.k[i];
      *reinterpret_cast<u32x4*>(Vs + row * D + 8 * (ch ^ vslot_swz<DC>(row))) = st.v[i];
    }
  };

  Stage nx;
  if (ntiles > 0) {
    load_tile(kbeg, nx);
    store_tile(0, nx);
  }
  lds_barrier();

  const int krow_a = swap_bits23(col);  // K row (within a 32-key block) this lane feeds to MFMA
  const int g16 = lane >> 4;
  const int r16 = lane & 15;

  for (int it = 0; it < ntiles; ++it) {
    const int j0 = kbeg + it * BK;
    // The prefetch of the next tile is unconditional (past the end it
    // re-reads the last tile, an L2 hit): with no branch around it the
    // compiler keeps it ahead of the compute instead of sinking it to its
    // LDS store.
    load_tile(kbeg + min(it + 1, ntiles - 1) * BK, nx);
    const uint16_t* Ks = smem + (it & 1) * C::STAGE;
    const uint16_t* Vs = Ks + C::KTILE;

    // S^T = K Q^T: register j of s[nb][mb] = key j0 + 32 mb + 16 (j >> 3) + 8 hl + (j & 7)
    f32x16 s[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb][0] = s[nb][1] = f32x16{};
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kk = *reinterpret_cast<const bf16x8*>(Ks + (32 * mb + krow_a) * C::KP +
                                                           16 * c + 8 * hl);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          s[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qf[nb][c], s[nb][mb], 0, 0, 0);
      }
    if (__builtin_expect(j0 + BK > wlo, 0)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int rem = lim[nb] - j0 - 8 * hl;  // first masked offset of this lane
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            if (32 * mb + 16 * (j >> 3) + (j & 7) >= rem) s[nb][mb][j] = -INFINITY;
      }
    }

    // online softmax: tile max, lazy reference move (rare O rescale)
    float mx[NB];
    bool move[NB];
    bool any_move = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float m = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) m = fmaxf(m, s[nb][mb][j]);
      mx[nb] = xor32_max(m) * a.scale_log2;
      mtrue[nb] = fmaxf(mtrue[nb], mx[nb]);
      move[nb] = mx[nb] > mref[nb] + kLazyRescale;
      any_move |= move[nb];
    }
    if (__any(any_move)) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float alpha = move[nb] ? ex2(mref[nb] - mx[nb]) : 1.f;  // 0 when mref = -inf
        l[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) acc[nb][db][j] *= alpha;
        mref[nb] = move[nb] ? mx[nb] : mref[nb];
      }
    }
    // P rounded to bf16 in pairs; the row sum is taken over the same rounded
    // values with a packed dot against (1, 1)
    bf16x8 pb[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float mu = (mref[nb] == -INFINITY) ? 0.f : mref[nb];
      float ls = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          bf16x2 pp;
          pp[0] = (__bf16)ex2(__builtin_fmaf(s[nb][t >> 1][8 * (t & 1) + e], a.scale_log2, -mu));
          pp[1] = (__bf16)ex2(__builtin_fmaf(s[nb][t >> 1][8 * (t & 1) + e + 1], a.scale_log2, -mu));
          pb[nb][t][e] = pp[0];
          pb[nb][t][e + 1] = pp[1];
          ls = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls, false);
        }
      l[nb] += ls;
    }

    // O^T += V^T P^T; the V operand is two transposing LDS reads per MFMA
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int cc = 32 * db + 16 * (g16 & 1) + 4 * (r16 & 3);
        i16x4 va[2];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int key = 16 * t + 8 * hl + 4 * half + (r16 >> 2);
          va[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4*)(Vs + key * D +
                                                         8 * ((cc >> 3) ^ vslot_swz<DC>(key)) +
                                                         (cc & 7)));
        }
        const bf16x8 vv = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(va[0], va[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[nb][t], acc[nb][db], 0, 0, 0);
      }
    }

    store_tile((it + 1) & 1, nx);
    lds_barrier();
  }

  // ---- epilogue; accumulator register j of d-block db holds
  //      d = 32 db + 8 (j >> 2) + 4 hl + (j & 3) of query row `col`
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float lt = xor32_sum(l[nb]);
    const int p = pq[nb], h = hq[nb];
    if constexpr (PARTIAL) {
      // report the state against the true max (as the partial format states)
      const float f = (mtrue[nb] == -INFINITY) ? 0.f : ex2(mref[nb] - mtrue[nb]);
      lt *= f;
      if (!rvalid[nb]) continue;
      int64_t row;
      if constexpr (PAGED)
        row = (int64_t)h * a.total_q + q_row0 + p;
      else
        row = ((int64_t)b * a.Hq + h) * a.Sq + p;
      const int64_t idx = row * a.n_split + split;
      if (hl == 0)
        a.ws_ml[idx] = make_float2(mtrue[nb] == -INFINITY ? -INFINITY : mtrue[nb] * kLn2, lt);
      float* op = a.ws_o + idx * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(op + 32 * db + 8 * q4 + 4 * hl) =
              make_float4(acc[nb][db][4 * q4] * f, acc[nb][db][4 * q4 + 1] * f,
                          acc[nb][db][4 * q4 + 2] * f, acc[nb][db][4 * q4 + 3] * f);
    } else {
      if (sl2[nb] != -INFINITY) lt += ex2(sl2[nb] - mref[nb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      if (!rvalid[nb]) continue;
      uint16_t* op;
      if constexpr (PAGED)
        op = a.o + (int64_t)(q_row0 + p) * a.o_ss + (int64_t)h * a.o_sh;
      else
        op = a.o + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + (int64_t)p * a.o_ss;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<uint2*>(op + 32 * db + 8 * q4 + 4 * hl) =
              make_uint2(pack_bf16x2(acc[nb][db][4 * q4] * inv, acc[nb][db][4 * q4 + 1] * inv),
                         pack_bf16x2(acc[nb][db][4 * q4 + 2] * inv, acc[nb][db][4 * q4 + 3] * inv));
    }
  }
}

}  // namespace gqa
