// GQA forward for wide heads (d = 512), two kernels.  The nvfp4-megamoe-kernel
// commit log sweeps head dims 64 to 512 and sends d = 512 to its multi-tile
// kernel; here a 32-row block's output alone would be 256 fp32 accumulators
// per lane at d = 512, so no wave holds all of it.  Groups of up to 32 rows
// per (b, kv head) split the head dim across the four waves of a workgroup
// (attn_wide_kernel); larger groups give each wave 16 rows over the whole
// head dim (attn_wide_rows_kernel, below).
//
// attn_wide_kernel:
// One workgroup per (b, kv head g, q-tile of 32 rows, kv split); its rows are
// the flattened (position, head-in-group) pairs of one kv group, as in the
// other kernels (AstrAI commit log, the commit that packs HB = min(G, warps)
// query heads per block), and every K/V element is read from memory once per
// workgroup.  Wave w owns d columns [128 w, 128 w + 128):
//   S_w^T = K_w Q_w^T        partial scores over its d slice; K_w is loaded
//                            straight into the MFMA operand layout
//                            (v_mfma_f32_32x32x16_bf16, 32 keys x 16 d per
//                            step, key rows in the bit-2/3-swapped order that
//                            makes the accumulators the next MFMA's operand)
//   S = S_0 + S_1 + S_2 + S_3 summed through LDS in that fixed order, so all
//                            four waves hold the same scores, bit for bit
//   softmax of S             the same in every wave (online, base 2, lazy
//                            reference, P rounded to bf16 with the row sum
//                            over the rounded values), so m and l agree
//   O_w^T += V_w^T P^T       its d slice of the output; V_w goes through a
//                            wave-private LDS tile for the transposing reads
// The partial-score exchange is double-buffered: one barrier per 32-key
// tile (a wave writing tile t + 1's scores has passed tile t's barrier, so
// every wave is done reading tile t - 1's from that buffer).
#pragma once

#include "common.hpp"

namespace gqa {

struct WideCfg {
  static constexpr int D = 512;
  static constexpr int NW = 4;             // waves = d slices
  static constexpr int DS = D / NW;        // 128 d per wave
  static constexpr int BK = 32;            // keys per tile
  static constexpr int ROWS = 32;          // query rows per workgroup
  static constexpr int NCK = DS / 16;      // 16-wide d steps of K Q^T per slice
  static constexpr int NDB = DS / 32;      // 32-row d blocks of O^T per slice
  static constexpr int DC = DS / 8;        // 16-byte chunks per slice row
  static constexpr int VPL = BK * DC / 64; // V chunks per lane per tile
  static constexpr int VTILE = BK * DS;    // elements of a wave's V tile
  static constexpr int XF = 64 * 16;       // floats of one wave's partial scores
  static constexpr int LDS_BYTES = NW * VTILE * 2 + 2 * NW * XF * 4;
};

template <bool PAGED, bool PARTIAL>
__global__ void __launch_bounds__(256, 1) attn_wide_kernel(const AttnArgs a) {
  using C = WideCfg;
  constexpr int D = C::D, DS = C::DS, BK = C::BK, NCK = C::NCK, NDB = C::NDB, DC = C::DC;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // d slice
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
  int wlo = kend;  // below wlo no row of the workgroup is masked
  if (a.causal) wlo = min(kend, min(max(n - q_len + row0 / G + 1, 0), n));

  const int rho = row0 + col;
  const bool rvalid = rho < rows_total;
  const int pq = rvalid ? rho / G : 0;
  const int hq = g * G + (rvalid ? rho - pq * G : 0);
  int lim = kend;
  if (a.causal) lim = min(kend, min(max(n - q_len + pq + 1, 0), n));

  // Q operand of this wave's slice: row `col`, d = 128 wv + 16 c + 8 hl + e
  bf16x8 qf[NCK];
  {
    const uint16_t* qp;
    if constexpr (PAGED)
      qp = a.q + (int64_t)(q_row0 + pq) * a.q_ss + (int64_t)hq * a.q_sh;
    else
      qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)pq * a.q_ss;
    qp += DS * wv;
#pragma unroll
    for (int c = 0; c < NCK; ++c)
      qf[c] = rvalid ? *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hl) : bf16x8{};
  }
  float sl2 = -INFINITY;  // sink in log2 units (final mode)
  if constexpr (!PARTIAL)
    if (a.sink && rvalid) sl2 = a.sink[hq] * kLog2e;
  float mref = sl2, mtrue = sl2, l = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  // ---- one tile in registers: this wave's K slice in MFMA operand layout
  // and its V slice as row chunks.  Loaded through buffer resources that end
  // at the tile's last row before kv_len (a 32-key tile never straddles a
  // 64-key page), so later rows read as zeros and are masked.
  struct Tile {
    u32x4 k[NCK];
    u32x4 v[C::VPL];
  };
  const uint32_t kss2 = (uint32_t)(PAGED ? a.kv_sr : a.k_ss) * 2u;
  const uint32_t vss2 = (uint32_t)(PAGED ? a.kv_sr : a.v_ss) * 2u;
  const int krow_a = swap_bits23(col);
  const uint32_t koff = (uint32_t)krow_a * kss2 + 2u * (DS * wv + 8 * hl);
  const uint32_t voff = (uint32_t)(lane / DC) * vss2 + 2u * (DS * wv + 8 * (lane % DC));
  const uint32_t vstep = (uint32_t)(64 / DC) * vss2;
  const uint16_t* khead = a.k + (PAGED ? (int64_t)g * a.k_sh
                                       : (int64_t)b * a.k_sb + (int64_t)g * a.k_sh);
  const uint16_t* vhead = a.v + (PAGED ? (int64_t)g * a.v_sh
                                       : (int64_t)b * a.v_sb + (int64_t)g * a.v_sh);
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)a.page_table;
  // `live` false: the prefetch past the last tile; its resources are empty,
  // so the loads return zeros without touching memory
  auto load = [&](int j0, Tile& t, bool live) {
    int64_t ko, vo;
    if constexpr (PAGED) {
      const int64_t off = (int64_t)ptab[(int64_t)b * a.max_pages + (j0 >> 6)] * a.kv_sp +
                          (int64_t)(j0 & 63) * a.kv_sr;
      ko = vo = off;
    } else {
      ko = (int64_t)j0 * a.k_ss;
      vo = (int64_t)j0 * a.v_ss;
    }
    const uint32_t valid = (uint32_t)min(BK, n - j0);  // >= 1: tiles start below kend <= n
    const BufRes kr = make_bufres(khead + ko, live ? (valid - 1u) * kss2 + (uint32_t)D * 2u : 0u);
    const BufRes vr = make_bufres(vhead + vo, live ? (valid - 1u) * vss2 + (uint32_t)D * 2u : 0u);
#pragma unroll
    for (int c = 0; c < NCK; ++c) t.k[c] = buf_load16v(kr, koff + 32u * c);
#pragma unroll
    for (int j = 0; j < C::VPL; ++j) t.v[j] = buf_load16v(vr, voff + (uint32_t)j * vstep);
  };

  uint16_t* vbuf = smem + wv * C::VTILE;  // wave-private V tile
  float* xbuf = reinterpret_cast<float*>(smem + C::NW * C::VTILE);
  // V^T operand of d block db, keys 16 t .. 16 t + 15 of the tile (two
  // transposing reads; the same slot swizzle as the prefill kernel's V tiles)
  int vbase[2][NDB];
  {
    const int g16 = lane >> 4, r16 = lane & 15;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int cc = 32 * db + 16 * (g16 & 1) + 4 * (r16 & 3);
        const int key = 8 * hl + 4 * half + (r16 >> 2);
        vbase[half][db] = key * DS + 8 * ((cc >> 3) ^ vslot_swz<DC>(key)) + (cc & 7);
      }
  }
  auto vread = [&](int t, int db) {
    i16x4 va[2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
      va[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vbuf + vbase[half][db] + 16 * t * DS));
    return __builtin_bit_cast(bf16x8,
                              __builtin_shufflevector(va[0], va[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- key loop: tile i uses register tile i & 1, the other holds the
  // next tile's loads in flight
  const int kt0 = kbeg;
  Tile tt[2];
  if (ntiles > 0) load(kt0, tt[0], true);
  auto body = [&](int i, Tile& cur, Tile& nxt) __attribute__((always_inline)) {
    const int j0 = kt0 + i * BK;
    load(kt0 + min(i + 1, ntiles - 1) * BK, nxt, i + 1 < ntiles);
    // partial scores over this wave's d slice; register j = key
    // j0 + 16 (j >> 3) + 8 hl + (j & 7) of query row `col`
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NCK; ++c)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cur.k[c]), qf[c], s,
                                                  0, 0, 0);
    // exchange through LDS (lane-major float4 slots), sum in wave order
    float* xb = xbuf + (i & 1) * C::NW * C::XF;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(xb + wv * C::XF + (q4 * 64 + lane) * 4) =
          make_float4(s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]);
    lds_barrier();
    s = f32x16{};
#pragma unroll
    for (int w = 0; w < C::NW; ++w)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = *reinterpret_cast<const float4*>(xb + w * C::XF + (q4 * 64 + lane) * 4);
        s[4 * q4] += x.x;
        s[4 * q4 + 1] += x.y;
        s[4 * q4 + 2] += x.z;
        s[4 * q4 + 3] += x.w;
      }
    // mask (keys at or past the row's limit), then the online softmax
    if (j0 + BK > wlo) {
      const int rem = lim - j0 - 8 * hl;
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (16 * (j >> 3) + (j & 7) >= rem) s[j] = -INFINITY;
    }
    float m = s[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) m = __builtin_elementwise_maximum(m, s[j]);
    {
      const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m),
                                                      false, false);
      m = __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    const float mx = m * a.scale_log2;
    mtrue = fmaxf(mtrue, mx);
    const bool move = mx > mref + 8.f;  // lazy reference (log2 units)
    const float alpha = move ? ex2(mref - mx) : 1.f;  // 0 when mref = -inf
    mref = move ? mx : mref;
    const float mu = (mref == -INFINITY) ? 0.f : mref;
    float ls = 0.f;
    bf16x8 pb[2];
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
    if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    // V slice -> the wave's LDS tile (row-major, swizzled 16-byte slots)
#pragma unroll
    for (int j = 0; j < C::VPL; ++j) {
      const int ci = lane + 64 * j;
      const int kl = ci / DC;
      *reinterpret_cast<u32x4*>(vbuf + kl * DS + 8 * ((ci % DC) ^ vslot_swz<DC>(kl))) = cur.v[j];
    }
    // O^T += V^T P^T over the tile's two 16-key steps
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vread(t, db), pb[t], acc[db], 0, 0, 0);
  };
  for (int i = 0; i < ntiles; i += 2) {
    body(i, tt[0], tt[1]);
    if (i + 1 < ntiles) body(i + 1, tt[1], tt[0]);
  }

  // ---- epilogue; accumulator register j of d block db holds
  //      d = 128 wv + 32 db + 8 (j >> 2) + 4 hl + (j & 3) of query row `col`
  float lt = l;
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(lt), __float_as_uint(lt), false,
                                                    false);
    lt = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if constexpr (PARTIAL) {
    const float f = (mtrue == -INFINITY) ? 0.f : ex2(mref - mtrue);
    lt *= f;
    if (!rvalid) return;
    int64_t row;
    if constexpr (PAGED)
      row = (int64_t)hq * a.total_q + q_row0 + pq;
    else
      row = ((int64_t)b * a.Hq + hq) * a.Sq + pq;
    const int64_t idx = row * a.n_split + split;
    if (wv == 0 && hl == 0)
      a.ws_ml[idx] = make_float2(mtrue == -INFINITY ? -INFINITY : mtrue * kLn2, lt);
    if (a.skip_empty_o && mtrue == -INFINITY) return;
    float* op = a.ws_o + idx * D + DS * wv;
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
    op += DS * wv;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<uint2*>(op + 32 * db + 8 * q4 + 4 * hl) =
            make_uint2(pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                       pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv));
  }
}

// ---- Wide heads over many query rows (d = 512, more than 32 rows per
// (b, kv head): prefill).  Splitting d across the waves, as above, sums
// four partial score blocks through LDS behind a barrier for every 32 keys
// (16 MFMAs per wave); here each wave instead owns 16 query rows over the
// whole head dim, and the eight waves of a workgroup (two per SIMD) share
// every K/V tile.  v_mfma_f32_16x16x32_bf16, the stream kernel's mapping
// (a lane holds one query column c16 and a quarter of the keys):
//   S^T = K Q^T     32 MFMAs per 32-key tile (two 16-key blocks x 16 d
//                   steps); K from LDS, Q in 64 registers
//   softmax         8 scores per lane, the row's four lanes combined by
//                   cross-lane max
//   O^T += V^T P^T  32 MFMAs, one per 16-d block (128 accumulators per
//                   lane), P straight from the S accumulators, V^T by
//                   transposing LDS reads
// so a tile carries 64 MFMAs per wave against some 50 vector instructions,
// and the two waves of a SIMD overlap one's softmax with the other's MFMAs.
// (32 rows per wave would need 256 accumulators per lane, the whole
// accumulator file, and spill.)  The tiles go to two LDS stages by LDS DMA
// (a 1 KiB block per 512-element row: 64 lanes x 16 bytes), requested one
// tile ahead; the barrier that ends a tile also waits for the next one's
// blocks.  K rows are padded by 32 bytes: with 16 bytes the operand reads
// (16 lanes over 16 rows) still met bank conflicts on a fifth of the
// kernel's cycles (LDS bank-conflict counter; none with 32).  V rows hold
// chunk p ^ vslot_swz(row) in slot p, for the transposing reads.  The stages are
// separate static arrays, so the compiler does not wait for the DMA into
// one before reading the other.
struct WideRowsCfg {
  static constexpr int D = 512;
  static constexpr int NW = 8;
  static constexpr int BK = 32;          // keys per tile
  static constexpr int ROWS = 16 * NW;   // query rows per workgroup
  static constexpr int NC = D / 32;      // 32-wide d steps of K Q^T
  static constexpr int NDB = D / 16;     // 16-row d blocks of O^T
  static constexpr int DC = D / 8;       // 16-byte chunks per row (one DMA block)
  static constexpr int KP = D + 16;      // K row pitch (elements)
  static constexpr int KTILE = BK * KP;
  static constexpr int VTILE = BK * D;
  static_assert(DC == 64, "one 64-lane DMA block per row");
};

template <bool PAGED, bool PARTIAL>
__global__ void __launch_bounds__(512, 1) attn_wide_rows_kernel(const AttnArgs a) {
  using C = WideRowsCfg;
  constexpr int D = C::D, BK = C::BK, NC = C::NC, NDB = C::NDB, DC = C::DC, KP = C::KP;
  constexpr int CP = kCpDefault;  // q-tiles of a (b, kv head) share its tiles through the L2
  __shared__ __attribute__((aligned(16))) uint16_t xk0[C::KTILE], xk1[C::KTILE];
  __shared__ __attribute__((aligned(16))) uint16_t xv0[C::VTILE], xv1[C::VTILE];
  using LdsPtr = __attribute__((address_space(3))) void*;

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;
  const int grp = lane >> 4;

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
  if (row0 >= rows_total) return;  // the whole workgroup: no barrier is skipped

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

  // this wave's 16 rows (column c16); below wlo none of them is masked
  const int wrow0 = row0 + 16 * wv;
  int wlo = kend;
  if (a.causal) wlo = min(kend, min(max(n - q_len + wrow0 / G + 1, 0), n));
  const int rho = wrow0 + c16;
  const bool rvalid = rho < rows_total;
  const int pq = rvalid ? rho / G : 0;
  const int hq = g * G + (rvalid ? rho - pq * G : 0);
  int lim = kend;
  if (a.causal) lim = min(kend, min(max(n - q_len + pq + 1, 0), n));

  // Q operand (B of K Q^T): column c16, d = 32 c + 8 grp + e
  bf16x8 qf[NC];
  {
    const uint16_t* qp;
    if constexpr (PAGED)
      qp = a.q + (int64_t)(q_row0 + pq) * a.q_ss + (int64_t)hq * a.q_sh;
    else
      qp = a.q + (int64_t)b * a.q_sb + (int64_t)hq * a.q_sh + (int64_t)pq * a.q_ss;
#pragma unroll
    for (int c = 0; c < NC; ++c)
      qf[c] = rvalid ? *reinterpret_cast<const bf16x8*>(qp + 32 * c + 8 * grp) : bf16x8{};
  }
  float sl2 = -INFINITY;  // sink in log2 units (final mode)
  if constexpr (!PARTIAL)
    if (a.sink && rvalid) sl2 = a.sink[hq] * kLog2e;
  float mref = sl2, mtrue = sl2, l = 0.f;  // l: this lane's keys only
  f32x4 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x4{};

  // ---- tile resources: rows past kv_len lie outside them and read as zeros
  const uint32_t kss2 = (uint32_t)(PAGED ? a.kv_sr : a.k_ss) * 2u;
  const uint32_t vss2 = (uint32_t)(PAGED ? a.kv_sr : a.v_ss) * 2u;
  const uint16_t* khead = a.k + (PAGED ? (int64_t)g * a.k_sh
                                       : (int64_t)b * a.k_sb + (int64_t)g * a.k_sh);
  const uint16_t* vhead = a.v + (PAGED ? (int64_t)g * a.v_sh
                                       : (int64_t)b * a.v_sb + (int64_t)g * a.v_sh);
  const __attribute__((address_space(4))) int32_t* ptab =
      (const __attribute__((address_space(4))) int32_t*)a.page_table;
  // DMA of the tile at key j0 (`live` false: past the last tile, empty
  // resources, nothing read) into stage (ks, vs); wave w takes rows w, w + 8, ...
  auto dma = [&](int j0, bool live, uint16_t* ks, uint16_t* vs) __attribute__((always_inline)) {
    int64_t ko, vo;
    if constexpr (PAGED) {
      const int64_t off = (int64_t)ptab[(int64_t)b * a.max_pages + (j0 >> 6)] * a.kv_sp +
                          (int64_t)(j0 & 63) * a.kv_sr;
      ko = vo = off;
    } else {
      ko = (int64_t)j0 * a.k_ss;
      vo = (int64_t)j0 * a.v_ss;
    }
    const uint32_t valid = (uint32_t)min(BK, n - j0);  // >= 1: tiles start below kend <= n
    // non-const resources: a const one makes the host pass drop the kernel
    BufRes kr = make_bufres(khead + ko, live ? (valid - 1u) * kss2 + (uint32_t)D * 2u : 0u);
    BufRes vr = make_bufres(vhead + vo, live ? (valid - 1u) * vss2 + (uint32_t)D * 2u : 0u);
    for (int i = wv; i < BK; i += C::NW) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (LdsPtr)(ks + KP * i), 16,
                                               (int)((uint32_t)i * kss2 + 16u * (uint32_t)lane),
                                               0, 0, CP);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vr, (LdsPtr)(vs + D * i), 16,
          (int)((uint32_t)i * vss2 + 16u * (uint32_t)(lane ^ vslot_swz<DC>(i))), 0, 0, CP);
    }
  };

  // K operand (A of K Q^T) of key block kb, d step c: key row 16 kb + c16,
  // d = 32 c + 8 grp + e
  const int kro = c16 * KP + 8 * grp;
  // V^T operand of d block db: keys 4 grp .. + 3 and 16 + 4 grp .. + 3 (the
  // order of P's registers), by two transposing reads whose source lane c16
  // points at key row 4 grp + c16 / 4 (+ 16) and d = 16 db + 4 (c16 & 3).
  // The swizzle repeats every 8 d blocks (16 slots): 8 per-lane bases.
  int vro[8];
  {
    const int kl = 4 * grp + (c16 >> 2);
    const int sw = vslot_swz<DC>(kl);
#pragma unroll
    for (int dl = 0; dl < 8; ++dl)
      vro[dl] = kl * D + 8 * ((2 * dl + ((c16 & 3) >> 1)) ^ sw) + 4 * (c16 & 1);
  }

  // one tile on stage (Ks, Vs) at key j0, the next one's DMA into (kn, vn)
  auto body = [&](int i, const uint16_t* Ks, const uint16_t* Vs, uint16_t* kn, uint16_t* vn)
      __attribute__((always_inline)) {
    const int j0 = kbeg + i * BK;
    dma(kbeg + min(i + 1, ntiles - 1) * BK, i + 1 < ntiles, kn, vn);
    // One MFMA per step, its operand read PD steps ahead, in a fixed order
    constexpr int PD = 3;
    // step g of K Q^T: key block g & 1, d step g >> 1 (the two blocks'
    // accumulations alternate, so consecutive MFMAs do not wait on each other)
    auto kread = [&](int g) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8*>(Ks + kro + 16 * (g & 1) * KP + 32 * (g >> 1));
    };
    auto vread = [&](int db) __attribute__((always_inline)) {
      i16x4 va[2];
#pragma unroll
      for (int half = 0; half < 2; ++half)
        va[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(Vs + vro[db % 8] + 128 * (db / 8) +
                                                       16 * half * D));
      return __builtin_bit_cast(bf16x8,
                                __builtin_shufflevector(va[0], va[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // register r of block kb = key j0 + 16 kb + 4 grp + r of column c16
    f32x4 s[2] = {f32x4{}, f32x4{}};
    bf16x8 ob[PD + 1];
#pragma unroll
    for (int gg = 0; gg < PD; ++gg) ob[gg] = kread(gg);
    __builtin_amdgcn_sched_barrier(0);
    auto qk_step = [&](auto gc) __attribute__((always_inline)) {
      constexpr int gs = decltype(gc)::value;
      s[gs & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ob[gs % (PD + 1)], qf[gs >> 1],
                                                         s[gs & 1], 0, 0, 0);
      if constexpr (gs + PD < 2 * NC) ob[(gs + PD) % (PD + 1)] = kread(gs + PD);
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<2 * NC>(qk_step);
    // the first V operands, read during the softmax
#pragma unroll
    for (int gg = 0; gg < PD; ++gg) ob[gg] = vread(gg);
    if (j0 + BK > wlo) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j0 + 16 * kb + 4 * grp + r >= lim) s[kb][r] = -INFINITY;
    }
    float m = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[0][0], s[0][1]),
                                      __builtin_elementwise_maximum(s[0][2], s[0][3])),
        __builtin_elementwise_maximum(__builtin_elementwise_maximum(s[1][0], s[1][1]),
                                      __builtin_elementwise_maximum(s[1][2], s[1][3])));
    m = __builtin_elementwise_maximum(m, __shfl_xor(m, 16, 64));
    m = __builtin_elementwise_maximum(m, __shfl_xor(m, 32, 64));
    const float mx = m * a.scale_log2;
    mtrue = fmaxf(mtrue, mx);
    const bool move = mx > mref + 8.f;  // lazy reference (log2 units)
    const float alpha = move ? ex2(mref - mx) : 1.f;  // 0 when mref = -inf
    mref = move ? mx : mref;
    const float mu = (mref == -INFINITY) ? 0.f : mref;
    float ls = 0.f;
    u32x4 w;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const f32x2 x = {ex2(__builtin_fmaf(s[kb][2 * e], a.scale_log2, -mu)),
                         ex2(__builtin_fmaf(s[kb][2 * e + 1], a.scale_log2, -mu))};
        const bf16x2 pp = __builtin_convertvector(x, bf16x2);
        ls = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, ls, false);
        w[2 * kb + e] = __builtin_bit_cast(uint32_t, pp);
      }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, w);
    l = l * alpha + ls;
    if (__builtin_expect(__any(alpha != 1.f), 0)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    __builtin_amdgcn_sched_barrier(0);
    auto pv_step = [&](auto gc) __attribute__((always_inline)) {
      constexpr int db = decltype(gc)::value;
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ob[db % (PD + 1)], pb, acc[db], 0, 0, 0);
      if constexpr (db + PD < NDB) ob[(db + PD) % (PD + 1)] = vread(db + PD);
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<NDB>(pv_step);
    lds_barrier();  // every wave is done with this stage; also waits for this wave's DMA
  };
  if (ntiles > 0) {
    dma(kbeg, true, xk0, xv0);
    lds_barrier();
  }
  int i = 0;
  for (; i + 1 < ntiles; i += 2) {
    body(i, xk0, xv0, xk1, xv1);
    body(i + 1, xk1, xv1, xk0, xv0);
  }
  if (i < ntiles) body(i, xk0, xv0, xk1, xv1);

  // ---- epilogue; acc[db][e] holds d = 16 db + 4 grp + e of column c16
  float lt = l;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if constexpr (PARTIAL) {
    const float f = (mtrue == -INFINITY) ? 0.f : ex2(mref - mtrue);
    lt *= f;
    if (!rvalid) return;
    int64_t row;
    if constexpr (PAGED)
      row = (int64_t)hq * a.total_q + q_row0 + pq;
    else
      row = ((int64_t)b * a.Hq + hq) * a.Sq + pq;
    const int64_t idx = row * a.n_split + split;
    if (grp == 0) a.ws_ml[idx] = make_float2(mtrue == -INFINITY ? -INFINITY : mtrue * kLn2, lt);
    if (a.skip_empty_o && mtrue == -INFINITY) return;
    float* op = a.ws_o + idx * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<float4*>(op + 16 * db) =
          make_float4(acc[db][0] * f, acc[db][1] * f, acc[db][2] * f, acc[db][3] * f);
  } else {
    if (sl2 != -INFINITY) lt += ex2(sl2 - mref);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (!rvalid) return;
    uint16_t* op;
    if constexpr (PAGED)
      op = a.o + (int64_t)(q_row0 + pq) * a.o_ss + (int64_t)hq * a.o_sh;
    else
      op = a.o + (int64_t)b * a.o_sb + (int64_t)hq * a.o_sh + (int64_t)pq * a.o_ss;
    op += 4 * grp;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<uint2*>(op + 16 * db) =
          make_uint2(pack_bf16x2(acc[db][0] * inv, acc[db][1] * inv),
                     pack_bf16x2(acc[db][2] * inv, acc[db][3] * inv));
  }
}

}  // namespace gqa
