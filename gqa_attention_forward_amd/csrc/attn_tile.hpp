// Workgroup-tiled GQA forward kernel: the K/V tile is shared through LDS by
// all waves of the workgroup (prefill shapes).  See common.hpp for the math.
#pragma once

#include "common.hpp"

namespace gqa {

// NR row groups of 32 query rows x NK key groups of BKW keys: NR * NK waves.
// Each iteration stages TK = NK * BKW keys of K and V in LDS; wave (rg, kg)
// works on rows [32 rg, 32 rg + 32) and keys [kg BKW, (kg + 1) BKW) of it.
template <int D, int NR, int NK, int BKW>
struct Cfg {
  static constexpr int NW = NR * NK;
  static constexpr int NT = NW * 64;
  static constexpr int TK = NK * BKW;
  static constexpr int KP = D + 8;           // K row pitch in LDS (elements)
  static constexpr int VP = TK + 8;          // Vt row pitch in LDS (elements)
  static constexpr int KSZ = TK * KP;        // elements per K stage
  static constexpr int VSZ = D * VP;         // elements per Vt stage
  static constexpr int STAGE = KSZ + VSZ;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int KCH = TK * D / 8;     // 16-byte K chunks per tile
  static constexpr int KPT = (KCH + NT - 1) / NT;
  static constexpr int VQ = (TK / 4) * (D / 8);   // (4-key quad, 8-d chunk) V pieces
  static constexpr int VPT = (VQ + NT - 1) / NT;
  static constexpr int RED_BYTES = (NK - 1) * NR * 64 * (D / 2 + 2) * 4;
  static_assert(BKW % 32 == 0 && TK >= 64, "key tiling");
  static_assert(D % 32 == 0, "head dim");
  static_assert(RED_BYTES <= LDS_BYTES, "combine buffer");
};

template <int D, int NR, int NK, int BKW, bool PAGED, bool PARTIAL>
__global__ void __launch_bounds__(NR * NK * 64)
attn_fwd_kernel(const AttnArgs a) {
  using C = Cfg<D, NR, NK, BKW>;
  constexpr int NT = C::NT;
  constexpr int TK = C::TK;
  constexpr int KP = C::KP;
  constexpr int VP = C::VP;
  constexpr int DC = D / 8;  // 16-byte chunks per row
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int rg = wv % NR;
  const int kg = wv / NR;
  const int col = lane & 31;
  const int hl = lane >> 5;

  // ---- which (b, g, split, q-tile) this workgroup owns; late q-tiles first
  const int L = blockIdx.x;
  const int nbg = a.B * a.Hkv;
  const int bg = L % nbg;
  const int rest = L / nbg;
  const int split = rest % a.n_split;
  const int qt = a.n_qtiles - 1 - rest / a.n_split;
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
  const int row0 = qt * (NR * 32);
  if (row0 >= rows_total) return;  // uniform: ragged q-tile past this sequence

  // key range of this workgroup
  int kbeg = 0, kend = n;
  if (a.tile > 0) {
    kbeg = split * a.tile;
    kend = min(n, kbeg + a.tile);
  }
  if (a.causal) {
    const int p_last = (min(row0 + NR * 32, rows_total) - 1) / G;
    kend = min(kend, min(max(n - q_len + p_last + 1, 0), n));
  }
  const int ntiles = kend > kbeg ? (kend - kbeg + TK - 1) / TK : 0;

  // ---- this lane's query row
  const int rho = row0 + rg * 32 + col;
  const bool rvalid = rho < rows_total;
  const int p = rvalid ? rho / G : 0;
  const int hh = rvalid ? rho - p * G : 0;
  const int h = g * G + hh;
  int lim = kend;  // keys >= lim are masked for this row
  if (a.causal) lim = min(lim, min(max(n - q_len + p + 1, 0), n));
  // wave-uniform bounds: below wlo no row of the wave is masked, at or past
  // whi every row is
  const int wrow0 = row0 + rg * 32;
  const int wrow1 = min(wrow0 + 32, rows_total) - 1;
  int wlo = kend, whi = kend;
  if (a.causal) {
    wlo = min(kend, min(max(n - q_len + wrow0 / G + 1, 0), n));
    whi = min(kend, min(max(n - q_len + wrow1 / G + 1, 0), n));
  }
  if (wrow0 >= rows_total) { wlo = kbeg; whi = kbeg; }

  // ---- Q operand (B of S^T = K Q^T): lane holds row `col`, d = 16c + 8hl + e
  bf16x8 qf[D / 16];
  {
    const uint16_t* qp;
    if constexpr (PAGED)
      qp = a.q + (int64_t)(q_row0 + p) * a.q_ss + (int64_t)h * a.q_sh;
    else
      qp = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh + (int64_t)p * a.q_ss;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      if (rvalid)
        qf[c] = *reinterpret_cast<const bf16x8*>(qp + 16 * c + 8 * hl);
      else
        qf[c] = bf16x8{};
    }
  }

  float sl2 = -INFINITY;  // sink, log2 units (final mode only)
  if constexpr (!PARTIAL) {
    if (a.sink && rvalid) sl2 = a.sink[h] * kLog2e;
  }
  float m = sl2;    // running max (log2 units); the sink takes part in it
  float l = 0.f;    // this lane's share of the running sum (sink added at the end)
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};

  // ---- global -> register staging of one TK-key tile of K and V
  uint4 kr[C::KPT];
  uint4 vr[C::VPT][4];

  auto row_ptr = [&](const uint16_t* base, int64_t sb, int64_t sh, int64_t ss,
                     int key) -> const uint16_t* {
    if constexpr (PAGED) {
      const int pg = a.page_table[(int64_t)b * a.max_pages + (key >> 6)];
      return base + (int64_t)pg * a.kv_sp + (int64_t)(key & 63) * a.kv_sr + (int64_t)g * sh;
    } else {
      return base + (int64_t)b * sb + (int64_t)g * sh + (int64_t)key * ss;
    }
  };

  // Keys at or past kend are never read: their loads go to row kend - 1
  // (real, finite data) and the keys are masked, so they get P = 0 exactly.
  // Branch-free loads keep the compiler's wait counts exact.
  const int klast = kend - 1;
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int ci = tid + i * NT;
      kr[i] = make_uint4(0, 0, 0, 0);
      if (C::KCH % NT == 0 || ci < C::KCH) {
        const int key = min(j0 + ci / DC, klast);
        kr[i] = *reinterpret_cast<const uint4*>(
            row_ptr(a.k, a.k_sb, a.k_sh, a.k_ss, key) + (ci % DC) * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int pi = tid + i * NT;
#pragma unroll
      for (int r = 0; r < 4; ++r) vr[i][r] = make_uint4(0, 0, 0, 0);
      if (C::VQ % NT == 0 || pi < C::VQ) {
        const int quad = pi / DC;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = min(j0 + 4 * quad + r, klast);
          vr[i][r] = *reinterpret_cast<const uint4*>(
              row_ptr(a.v, a.v_sb, a.v_sh, a.v_ss, key) + (pi % DC) * 8);
        }
      }
    }
  };

  // register -> LDS; V is transposed on the way (4 keys x 8 d per thread)
  auto store_tile = [&](int stage) {
    uint16_t* Ks = smem + stage * C::STAGE;
    uint16_t* Vs = Ks + C::KSZ;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int ci = tid + i * NT;
      if (C::KCH % NT == 0 || ci < C::KCH)
        *reinterpret_cast<uint4*>(Ks + (ci / DC) * KP + (ci % DC) * 8) = kr[i];
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int pi = tid + i * NT;
      if (C::VQ % NT == 0 || pi < C::VQ) {
        const int quad = pi / DC;
        const int d0 = (pi % DC) * 8;
        const uint32_t* k0 = reinterpret_cast<const uint32_t*>(&vr[i][0]);
        const uint32_t* k1 = reinterpret_cast<const uint32_t*>(&vr[i][1]);
        const uint32_t* k2 = reinterpret_cast<const uint32_t*>(&vr[i][2]);
        const uint32_t* k3 = reinterpret_cast<const uint32_t*>(&vr[i][3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo01 = __builtin_amdgcn_perm(k1[e], k0[e], 0x05040100u);
          const uint32_t hi01 = __builtin_amdgcn_perm(k1[e], k0[e], 0x07060302u);
          const uint32_t lo23 = __builtin_amdgcn_perm(k3[e], k2[e], 0x05040100u);
          const uint32_t hi23 = __builtin_amdgcn_perm(k3[e], k2[e], 0x07060302u);
          const int dA = d0 + 2 * e;
          const int dB = dA + 1;
          const int qA = quad ^ (4 * ((dA >> 4) & 3));
          const int qB = quad ^ (4 * ((dB >> 4) & 3));
          *reinterpret_cast<uint2*>(Vs + dA * VP + 4 * qA) = make_uint2(lo01, lo23);
          *reinterpret_cast<uint2*>(Vs + dB * VP + 4 * qB) = make_uint2(hi01, hi23);
        }
      }
    }
  };

  if (ntiles > 0) {
    load_tile(kbeg);
    store_tile(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int j0 = kbeg + it * TK;
    const bool more = it + 1 < ntiles;
    if (more) load_tile(j0 + TK);

    const int jw0 = j0 + kg * BKW;  // first key of this wave's sub-tile
    if (jw0 < whi) {
      const uint16_t* Ks = smem + (it & 1) * C::STAGE + kg * BKW * KP;
      const uint16_t* Vs = smem + (it & 1) * C::STAGE + C::KSZ;

      // S^T = K Q^T over this wave's BKW keys
      f32x16 s[BKW / 32];
#pragma unroll
      for (int mb = 0; mb < BKW / 32; ++mb) {
        s[mb] = f32x16{};
        const uint16_t* kp = Ks + (32 * mb + swap_bits23(col)) * KP + 8 * hl;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8 kk = *reinterpret_cast<const bf16x8*>(kp + 16 * c);
          s[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qf[c], s[mb], 0, 0, 0);
        }
      }
      // register j of block mb holds key jw0 + 32 mb + 16 (j >> 3) + 8 hl + (j & 7)
      if (jw0 + BKW > wlo) {
#pragma unroll
        for (int mb = 0; mb < BKW / 32; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = jw0 + 32 * mb + 16 * (j >> 3) + 8 * hl + (j & 7);
            if (key >= lim) s[mb][j] = -INFINITY;
          }
      }
      // online softmax, base 2
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < BKW / 32; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[mb][j]);
      mx = xor32_max(mx);
      const float m_new = fmaxf(m, mx * a.scale_log2);
      const float mu = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = ex2(m - mu);
      float ls = 0.f;
#pragma unroll
      for (int mb = 0; mb < BKW / 32; ++mb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pj = ex2(__builtin_fmaf(s[mb][j], a.scale_log2, -mu));
          s[mb][j] = pj;
          ls += pj;
        }
      l = l * alpha + ls;
      m = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[db][j] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int t = 0; t < BKW / 16; ++t) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[t >> 1][8 * (t & 1) + e];
        const int oct = (kg * BKW) / 8 + 2 * t + hl;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int d = 32 * db + col;
          const int po = oct ^ (2 * ((d >> 4) & 3));
          const bf16x8 vv = *reinterpret_cast<const bf16x8*>(Vs + d * VP + 8 * po);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb, acc[db], 0, 0, 0);
        }
      }
    }

    if (more) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // ---- combine the NK key groups of each row group (through LDS)
  if constexpr (NK > 1) {
    float* red = reinterpret_cast<float*>(smem);
    constexpr int SLOT = 64 * (D / 2 + 2);
    if (kg > 0) {
      float* r = red + ((kg - 1) * NR + rg) * SLOT;
      r[lane] = m;
      r[64 + lane] = l;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) r[(2 + db * 16 + j) * 64 + lane] = acc[db][j];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int k2 = 1; k2 < NK; ++k2) {
        const float* r = red + ((k2 - 1) * NR + rg) * SLOT;
        const float m2 = r[lane];
        const float l2 = r[64 + lane];
        const float mn = fmaxf(m, m2);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float wa = ex2(m - mu);
        const float wb = ex2(m2 - mu);
        l = l * wa + l2 * wb;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j)
            acc[db][j] = acc[db][j] * wa + r[(2 + db * 16 + j) * 64 + lane] * wb;
        m = mn;
      }
    }
  }
  if (kg != 0) return;

  // ---- epilogue; accumulator register j of d-block db holds
  //      d = 32 db + 8 (j >> 2) + 4 hl + (j & 3) of query row `col`
  float lt = xor32_sum(l);
  if constexpr (PARTIAL) {
    if (!rvalid) return;
    const int64_t row = ((int64_t)b * a.Hq + h) * a.Sq + p;
    const int64_t idx = row * a.n_split + split;
    if (hl == 0) a.ws_ml[idx] = make_float2(m == -INFINITY ? -INFINITY : m * kLn2, lt);
    float* op = a.ws_o + idx * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(op + 32 * db + 8 * q4 + 4 * hl) =
            make_float4(acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                        acc[db][4 * q4 + 3]);
  } else {
    if (sl2 != -INFINITY) lt += ex2(sl2 - m);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (!rvalid) return;
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
            make_uint2(pack_bf16x2(acc[db][4 * q4] * inv, acc[db][4 * q4 + 1] * inv),
                       pack_bf16x2(acc[db][4 * q4 + 2] * inv, acc[db][4 * q4 + 3] * inv));
  }
}

}  // namespace gqa
