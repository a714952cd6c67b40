// Split-KV merge kernel.
#pragma once

#include "common.hpp"

namespace gqa {

// Split-KV merge (kernbench2 benches commit log: the (m, l, O) state and its
// associative merge; nvfp4-megamoe-kernel commit log: normalise once).
// Each query row takes LPR lanes of a wave, E = D / LPR output elements per
// lane: RPW = 64 / LPR rows per wave.  The packed forms (E = 4, 16-byte
// loads: 8 rows per wave at d = 32, 4 at 64, 2 at 128) carry many rows; at
// d = 128 a small merge (decode: one row per (b, head)) keeps one row per
// wave (E = 2), twice the waves to hide the load latency with.
// SPARSE: a state's O~ is read only when its m is finite (where many splits
// are empty: causal or ragged rows over large groups); otherwise all loads
// of a round issue together.
template <int D, int LPR>
struct MergeCfg {
  static_assert(LPR <= 64 && D % LPR == 0 && (D / LPR == 2 || D / LPR % 4 == 0), "lanes per row");
  static constexpr int E = D / LPR;
  static constexpr int RPW = 64 / LPR;
  static constexpr int ROWS_PER_BLOCK = 4 * RPW;  // 256-thread workgroups
};
// the packed lane count per row (16-byte loads)
template <int D>
constexpr int kMergePackedLpr = D >= 256 ? 64 : D / 4;

template <int D, bool SPARSE, int LPR>
__global__ void __launch_bounds__(256)
merge_kernel(const float2* __restrict__ ml, const float* __restrict__ ot, uint16_t* o,
             int64_t o_sb, int64_t o_sh, int64_t o_ss, const float* sink, int Hq, int Sq,
             int n_split, int64_t rows) {
  using C = MergeCfg<D, LPR>;
  constexpr int E = C::E;
  constexpr int CH = 8;  // partial states loaded per round
  const int lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * C::RPW + lane / LPR;
  const int ln = lane % LPR;
  if (row >= rows) return;
  const float2* mlr = ml + row * n_split;
  const float* otr = ot + row * n_split * D + ln * E;
  // this lane's E elements of split s's O~ (zeros when !live)
  auto load_o = [&](int s, bool live, float (&v)[E]) {
    if constexpr (E == 2) {
      float2 x = make_float2(0.f, 0.f);
      if (live) x = *reinterpret_cast<const float2*>(otr + (int64_t)s * D);
      v[0] = x.x; v[1] = x.y;
    } else {
#pragma unroll
      for (int e = 0; e < E; e += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (live) x = *reinterpret_cast<const float4*>(otr + (int64_t)s * D + e);
        v[e] = x.x; v[e + 1] = x.y; v[e + 2] = x.z; v[e + 3] = x.w;
      }
    }
  };
  const int i = (int)(row % Sq);
  const int h = (int)((row / Sq) % Hq);
  const int64_t b = row / ((int64_t)Sq * Hq);

  // running merge over chunks of CH splits; the sink is the initial state
  // (m = sink, l = 1, O~ = 0), or the identity (-inf, 0, 0) without one
  const float sk = sink ? sink[h] : -INFINITY;
  float M = sk;
  float Lsum = (sk == -INFINITY) ? 0.f : 1.f;
  float accv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) accv[e] = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += CH) {
    float2 st[CH];
    float ov[CH][E];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      // past the last split: the identity state, and no loads (the test is
      // wave-uniform, so the loads of a round still issue together)
      const bool in = s0 + j < n_split;
      st[j] = in ? mlr[s0 + j] : make_float2(-INFINITY, 0.f);
      if constexpr (!SPARSE) load_o(s0 + j, in, ov[j]);
    }
    if constexpr (SPARSE) {
#pragma unroll
      for (int j = 0; j < CH; ++j)  // live is uniform over the row's lanes
        load_o(s0 + j, s0 + j < n_split && st[j].x != -INFINITY, ov[j]);
    }
    float mc = M;
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (s0 + j < n_split) mc = fmaxf(mc, st[j].x);
    if (mc == -INFINITY) continue;  // nothing visible so far
    const float r = (M == -INFINITY) ? 0.f : __expf(M - mc);
    Lsum *= r;
#pragma unroll
    for (int e = 0; e < E; ++e) accv[e] *= r;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      if (s0 + j >= n_split || st[j].x == -INFINITY) continue;
      const float w = __expf(st[j].x - mc);
      Lsum += st[j].y * w;
#pragma unroll
      for (int e = 0; e < E; ++e) accv[e] += w * ov[j][e];
    }
    M = mc;
  }
  float out[E];
  const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) out[e] = (M == -INFINITY) ? 0.f : accv[e] * inv;
  uint16_t* op = o + b * o_sb + (int64_t)h * o_sh + (int64_t)i * o_ss + ln * E;
  if constexpr (E == 8) {
    *reinterpret_cast<uint4*>(op) =
        make_uint4(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]),
                   pack_bf16x2(out[4], out[5]), pack_bf16x2(out[6], out[7]));
  } else if constexpr (E == 4) {
    *reinterpret_cast<uint2*>(op) =
        make_uint2(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]));
  } else {
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(out[0], out[1]);
  }
}

}  // namespace gqa
