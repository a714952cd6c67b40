// Split-KV merge kernel.
#pragma once

#include "common.hpp"

namespace gqa {

// Split-KV merge (kernbench2 benches commit log: the (m, l, O) state and its
// associative merge; nvfp4-megamoe-kernel commit log: normalise once).
// One 64-lane wave per query row; D / 64 output elements per lane (one per
// lane of the first 32 at d = 32).  SPARSE: a state's O~ is read only when
// its m is finite (where many splits are empty: causal or ragged rows over
// large groups); otherwise all loads of a round issue together.
template <int D, bool SPARSE>
__global__ void __launch_bounds__(256)
merge_kernel(const float2* __restrict__ ml, const float* __restrict__ ot, uint16_t* o,
             int64_t o_sb, int64_t o_sh, int64_t o_ss, const float* sink, int Hq, int Sq,
             int n_split, int64_t rows) {
  constexpr int E = D >= 64 ? D / 64 : 1;
  constexpr int CH = 8;  // partial states loaded per round
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows || lane * E >= D) return;
  const int i = (int)(row % Sq);
  const int h = (int)((row / Sq) % Hq);
  const int64_t b = row / ((int64_t)Sq * Hq);
  const float2* mlr = ml + row * n_split;
  const float* otr = ot + row * n_split * D + lane * E;

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
      const int s = min(s0 + j, n_split - 1);  // branch-free: duplicates are dropped below
      st[j] = mlr[s];
      if constexpr (!SPARSE) {
#pragma unroll
        for (int e = 0; e < E; ++e) ov[j][e] = otr[(int64_t)s * D + e];
      }
    }
    if constexpr (SPARSE) {
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const bool live = s0 + j < n_split && st[j].x != -INFINITY;  // wave-uniform
#pragma unroll
        for (int e = 0; e < E; ++e) ov[j][e] = live ? otr[(int64_t)(s0 + j) * D + e] : 0.f;
      }
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
  uint16_t* op = o + b * o_sb + (int64_t)h * o_sh + (int64_t)i * o_ss + lane * E;
  if constexpr (E == 8) {
    *reinterpret_cast<uint4*>(op) =
        make_uint4(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]),
                   pack_bf16x2(out[4], out[5]), pack_bf16x2(out[6], out[7]));
  } else if constexpr (E == 4) {
    *reinterpret_cast<uint2*>(op) =
        make_uint2(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]));
  } else if constexpr (E == 2) {
    *reinterpret_cast<uint32_t*>(op) = pack_bf16x2(out[0], out[1]);
  } else {
    *reinterpret_cast<__bf16*>(op) = (__bf16)out[0];
  }
}

}  // namespace gqa
