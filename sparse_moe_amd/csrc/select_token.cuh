// Per-token score and top-K selection (used by the select kernel).
//
// Sigmoid mode (hy3 README "Model facts", MoE routing row; HYV3Config
// moe_router_use_sigmoid / route_norm / router_scaling_factor):
//   s = sigmoid(logit);  pick the K largest of s + expert_bias;
//   w_j = scale * s[pick_j] / sum_j' s[pick_j'].
// Softmax mode (HunyuanImage 3.0 MoE reading, easy_topk):
//   p = softmax(logits);  pick the K largest p;
//   w_j = p[pick_j] / max(sum_j' p[pick_j'], renorm_eps).
//
// The router's float64 K-slice partial sums are added in slice order and
// the scores are evaluated in float64, so the selection is decided on
// fp32-accurate logits with no further rounding.  Picks come out in
// descending selection score; equal scores go to the lower expert index.
// Each lane owns experts lane, lane+64, lane+128, lane+192 (E <= 256); the
// arg-max of every round is a butterfly over the wavefront.
#pragma once

#include "common.cuh"

namespace hy3moe {

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Token t, all 64 lanes of one wavefront; writes idx_out[t][0..K) and
// w_out[t][0..K).  SB: slices loaded per round (S is a multiple of SB).
template <int SB>
__device__ __forceinline__ void select_token(const double *__restrict__ part, int S, int T, int E,
                                             int K, const float *__restrict__ bias, int mode,
                                             float scale, float renorm_eps, int t, int lane,
                                             int32_t *__restrict__ idx_out,
                                             float *__restrict__ w_out) {
  double sel[4], prob[4], logit[4];
  float bq[4];
  bool live[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    live[q] = e < E;
    logit[q] = 0.0;
    bq[q] = (mode == 0 && bias && live[q]) ? bias[e] : 0.f;   // issued with the partials
  }
  // The partials of SB slices of all 4 experts go out together (one memory
  // round trip per SB slices, not per expert); the adds stay in slice order.
  // Experts past E re-read expert 0 and are not used.
  for (int s0 = 0; s0 < S; s0 += SB) {
    double v[4][SB];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = live[q] ? lane + 64 * q : 0;
#pragma unroll
      for (int j = 0; j < SB; ++j) v[q][j] = part[((size_t)(s0 + j) * T + t) * E + e];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < SB; ++j) logit[q] += v[q][j];
  }
  if (mode == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      prob[q] = 1.0 / (1.0 + exp(-logit[q]));
      sel[q] = live[q] ? prob[q] + (double)bq[q] : -INFINITY;
    }
  } else {
    double m = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) if (live[q]) m = fmax(m, logit[q]);
    m = wave_max_f64(m);
    double z = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      prob[q] = live[q] ? exp(logit[q] - m) : 0.0;
      z += prob[q];
    }
    z = wave_sum_f64(z);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      prob[q] = prob[q] / z;
      sel[q] = live[q] ? prob[q] : -INFINITY;
    }
  }

  bool taken[4] = {false, false, false, false};
  int my_pick = -1;
  double my_prob = 0.0, tot = 0.0;
  for (int j = 0; j < K; ++j) {
    double bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (live[q] && !taken[q] && sel[q] > bv) { bv = sel[q]; be = lane + 64 * q; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
    }
    // Every lane now agrees on the winner be.
    const int owner = be & 63, slot = be >> 6;
    double p = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) if (q == slot) p = prob[q];
    p = __shfl(p, owner, 64);
    if (lane == owner) {
#pragma unroll
      for (int q = 0; q < 4; ++q) if (q == slot) taken[q] = true;
    }
    if (lane == j) { my_pick = be; my_prob = p; }
    tot += p;
  }
  if (lane < K) {
    double w;
    if (mode == 0) w = (double)scale * (my_prob / tot);
    else w = my_prob / fmax(tot, (double)renorm_eps);
    idx_out[(size_t)t * K + lane] = my_pick;
    w_out[(size_t)t * K + lane] = (float)w;
  }
}

}  // namespace hy3moe
