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
// Each lane owns experts lane, lane+64, lane+128, lane+192 (E <= 256).  A
// selection round takes the largest remaining score of the wavefront (DPP
// moves within each row of 16 lanes, then the four row maxima) and the
// lowest expert index holding it (one ballot per slot, lowest slot first).
#pragma once

#include "common.cuh"

namespace hy3moe {

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}
// max(v, v of lane CTRL(lane)) for a DPP lane pattern CTRL that stays in the row.
template <int CTRL>
__device__ __forceinline__ double dpp_max_f64(double v) {
  const uint64_t b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp((int)b, (int)b, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(b >> 32), (int)(b >> 32), CTRL, 0xF, 0xF, false);
  return fmax(v, __longlong_as_double(((int64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = __builtin_amdgcn_readlane((int)b, l);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((int64_t)hi << 32) | lo);
}
// Maximum over the wavefront, the same in every lane (exact: no rounding).
// Row of 16: swap neighbours (quad_perm 1,0,3,2), pairs (2,3,0,1), then the
// mirrored half row and the mirrored row; then the four rows' maxima.
__device__ __forceinline__ double wave_max_f64_dpp(double v) {
  v = dpp_max_f64<0xB1>(v);
  v = dpp_max_f64<0x4E>(v);
  v = dpp_max_f64<0x141>(v);
  v = dpp_max_f64<0x140>(v);
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)),
              fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
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
    double lv = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (live[q] && !taken[q]) lv = fmax(lv, sel[q]);
    const double bv = wave_max_f64_dpp(lv);
    // The winner: the lowest expert index lane + 64 q whose score is bv
    // (slots in order, then the lowest lane).  Should no remaining score
    // equal bv (only possible with NaN scores), the lowest remaining expert.
    int owner = -1, slot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t m = __ballot(live[q] && !taken[q] && sel[q] == bv);
      if (owner < 0 && m) { owner = __builtin_ctzll(m); slot = q; }
    }
    if (owner < 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint64_t m = __ballot(live[q] && !taken[q]);
        if (owner < 0 && m) { owner = __builtin_ctzll(m); slot = q; }
      }
    }
    const int be = owner + 64 * slot;
    double p = 0.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) if (q == slot) p = prob[q];
    p = readlane_f64(p, owner);   // owner is uniform
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
