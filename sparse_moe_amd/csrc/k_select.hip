// Scores, top-K selection and combine weights, one wavefront per token (the
// per-token steps are in select_token.cuh); the launch can also host an
// activation quantisation in workgroups of its own, saving the decode
// batches a launch of their own for it.
#include "common.cuh"
#include "internal.h"
#include "quant_dev.cuh"
#include "select_token.cuh"

namespace hy3moe {

namespace {

// The hosted quantisation (HostedQuant): workgroups sel_blocks.. of the
// launch stride over the 8-element chunks (a multiple of 4 threads, so that
// the four lanes of an MXFP8 block stay together).
__device__ void hosted_quant(const HostedQuant &hq, int qb, int nqb) {
  const int64_t n8 = hq.n / 8, stride = (int64_t)nqb * 256;
  for (int64_t i = (int64_t)qb * 256 + threadIdx.x; i < n8; i += stride) {
    if (hq.mode == QH_MXFP8) {
      const bf16_t *x = static_cast<const bf16_t *>(hq.x);
      if (hq.carrier) quant_mxfp8_8<true>(x, i, hq.q, hq.scales);
      else quant_mxfp8_8<false>(x, i, hq.q, hq.scales);
    } else if (hq.dtype == DT_F32) {
      const float *x = static_cast<const float *>(hq.x);
      if (hq.carrier) quant_e4m3_8<float, true>(x, i, *hq.scale, hq.q);
      else quant_e4m3_8<float, false>(x, i, *hq.scale, hq.q);
    } else {
      const bf16_t *x = static_cast<const bf16_t *>(hq.x);
      if (hq.carrier) quant_e4m3_8<bf16_t, true>(x, i, *hq.scale, hq.q);
      else quant_e4m3_8<bf16_t, false>(x, i, *hq.scale, hq.q);
    }
  }
}

template <int SB>
__global__ __launch_bounds__(256) void select_kernel(const double *__restrict__ part, int S, int T,
                                                     int E, int K,
                                                     const float *__restrict__ bias, int mode,
                                                     float scale, float renorm_eps,
                                                     int32_t *__restrict__ idx_out,
                                                     float *__restrict__ w_out, HostedQuant hq,
                                                     int sel_blocks) {
  if ((int)blockIdx.x >= sel_blocks) {   // uniform per workgroup
    hosted_quant(hq, blockIdx.x - sel_blocks, gridDim.x - sel_blocks);
    return;
  }
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole wavefront leaves together
  select_token<SB>(part, S, T, E, K, bias, mode, scale, renorm_eps, t, lane, idx_out, w_out);
}

}  // namespace

hipError_t launch_select(const double *part, int S, int T, int E, int K, const float *bias,
                         int route_mode, float scale, float renorm_eps, int32_t *idx,
                         float *weight, hipStream_t stream, const HostedQuant &hq) {
  // S is a power of two <= MAX_KSPLIT: load min(S, 4) slices per round (of
  // 4, 8 and 16 per round, 4 measured fastest).
  const int sel_blocks = (T + 3) / 4;
  int q_blocks = 0;
  if (hq.mode != QH_NONE) {
    if (hq.n % (hq.mode == QH_MXFP8 ? 32 : 8) || !hq.x || !hq.q ||
        (hq.mode == QH_E4M3 && !hq.scale) || (hq.mode == QH_MXFP8 && !hq.carrier && !hq.scales))
      return hipErrorInvalidValue;
    const int64_t want = (hq.n / 8 + 255) / 256;
    q_blocks = (int)(want < 4096 ? want : 4096);
  }
  const dim3 grid(sel_blocks + q_blocks);
#define HY3_SEL(SB)                                                                    \
  hipLaunchKernelGGL(select_kernel<SB>, grid, dim3(256), 0, stream, part, S, T, E, K, bias, \
                     route_mode, scale, renorm_eps, idx, weight, hq, sel_blocks)
  if (S >= 4) HY3_SEL(4);
  else if (S == 2) HY3_SEL(2);
  else HY3_SEL(1);
#undef HY3_SEL
  return hipGetLastError();
}

}  // namespace hy3moe
