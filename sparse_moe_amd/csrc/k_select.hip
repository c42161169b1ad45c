// Scores, top-K selection and combine weights, one wavefront per token (the
// per-token steps are in select_token.cuh).
#include "common.cuh"
#include "internal.h"
#include "select_token.cuh"

namespace hy3moe {

namespace {

template <int SB>
__global__ __launch_bounds__(256) void select_kernel(const double *__restrict__ part, int S, int T,
                                                     int E, int K,
                                                     const float *__restrict__ bias, int mode,
                                                     float scale, float renorm_eps,
                                                     int32_t *__restrict__ idx_out,
                                                     float *__restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole wavefront leaves together
  select_token<SB>(part, S, T, E, K, bias, mode, scale, renorm_eps, t, lane, idx_out, w_out);
}

}  // namespace

hipError_t launch_select(const double *part, int S, int T, int E, int K, const float *bias,
                         int route_mode, float scale, float renorm_eps, int32_t *idx,
                         float *weight, hipStream_t stream) {
  // S is a power of two <= MAX_KSPLIT: load min(S, 4) slices per round (of
  // 4, 8 and 16 per round, 4 measured fastest).
  const dim3 grid((T + 3) / 4);
#define HY3_SEL(SB)                                                                    \
  hipLaunchKernelGGL(select_kernel<SB>, grid, dim3(256), 0, stream, part, S, T, E, K, bias, \
                     route_mode, scale, renorm_eps, idx, weight)
  if (S >= 4) HY3_SEL(4);
  else if (S == 2) HY3_SEL(2);
  else HY3_SEL(1);
#undef HY3_SEL
  return hipGetLastError();
}

}  // namespace hy3moe
