// Top-K weighted combine back to token order, with the shared expert added.
//
//   out[t] = sum_{j<K} w[t][j] * y[pos_of[t][j]]  +  y[offsets[E] + t]
//
// (Hy3 Preview inference case, section 3 table: top-K weighted aggregation at
// the end of the chain; HunyuanImage 3.0 MoE reading: routed outputs viewed as
// [T, K, H], multiplied by the routing weights and summed over K, then the
// shared branch added.)  Accumulation is fp32 in a fixed order (j = 0..K-1,
// then the shared row) with one rounding to the output type, so results are
// deterministic.  y is fp16 for bf16 layers (11 significant bits: the bf16
// rounding of every routed row's output before the weighted sum pushed the
// Hy3 prefill layer past its error bound) and float32 for float32 layers.
// Each thread handles 8 output values (bf16) or 4 (float32).
#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

// One 16-byte load of a y row: 8 fp16 values (bf16 layers) or 4 float32.
// The fp16 rows are read once, with the non-temporal hint (Hy3 prefill
// combine 0.133 -> 0.122 ms).
__device__ __forceinline__ void load_y(const f16_t *p, float *v) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  const uint4 u = make_uint4(q[0], q[1], q[2], q[3]);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = f16_lo(w[i]);
    v[2 * i + 1] = f16_hi(w[i]);
  }
}
__device__ __forceinline__ void load_y(const float *p, float *v) {
  const float4 u = *reinterpret_cast<const float4 *>(p);
  v[0] = u.x; v[1] = u.y; v[2] = u.z; v[3] = u.w;
}

template <typename T>
__device__ __forceinline__ void store_vec(T *p, const float *v);
template <>
__device__ __forceinline__ void store_vec<bf16_t>(bf16_t *p, const float *v) {
  uint4 u;
  u.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  u.z = (uint32_t)f32_to_bf16(v[4]) | ((uint32_t)f32_to_bf16(v[5]) << 16);
  u.w = (uint32_t)f32_to_bf16(v[6]) | ((uint32_t)f32_to_bf16(v[7]) << 16);
  *reinterpret_cast<uint4 *>(p) = u;
}
template <>
__device__ __forceinline__ void store_vec<float>(float *p, const float *v) {
  *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const typename YElem<T>::type *__restrict__ y,
                                                      const int32_t *__restrict__ pos_of,
                                                      const float *__restrict__ weight,
                                                      const int32_t *__restrict__ offsets, int K,
                                                      int H, int E, int has_shared,
                                                      T *__restrict__ out) {
  constexpr int V = Elem<T>::kPerChunk;
  const int t = blockIdx.x;
  const int n = (blockIdx.y * blockDim.x + threadIdx.x) * V;
  if (n >= H) return;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  // Blocks of 8 picks: all row loads of a block are issued before its FMAs.
  for (int j0 = 0; j0 < K; j0 += 8) {
    float v[8][V], w[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = j0 + jj < K ? j0 + jj : K - 1;
      const int p = pos_of[(size_t)t * K + j];
      w[jj] = weight[(size_t)t * K + j];
      load_y(y + (size_t)p * H + n, v[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < K) {
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = __builtin_fmaf(w[jj], v[jj][i], acc[i]);
      }
    }
  }
  if (has_shared) {
    float v[V];
    load_y(y + (size_t)(offsets[E] + t) * H + n, v);
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] += v[i];
  }
  store_vec<T>(out + (size_t)t * H + n, acc);
}

}  // namespace

hipError_t launch_combine(const void *y, const int32_t *pos_of, const float *weight,
                          const int32_t *offsets, int T, int K, int H, int E, int has_shared,
                          void *out, int dtype, hipStream_t stream) {
  if (dtype == DT_F32) {
    dim3 grid(T, (H / 4 + 255) / 256);
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, stream,
                       static_cast<const float *>(y), pos_of, weight, offsets, K, H, E, has_shared,
                       static_cast<float *>(out));
  } else {
    dim3 grid(T, (H / 8 + 255) / 256);
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, stream,
                       static_cast<const f16_t *>(y), pos_of, weight, offsets, K, H, E, has_shared,
                       static_cast<bf16_t *>(out));
  }
  return hipGetLastError();
}

}  // namespace hy3moe
