// Activation quantisation for the quantised-expert formats.
//
// Static FP8 activation quantisation (W8A8 experts).  Every element of x is
// divided by one float32 scale and rounded to E4M3 (saturating, nearest
// even): an FP8 Linear quantises its input with a static per-tensor scale
// (CANN deployment article on Hy3, section 六, FP8 path; section 8.2 W8A8).
// The result is either the code bytes or their exact bf16 values (the form
// the bf16-MFMA expert paths read).  HBM-bound: each thread converts 8
// elements per step with 16-byte loads.
#include "common.cuh"
#include "internal.h"
#include "quant_dev.cuh"

namespace hy3moe {

namespace {

__device__ __forceinline__ float load1(const bf16_t *p) {
  return __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(p) << 16);
}
__device__ __forceinline__ float load1(const float *p) { return *p; }

// Elements [0, 8 * n8): 8 per thread per step.
template <typename T, bool CARRIER>
__global__ __launch_bounds__(256) void quant_vec_kernel(const T *x, int64_t n8,
                                                        const float *scale, void *q) {
  const float s = *scale;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride)
    quant_e4m3_8<T, CARRIER>(x, i, s, q);
}

// Elements [begin, n): one per thread (the tail of the vector kernel).
template <typename T, bool CARRIER>
__global__ __launch_bounds__(64) void quant_tail_kernel(const T *x, int64_t begin, int64_t n,
                                                        const float *scale, void *q) {
  const int64_t i = begin + threadIdx.x;
  if (i >= n) return;
  const uint32_t c = quant_e4m3x4(load1(x + i), 0.0f, 0.0f, 0.0f, *scale);
  if (CARRIER)
    reinterpret_cast<uint16_t *>(q)[i] = (uint16_t)(e4m3x4_to_bf16(c).x & 0xFFFFu);
  else
    reinterpret_cast<uint8_t *>(q)[i] = (uint8_t)(c & 0xFFu);
}

// Dynamic MXFP8 quantisation of rows of a multiple of 32 values (see
// quant_dev.cuh).
template <bool CARRIER>
__global__ __launch_bounds__(256) void mxq_kernel(const bf16_t *in, int64_t n8, void *q,
                                                  uint8_t *scales) {
  // stride and n8 are multiples of 4, so the four lanes of a block (which
  // exchange maxima) stay in or leave the loop together
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += stride)
    quant_mxfp8_8<CARRIER>(in, i, q, scales);
}

template <typename T, bool CARRIER>
hipError_t launch_t(const T *x, int64_t n, const float *scale, void *q, hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 > 0) {
    const int64_t want = (n8 + 255) / 256;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL((quant_vec_kernel<T, CARRIER>), dim3(blocks), dim3(256), 0, stream, x, n8,
                       scale, q);
  }
  if (n > 8 * n8)
    hipLaunchKernelGGL((quant_tail_kernel<T, CARRIER>), dim3(1), dim3(64), 0, stream, x, 8 * n8,
                       n, scale, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_mxfp8(const void *in, int64_t n, void *q, uint8_t *scales, int carrier,
                              hipStream_t stream) {
  const int64_t n8 = n / 8;   // n % 32 == 0
  if (n8 <= 0) return hipSuccess;
  const int64_t want = (n8 + 255) / 256;
  const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
  const bf16_t *x = static_cast<const bf16_t *>(in);
  if (carrier)
    hipLaunchKernelGGL((mxq_kernel<true>), dim3(blocks), dim3(256), 0, stream, x, n8, q, scales);
  else
    hipLaunchKernelGGL((mxq_kernel<false>), dim3(blocks), dim3(256), 0, stream, x, n8, q, scales);
  return hipGetLastError();
}

hipError_t launch_quant_e4m3(const void *x, int dtype, int64_t n, const float *scale, void *q,
                             int carrier, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  if (dtype == DT_F32)
    return carrier ? launch_t<float, true>(static_cast<const float *>(x), n, scale, q, stream)
                   : launch_t<float, false>(static_cast<const float *>(x), n, scale, q, stream);
  return carrier ? launch_t<bf16_t, true>(static_cast<const bf16_t *>(x), n, scale, q, stream)
                 : launch_t<bf16_t, false>(static_cast<const bf16_t *>(x), n, scale, q, stream);
}

}  // namespace hy3moe
