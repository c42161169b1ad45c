// Per-thread bodies of the activation quantisers (k_quant.hip's kernels,
// and the select launch that hosts the decode batches' x quantisation).
//
// Static FP8 (W8A8 experts): every element divided by one float32 scale and
// rounded to E4M3, saturating, nearest even (CANN deployment article on Hy3,
// section 六, FP8 path; section 8.2 W8A8).  Dynamic MXFP8 (W4A8 experts): the
// OCP microscaling conversion of blocks of 32 consecutive values along a row,
// four threads holding a block's 32 values (mxfp8_quant8).  Either writes the
// code bytes (and E8M0 block scales) or, as the "carrier", their exact bf16
// values.
#pragma once

#include "common.cuh"

namespace hy3moe {

template <typename T>
__device__ __forceinline__ void quant_load8(const T *p, float *v);
template <>
__device__ __forceinline__ void quant_load8<bf16_t>(const bf16_t *p, float *v) {
  const uint4 u = *reinterpret_cast<const uint4 *>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void quant_load8<float>(const float *p, float *v) {
  const float4 a = reinterpret_cast<const float4 *>(p)[0];
  const float4 b = reinterpret_cast<const float4 *>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Static FP8: elements [8 i, 8 i + 8) of x.
template <typename T, bool CARRIER>
__device__ __forceinline__ void quant_e4m3_8(const T *x, int64_t i, float s, void *q) {
  float v[8];
  quant_load8(x + 8 * i, v);
  const uint32_t c0 = quant_e4m3x4(v[0], v[1], v[2], v[3], s);
  const uint32_t c1 = quant_e4m3x4(v[4], v[5], v[6], v[7], s);
  if (CARRIER) {
    const uint2 lo = e4m3x4_to_bf16(c0), hi = e4m3x4_to_bf16(c1);
    reinterpret_cast<uint4 *>(q)[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
    reinterpret_cast<uint2 *>(q)[i] = make_uint2(c0, c1);
  }
}

// Dynamic MXFP8: elements [8 i, 8 i + 8) of a block of 32 whose other three
// quarters are held by the neighbouring lanes (i % 4 == lane % 4, all four
// active).  CARRIER: the bf16 values (code value x 2^exponent) in place of
// codes and scales; `in` may alias q then (each thread rewrites only the 16
// bytes it read).
template <bool CARRIER>
__device__ __forceinline__ void quant_mxfp8_8(const bf16_t *in, int64_t i, void *q,
                                              uint8_t *scales) {
  float v[8];
  quant_load8(in + 8 * i, v);
  uint32_t code;
  const uint2 c = mxfp8_quant8(v, code);
  if (CARRIER) {
    const float sc = e8m0_to_f32(code);
    const uint32_t w[4] = {
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.x, sc, true)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, false)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c.y, sc, true))};
    reinterpret_cast<uint4 *>(q)[i] = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    reinterpret_cast<uint2 *>(q)[i] = c;
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)code;
  }
}

}  // namespace hy3moe
