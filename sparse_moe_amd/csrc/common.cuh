// Device-side helpers shared by the gfx950 kernels of the MoE layer.
//
// MFMA operand convention used by every kernel here
// -------------------------------------------------
// Each lane of a 64-wide wavefront supplies one 16-byte "chunk" of an A row
// and one of a B row.  Lane l = 16*g + r supplies chunk g (bytes 16g..16g+15
// of a 64-byte K segment) of row r.  One call of Mma<T>::step() adds
//     D[m][n] += sum_{g, i} A_chunk(row m, chunk g)[i] * B_chunk(row n, chunk g)[i]
// i.e. the dot product of row m of A with row n of B over a 64-byte K slab
// (32 bf16 or 16 fp32 values).  bf16 uses one v_mfma_f32_16x16x32_bf16;
// fp32 uses four v_mfma_f32_16x16x4_f32, element i of every lane's chunk
// feeding the i-th one.  The result tile is the standard 16x16 C layout:
// lane l holds D[4*(l/16) + q][l % 16] in acc[q], q = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hy3moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// bfloat16 stored as its raw 16 bits.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float -> bfloat16 bits (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats -> packed bfloat16 pair (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kPerChunk = 8;   // elements in 16 bytes
  static constexpr int kBytes = 2;
};
template <> struct Elem<float> {
  static constexpr int kPerChunk = 4;
  static constexpr int kBytes = 4;
};

template <typename T> struct Mma;

template <> struct Mma<bf16_t> {
  __device__ __forceinline__ static void step(f32x4_t &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  __device__ __forceinline__ static void step(f32x4_t &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// Store four consecutive output values (one lane's column of a 16x16 tile).
__device__ __forceinline__ void store4(bf16_t *p, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

// Expert outputs y (the down GEMMs' results before the combine): IEEE fp16
// (11 significant bits, round to nearest even) for bf16 layers, float32 for
// float32 layers.
struct f16_t { uint16_t bits; };
template <typename T> struct YElem { typedef f16_t type; };
template <> struct YElem<float> { typedef float type; };

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 ha = (_Float16)a, hb = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ void store4(f16_t *p, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_f16x2(a, b);
  v.y = pack_f16x2(c, d);
  *reinterpret_cast<uint2 *>(p) = v;
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// OCP FP8 E4M3 bytes -> bf16, exact (every E4M3 value is a bf16 value).  The
// gfx950 scaled conversion with scale 1 decodes two bytes per instruction,
// low bytes first.
#define HY3_E4M3_PAIR(w, h) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((w), 1.0f, (h)))
// 8 codes (bytes 0..7 of q) -> 8 bf16.
__device__ __forceinline__ uint4 e4m3x8_to_bf16(const uint2 &q) {
  return make_uint4(HY3_E4M3_PAIR(q.x, false), HY3_E4M3_PAIR(q.x, true),
                    HY3_E4M3_PAIR(q.y, false), HY3_E4M3_PAIR(q.y, true));
}
// 16 codes -> two fragments of 8 bf16 (bytes 0-7, bytes 8-15).
__device__ __forceinline__ void e4m3x16_to_bf16(const uint4 &q, uint4 &lo, uint4 &hi) {
  lo = e4m3x8_to_bf16(make_uint2(q.x, q.y));
  hi = e4m3x8_to_bf16(make_uint2(q.z, q.w));
}

// Static FP8 activation quantisation: E4M3 code of v / s, the quotient a
// correctly rounded float32 division, clamped to +-448 (saturating) and
// rounded to the nearest E4M3 value, ties to even (v_cvt_pk_fp8_f32).
// Four values -> bytes 0..3 of the result.
__device__ __forceinline__ uint32_t quant_e4m3x4(float a, float b, float c, float d, float s) {
  const float lim = 448.0f;
  a = fminf(fmaxf(a / s, -lim), lim);
  b = fminf(fmaxf(b / s, -lim), lim);
  c = fminf(fmaxf(c / s, -lim), lim);
  d = fminf(fmaxf(d / s, -lim), lim);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// The same with the quotient taken as v * r for a reciprocal r given by the
// caller: exact when r is a power of two (the MXFP8 block scales below).
__device__ __forceinline__ uint32_t quant_e4m3x4_rcp(float a, float b, float c, float d,
                                                     float r) {
  const float lim = 448.0f;
  a = fminf(fmaxf(a * r, -lim), lim);
  b = fminf(fmaxf(b * r, -lim), lim);
  c = fminf(fmaxf(c * r, -lim), lim);
  d = fminf(fmaxf(d * r, -lim), lim);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
// v rounded to bfloat16 (nearest even) and back: the value an activation
// takes as the layer's bf16 tensor (finite inputs).
__device__ __forceinline__ float round_bf16(float v) {
  uint32_t u = __float_as_uint(v);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}
// Static FP8 quantisation of the layer's bf16 h: E4M3 codes of round_bf16(v)
// / s, four values (the SwiGLU outputs of a GEMM epilogue) at a time.
__device__ __forceinline__ uint32_t quant_e4m3x4_bf16(float a, float b, float c, float d,
                                                      float s) {
  return quant_e4m3x4(round_bf16(a), round_bf16(b), round_bf16(c), round_bf16(d), s);
}
// Dynamic MXFP8 (OCP microscaling conversion) of a block of 32 consecutive
// values held by four adjacent lanes, 8 each: the lanes exchange their
// maxima, the block's shared exponent is floor(log2 amax) - 8 (8: E4M3's
// largest exponent), floored at -127, i.e. the E8M0 code max(exponent field
// - 8, 0); each value is multiplied by 2^-exponent (exact) and rounded to
// E4M3 (saturating, nearest even).  Returns the lane's 8 codes and sets
// `code` to the block's E8M0 code.  Every lane of the wavefront must call it.
__device__ __forceinline__ uint2 mxfp8_quant8(const float (&v)[8], uint32_t &code) {
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = fmaxf(m, fabsf(v[k]));
  m = fmaxf(m, __shfl_xor(m, 1));
  m = fmaxf(m, __shfl_xor(m, 2));
  const uint32_t ef = (__float_as_uint(m) >> 23) & 0xFFu;
  code = ef > 8u ? ef - 8u : 0u;
  const float inv = __uint_as_float((254u - code) << 23);   // 2^-(code - 127)
  return make_uint2(quant_e4m3x4_rcp(v[0], v[1], v[2], v[3], inv),
                    quant_e4m3x4_rcp(v[4], v[5], v[6], v[7], inv));
}

// Four codes -> their values as 4 bf16 (exact): the bf16 form in which the
// bf16-MFMA paths carry quantised activations.
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
  return make_uint2(HY3_E4M3_PAIR(w, false), HY3_E4M3_PAIR(w, true));
}
#undef HY3_E4M3_PAIR

// E8M0 scale code -> float 2^(c - 127) (c = 0: the float32 subnormal 2^-127;
// c = 255, NaN in E8M0, is not expected).
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
  return c ? __uint_as_float(c << 23) : __uint_as_float(0x00400000u);
}
// 8 FP4 E2M1 codes (4 bytes, element 2j in the low nibble of byte j) times a
// float scale -> 8 bf16 (exact for scales down to 2^-124).
#define HY3_FP4_PAIR(w, sc, b) \
  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((w), (sc), (b)))
__device__ __forceinline__ uint4 fp4x8_to_bf16(uint32_t w, float sc) {
  return make_uint4(HY3_FP4_PAIR(w, sc, 0), HY3_FP4_PAIR(w, sc, 1), HY3_FP4_PAIR(w, sc, 2),
                    HY3_FP4_PAIR(w, sc, 3));
}
#undef HY3_FP4_PAIR

// One block-scaled 16x16x128 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4): A = 32 FP4 E2M1 weights of the lane (16
// bytes) with E8M0 scale sa, B = 32 FP8 E4M3 token values (two 16-byte
// chunks) with E8M0 scale sb.
// One 16x16x128 FP8 (E4M3 x E4M3) MFMA; each operand is two 16-byte chunks.
// A and B lane group g's 32 bytes pair up byte for byte (both operands are
// 8-bit), so any K order that both sides share gives the same sum.
__device__ __forceinline__ void mma_fp8(f32x4_t &acc, const uint4 &a0, const uint4 &a1,
                                        const uint4 &b0, const uint4 &b1) {
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const i32x8_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                      (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const i32x8_t bv = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                      (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ void mma_fp4_fp8(f32x4_t &acc, const uint4 &w, uint32_t sa,
                                            const uint4 &x0, const uint4 &x1, uint32_t sb) {
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const i32x8_t av = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  const i32x8_t bv = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                      (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  // formats: 4 = FP4 E2M1 (A), 0 = FP8 E4M3 (B); scale byte 0 of each operand
  acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 0, 0, (int)sa, 0,
                                                         (int)sb);
}

// SiLU(g) * u in fp32: g / (1 + e^-g) * u, the quotient by the hardware
// reciprocal (within an ulp; the result is rounded to bf16 or E4M3 after).
__device__ __forceinline__ float swiglu(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) {
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// Mask of the active lanes (among `live`) whose key equals this lane's key.
// Keys are < 512 (9 bits).
__device__ __forceinline__ uint64_t match_key(int key, uint64_t live) {
  uint64_t m = live;
#pragma unroll
  for (int b = 0; b < 9; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__device__ __forceinline__ size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace hy3moe
