// Achievable-ceiling probes for the roofline (measurement helpers, not part
// of the MoE layer): dense bf16 and FP8 MFMA microkernels with register
// operands only, a 16-byte-per-lane device copy, 16-byte-per-lane streaming
// reads (grid-strided, and in contiguous per-workgroup segments with 8 or 16
// loads in flight per lane), the weight-streaming GEMMs' fragment reads with
// the MFMAs removed (16 rows x 64 B or 4 rows x 256 B per load), and one FP8 MFMA per
// wavefront on given operands (its accumulation error, measured against
// exact sums by the caller).  Built into libhy3moe_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;

namespace {

// 16 independent accumulator chains per wavefront, so the MFMA pipe never
// waits on a dependency; operands live in registers.
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float *out) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
  }
  f32x4_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 16; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void copy_kernel(const uint4 *__restrict__ src,
                                                   uint4 *__restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

// Reads n16 16-byte chunks, 4 per thread per step in flight, and writes one
// word per thread (so the loads are not removed).
__global__ __launch_bounds__(256) void read_kernel(const uint4 *__restrict__ src, size_t n16,
                                                   uint32_t *__restrict__ out) {
  const size_t tid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ b.y ^ c.z ^ d.w;
  }
  for (; i < n16; i += stride) acc ^= src[i].x;
  out[tid] = acc;
}

// Streaming read the way the weight-streaming GEMMs read weights: each
// workgroup owns one contiguous segment of the buffer and its threads keep
// DEPTH 16-byte non-temporal loads in flight, consecutive lanes on
// consecutive 16 bytes (a wavefront load covers 1 KB), each round moving
// DEPTH x 4 KB of the segment.  One word per thread is written so that the
// loads stay.
template <int DEPTH>
__global__ __launch_bounds__(256) void read_segment_kernel(const uint4 *__restrict__ src,
                                                           size_t n16, size_t seg16,
                                                           uint32_t *__restrict__ out) {
  const size_t beg = (size_t)blockIdx.x * seg16;
  const size_t end = beg + seg16 < n16 ? beg + seg16 : n16;
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
  const u32x4_t *s4 = reinterpret_cast<const u32x4_t *>(src);
  uint32_t acc = 0;
  size_t i = beg + threadIdx.x;
  for (; i + (DEPTH - 1) * 256 < end; i += DEPTH * 256) {
    u32x4_t v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) v[d] = __builtin_nontemporal_load(s4 + i + d * 256);
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) acc ^= v[d][0] ^ v[d][3];
  }
  for (; i < end; i += 256) acc ^= src[i].y;
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}
// The weight-streaming GEMMs' read with the MFMAs removed: a unit is two
// fragments of 16 rows x rowbytes (the second half a buffer away, like the
// gate and up matrices), units striped over the wavefronts, each fragment
// read in sets of 8 loads (16 rows x 512 B) with two sets in flight.  A load
// covers R rows x 1024 / R contiguous bytes: R = 16 is the MFMA operand
// layout (64 B per row per load), R = 4 the four-row loads that the kernels
// transpose through LDS; NT adds the non-temporal hint.  One word per thread
// is written so that the loads stay.
template <int R, bool NT>
__global__ __launch_bounds__(256, 2) void read_fragments_kernel(const char *__restrict__ w,
                                                                size_t half, int rowbytes,
                                                                int n_units,
                                                                uint32_t *__restrict__ out) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
  constexpr int U = 8, LPR = 64 / R, W = 1024 / R, NRG = 16 / R;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nw = gridDim.x * 4, wid = blockIdx.x * 4 + wave;
  const int spu = rowbytes / 512;   // sets per unit
  const int my_units = wid < n_units ? (n_units - wid + nw - 1) / nw : 0;
  const int total_sets = my_units * spu;
  uint32_t acc = 0;
  // set -> (unit, 512-byte column), load j -> (row group, column group);
  // every address lies inside its unit's 16 x rowbytes fragment
  auto addr = [&](int set, int j) -> const u32x4_t * {
    const int k = set / spu, sc = set - k * spu;
    const size_t f = (size_t)(wid + k * nw) * 16 * rowbytes;
    const int row = (j % NRG) * R + lane / LPR;
    const size_t byte = (size_t)sc * 512 + (j / NRG) * W + (lane % LPR) * 16;
    return reinterpret_cast<const u32x4_t *>(w + f + (size_t)row * rowbytes + byte);
  };
  auto ld = [&](const u32x4_t *p) { return NT ? __builtin_nontemporal_load(p) : *p; };
  auto second = [&](const u32x4_t *p) {
    return reinterpret_cast<const u32x4_t *>(reinterpret_cast<const char *>(p) + half);
  };
  u32x4_t a0[U], a1[U], b0[U], b1[U];
  if (total_sets > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) { a0[u] = ld(addr(0, u)); a1[u] = ld(second(addr(0, u))); }
  }
  for (int set = 0; set < total_sets; set += 2) {
    if (set + 1 < total_sets) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        b0[u] = ld(addr(set + 1, u));
        b1[u] = ld(second(addr(set + 1, u)));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc ^= a0[u][0] ^ a0[u][1] ^ a0[u][2] ^ a0[u][3] ^ a1[u][0] ^ a1[u][1] ^ a1[u][2] ^ a1[u][3];
    if (set + 1 >= total_sets) break;
    if (set + 2 < total_sets) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        a0[u] = ld(addr(set + 2, u));
        a1[u] = ld(second(addr(set + 2, u)));
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      acc ^= b0[u][0] ^ b0[u][1] ^ b0[u][2] ^ b0[u][3] ^ b1[u][0] ^ b1[u][1] ^ b1[u][2] ^ b1[u][3];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

// The same with 16x16x128 E4M3 x E4M3 MFMAs (one per chain per iteration).
__global__ __launch_bounds__(256) void mfma_fp8_peak_kernel(int iters, float *out) {
  const int lane = threadIdx.x & 63;
  i32x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = 0x38303830 + ((lane + i) & 7);
    b[i] = 0x30383038 + ((lane * 3 + i) & 7);
  }
  f32x4_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 16; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Instance b (one wavefront): D = A B with C = 0, one 16x16x128 FP8 MFMA on
// the lane operands a[b][lane] and b[b][lane] (32 bytes each).
__global__ __launch_bounds__(64) void mfma_fp8_once_kernel(const i32x8_t *a, const i32x8_t *b,
                                                          f32x4_t *d, int n) {
  const int inst = blockIdx.x, lane = threadIdx.x;
  if (inst >= n) return;
  const size_t i = (size_t)inst * 64 + lane;
  d[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[i], f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                          0, 0, 0, 0, 0, 0);
}

// Instance b: D = A B with C = 0, one block-scaled 16x16x128 MFMA with FP4
// E2M1 A (16 bytes per lane) and FP8 E4M3 B (32 bytes per lane) and one E8M0
// scale byte per lane on each side (byte 0 of sa[b][lane], sb[b][lane]).
__global__ __launch_bounds__(64) void mfma_fp4fp8_once_kernel(const i32x8_t *a, const i32x8_t *b,
                                                             const int *sa, const int *sb,
                                                             f32x4_t *d, int n) {
  const int inst = blockIdx.x, lane = threadIdx.x;
  if (inst >= n) return;
  const size_t i = (size_t)inst * 64 + lane;
  d[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[i], f32x4_t{0.f, 0.f, 0.f, 0.f},
                                                          4, 0, 0, sa[i], 0, sb[i]);
}

}  // namespace

extern "C" {

// n instances of one block-scaled FP4 x FP8 MFMA: a, b hold n x 64 lanes x
// 32 bytes (A uses the first 16 bytes: 32 E2M1 codes, element 2j in the low
// nibble of byte j), sa, sb n x 64 ints (E8M0 in byte 0), d n x 64 x 4 floats
// (lane 16 c + r: rows 4 c + q, column r).
int hy3moe_probe_mfma_fp4fp8_once(const void *a, const void *b, const int *sa, const int *sb,
                                  float *d, int n, void *stream) {
  if (!a || !b || !sa || !sb || !d || n <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_fp4fp8_once_kernel, dim3(n), dim3(64), 0,
                     static_cast<hipStream_t>(stream), static_cast<const i32x8_t *>(a),
                     static_cast<const i32x8_t *>(b), sa, sb, reinterpret_cast<f32x4_t *>(d), n);
  return (int)hipGetLastError();
}

// FLOPs done = n_blocks * 4 waves * iters * 16 MFMAs * 2*16*16*128.
// `out` needs n_blocks * 256 floats.  Returns a hipError_t code.
int hy3moe_probe_mfma_fp8(int n_blocks, int iters, float *out, void *stream) {
  if (n_blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_fp8_peak_kernel, dim3(n_blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return (int)hipGetLastError();
}

// n instances of one FP8 MFMA: a, b hold n x 64 lanes x 32 bytes (E4M3
// codes), d receives n x 64 lanes x 4 floats (lane 16 c + r: rows 4 c + q,
// column r).  Lane 16 g + r of a supplies row r and lane 16 g + r of b
// column r, with the same 32 K positions.
int hy3moe_probe_mfma_fp8_once(const void *a, const void *b, float *d, int n, void *stream) {
  if (!a || !b || !d || n <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_fp8_once_kernel, dim3(n), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const i32x8_t *>(a), static_cast<const i32x8_t *>(b),
                     reinterpret_cast<f32x4_t *>(d), n);
  return (int)hipGetLastError();
}

// FLOPs done = n_blocks * 4 waves * iters * 16 MFMAs * 2*16*16*32.
// `out` needs n_blocks * 256 floats.  Returns a hipError_t code.
int hy3moe_probe_mfma(int n_blocks, int iters, float *out, void *stream) {
  if (n_blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(n_blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return (int)hipGetLastError();
}

// Copies `bytes` (multiple of 16) from src to dst with n_blocks x 256 threads.
int hy3moe_probe_copy(const void *src, void *dst, size_t bytes, int n_blocks, void *stream) {
  if (!src || !dst || (bytes & 15) || n_blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_kernel, dim3(n_blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), bytes / 16);
  return (int)hipGetLastError();
}

// Reads `bytes` (multiple of 16) from src with n_blocks x 256 threads; out
// holds n_blocks x 256 words.
int hy3moe_probe_read(const void *src, size_t bytes, int n_blocks, void *out, void *stream) {
  if (!src || !out || (bytes & 15) || n_blocks <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_kernel, dim3(n_blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4 *>(src), bytes / 16, static_cast<uint32_t *>(out));
  return (int)hipGetLastError();
}

// Reads the units of 2 x 16 rows x rowbytes that fit in `bytes` in the
// weight-streaming GEMMs' pattern (read_fragments_kernel): rows_per_load 16
// or 4, nontemporal 0 or 1, rowbytes a positive multiple of 512; returns
// the bytes read through *read_bytes.  out holds n_blocks x 256 words.
int hy3moe_probe_read_fragments(const void *src, size_t bytes, int rowbytes, int rows_per_load,
                                int nontemporal, int n_blocks, void *out, size_t *read_bytes,
                                void *stream) {
  if (!src || !out || !read_bytes || n_blocks <= 0 || rowbytes <= 0 || rowbytes % 512 ||
      (rows_per_load != 16 && rows_per_load != 4))
    return (int)hipErrorInvalidValue;
  const size_t half = bytes / 2;
  const size_t units = half / ((size_t)16 * rowbytes);
  if (units == 0 || units > (size_t)1 << 30) return (int)hipErrorInvalidValue;
  *read_bytes = 2 * units * 16 * (size_t)rowbytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char *w = static_cast<const char *>(src);
  uint32_t *o = static_cast<uint32_t *>(out);
  const int n = (int)units;
#define HY3_RF(R_, NT_)                                                                \
  hipLaunchKernelGGL((read_fragments_kernel<R_, NT_>), dim3(n_blocks), dim3(256), 0, s, w, half, \
                     rowbytes, n, o)
  if (rows_per_load == 16) {
    if (nontemporal) HY3_RF(16, true); else HY3_RF(16, false);
  } else {
    if (nontemporal) HY3_RF(4, true); else HY3_RF(4, false);
  }
#undef HY3_RF
  return (int)hipGetLastError();
}

// Reads `bytes` (multiple of 16) from src as n_blocks contiguous segments,
// depth (8 or 16) loads in flight per thread; out holds n_blocks x 256 words.
int hy3moe_probe_read_segments(const void *src, size_t bytes, int n_blocks, int depth, void *out,
                               void *stream) {
  if (!src || !out || (bytes & 15) || n_blocks <= 0 || (depth != 8 && depth != 16))
    return (int)hipErrorInvalidValue;
  const size_t n16 = bytes / 16, seg16 = (n16 + n_blocks - 1) / n_blocks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (depth == 8)
    hipLaunchKernelGGL(read_segment_kernel<8>, dim3(n_blocks), dim3(256), 0, s,
                       static_cast<const uint4 *>(src), n16, seg16, static_cast<uint32_t *>(out));
  else
    hipLaunchKernelGGL(read_segment_kernel<16>, dim3(n_blocks), dim3(256), 0, s,
                       static_cast<const uint4 *>(src), n16, seg16, static_cast<uint32_t *>(out));
  return (int)hipGetLastError();
}

}  // extern "C"
