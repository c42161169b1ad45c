// Router GEMM: partial logits  part[s][t][e] = sum_{h in K-slice s} x[t,h] * W_r[e,h].
//
// The router is a bias-free H->E linear whose weight stays fp32 (HunyuanImage
// 3.0 MoE reading, HunyuanTopKGate `wg`; hy3 README keeps the router gate in
// F32 for routing stability).  On gfx950 the fp32 weight is split on the fly
// into bf16 terms and run on bf16 MFMA with fp32 accumulation:
//
//  * ROUTER_FP32 with bf16 x: W = W_hi + W_mid + W_lo exactly (each term is the
//    bf16 rounding of what is left), one accumulator per term, summed in the
//    epilogue.  Every bf16 x bf16 product is exact in fp32, so the logits are
//    as accurate as an fp32 dot product.
//  * ROUTER_SPLIT2_BF16 (Hy3 Preview inference case, section 2 "Router GEMM"):
//    W ~ W_hi + W_lo / 256 with W_lo = bf16(256 (W - W_hi)), two accumulators,
//    and one fused multiply-add acc_hi + acc_lo / 256 in the epilogue.
//  * fp32 x: fp32 MFMA on the fp32 weight directly.
//
// Tiling: a workgroup (4 waves) owns 64 experts x 64 tokens over one K-slice.
// The x tile is staged through LDS (shared by the 4 waves); each wave reads
// its own 16 expert rows of W straight from global memory.
//
// Accuracy: MFMA accumulates in fp32 over chunks of RT_CHUNK k values only;
// each chunk sum is added into a float64 running total, and the K-slice
// partials are written in float64 and summed by the select kernel in slice
// order.  A long fp32 accumulator chain would otherwise carry an error of
// several fp32 ulps of the logit at K = 4096.
#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

constexpr int RT_TOK = 64;        // tokens per workgroup
constexpr int RT_EXP = 64;        // experts per workgroup (16 per wave)
constexpr int RT_KB = 128;        // bytes of K per row per LDS stage (8 chunks)
constexpr int RT_CHUNK = 256;     // k values accumulated in fp32 before the fp64 add

// LDS chunk index of (row, chunk) with an XOR swizzle on the 8 chunks of a row.
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

__device__ __forceinline__ void split3(float w, uint16_t &hi, uint16_t &mid, uint16_t &lo) {
  hi = f32_to_bf16(w);
  const float r1 = w - bf16_to_f32(hi);     // exact
  mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);   // exact, fits 8 significant bits
  lo = f32_to_bf16(r2);
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) {
  return (uint32_t)a | ((uint32_t)b << 16);
}

// bf16 activations.  PREC: 0 = three-term exact split, 1 = two-term (x256) split.
template <int PREC>
__global__ __launch_bounds__(256) void router_bf16_kernel(const uint16_t *__restrict__ x,
                                                          const float *__restrict__ wr,
                                                          double *__restrict__ part, int T,
                                                          int H, int E, int kslice) {
  __shared__ uint4 xs[RT_TOK * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TOK, e0 = blockIdx.y * RT_EXP, s = blockIdx.z;
  const int kbeg = s * kslice;
  const int r16 = lane & 15, g = lane >> 4;
  const int e_row = e0 + wave * 16 + r16;
  const float *wrow = wr + (size_t)(e_row < E ? e_row : 0) * H;

  constexpr int NT = (PREC == 0) ? 3 : 2;
  f32x4_t acc[NT][4];
  double tot[4][4];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[a][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[n][q] = 0.0;

  for (int k0 = kbeg; k0 < kbeg + kslice; k0 += RT_KB / 2) {
    // Stage x[t0..t0+63][k0..k0+63] (bf16): 64 rows x 8 chunks, 2 per thread.
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = (tid >> 3) + 32 * rr, c = tid & 7;
      const int t = t0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t < T) v = *reinterpret_cast<const uint4 *>(x + (size_t)t * H + k0 + c * 8);
      xs[swz(row, c)] = v;
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kk = k0 + sub * 32 + g * 8;   // this lane's 8 k values
      const float4 wa = *reinterpret_cast<const float4 *>(wrow + kk);
      const float4 wb = *reinterpret_cast<const float4 *>(wrow + kk + 4);
      const float wv[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      uint16_t th[8], tm[8], tl[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (PREC == 0) {
          split3(wv[i], th[i], tm[i], tl[i]);
        } else {
          th[i] = f32_to_bf16(wv[i]);
          tm[i] = f32_to_bf16((wv[i] - bf16_to_f32(th[i])) * 256.0f);
        }
      }
      uint4 fa[NT];
      fa[0] = make_uint4(pack2(th[0], th[1]), pack2(th[2], th[3]), pack2(th[4], th[5]), pack2(th[6], th[7]));
      fa[1] = make_uint4(pack2(tm[0], tm[1]), pack2(tm[2], tm[3]), pack2(tm[4], tm[5]), pack2(tm[6], tm[7]));
      if (PREC == 0)
        fa[NT - 1] = make_uint4(pack2(tl[0], tl[1]), pack2(tl[2], tl[3]), pack2(tl[4], tl[5]), pack2(tl[6], tl[7]));
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint4 xb = xs[swz(n * 16 + r16, sub * 4 + g)];
#pragma unroll
        for (int a = 0; a < NT; ++a) Mma<bf16_t>::step(acc[a][n], fa[a], xb);
      }
    }
    __syncthreads();
    if (((k0 + RT_KB / 2 - kbeg) % RT_CHUNK) == 0 || k0 + RT_KB / 2 == kbeg + kslice) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (PREC == 0)
            tot[n][q] += (double)acc[0][n][q] + ((double)acc[1][n][q] + (double)acc[2][n][q]);
          else  // two accumulators, hi + lo/256 (one fused multiply-add per output)
            tot[n][q] = __builtin_fma((double)acc[1][n][q], 1.0 / 256.0,
                                      tot[n][q] + (double)acc[0][n][q]);
        }
#pragma unroll
        for (int a = 0; a < NT; ++a) acc[a][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // Lane holds D[expert 4g+q][token r16] of each token fragment n.
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int t = t0 + n * 16 + r16;
    if (t >= T) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + wave * 16 + 4 * g + q;
      if (e < E) part[((size_t)s * T + t) * E + e] = tot[n][q];
    }
  }
}

// fp32 activations: fp32 MFMA on the fp32 weight.
__global__ __launch_bounds__(256) void router_f32_kernel(const float *__restrict__ x,
                                                         const float *__restrict__ wr,
                                                         double *__restrict__ part, int T, int H,
                                                         int E, int kslice) {
  __shared__ uint4 xs[RT_TOK * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * RT_TOK, e0 = blockIdx.y * RT_EXP, s = blockIdx.z;
  const int kbeg = s * kslice;
  const int r16 = lane & 15, g = lane >> 4;
  const int e_row = e0 + wave * 16 + r16;
  const float *wrow = wr + (size_t)(e_row < E ? e_row : 0) * H;

  f32x4_t acc[4];
  double tot[4][4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[n][q] = 0.0;
  }

  for (int k0 = kbeg; k0 < kbeg + kslice; k0 += RT_KB / 4) {
    // Stage x[t0..t0+63][k0..k0+31] (fp32): 64 rows x 8 chunks.
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = (tid >> 3) + 32 * rr, c = tid & 7;
      const int t = t0 + row;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t < T) v = *reinterpret_cast<const uint4 *>(x + (size_t)t * H + k0 + c * 4);
      xs[swz(row, c)] = v;
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const uint4 wa = *reinterpret_cast<const uint4 *>(wrow + k0 + sub * 16 + g * 4);
#pragma unroll
      for (int n = 0; n < 4; ++n)
        Mma<float>::step(acc[n], wa, xs[swz(n * 16 + r16, sub * 4 + g)]);
    }
    __syncthreads();
    if (((k0 + RT_KB / 4 - kbeg) % RT_CHUNK) == 0 || k0 + RT_KB / 4 == kbeg + kslice) {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
#pragma unroll
        for (int q = 0; q < 4; ++q) tot[n][q] += (double)acc[n][q];
        acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    }
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int t = t0 + n * 16 + r16;
    if (t >= T) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + wave * 16 + 4 * g + q;
      if (e < E) part[((size_t)s * T + t) * E + e] = tot[n][q];
    }
  }
}

}  // namespace

int router_ksplit(int64_t T, int H, int E) {
  // Enough workgroups to spread the weight read over the chip; each K-slice
  // stays a multiple of 64 and at least 128 long.
  const int64_t tiles = ((T + RT_TOK - 1) / RT_TOK) * ((E + RT_EXP - 1) / RT_EXP);
  int S = 1;
  while (S < MAX_KSPLIT && tiles * S < 256 && (H / (2 * S)) >= 128 && (H % (2 * S * 64)) == 0)
    S *= 2;
  return S;
}

hipError_t launch_router(const void *x, int dtype, int router_prec, const float *wr, double *part,
                         int T, int H, int E, int S, hipStream_t stream) {
  const int kslice = H / S;
  dim3 grid((T + RT_TOK - 1) / RT_TOK, (E + RT_EXP - 1) / RT_EXP, S);
  if (dtype == DT_F32) {
    hipLaunchKernelGGL(router_f32_kernel, grid, dim3(256), 0, stream,
                       static_cast<const float *>(x), wr, part, T, H, E, kslice);
  } else if (router_prec == 0) {
    hipLaunchKernelGGL(router_bf16_kernel<0>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t *>(x), wr, part, T, H, E, kslice);
  } else {
    hipLaunchKernelGGL(router_bf16_kernel<1>, grid, dim3(256), 0, stream,
                       static_cast<const uint16_t *>(x), wr, part, T, H, E, kslice);
  }
  return hipGetLastError();
}

}  // namespace hy3moe
