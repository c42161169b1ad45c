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
// Large batches (router_planes): every token tile would repeat the same split
// of the same weight, so the split runs once per call into bf16 planes
// [NP][E][H] in the workspace, and the GEMM streams the planes with the next
// K step's weight fragments and the x tile after it already in flight (x
// double-buffered in LDS).  The mid and lo products share one fp32
// accumulator there (their sum is 2^-8 of the logit, so its rounding is far
// below the hi accumulator's); the fp64 folding is the same.
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

// Small batches (T <= 64, one token tile): every workgroup has little work and
// the per-step weight-load latency dominates, so each 256-long K chunk is
// fetched at once: the x chunk (T rows x 512 B) into LDS and the lane's 8
// weight slices of 8 floats into registers, then 8 x-steps of MFMA on the
// split terms.  Token fragments past T are skipped (uniform branch).  Same
// arithmetic as router_bf16_kernel: three (or two) fp32 accumulators per
// 256-value chunk, folded into float64.
template <int PREC>
__global__ __launch_bounds__(256) void router_small_kernel(const uint16_t *__restrict__ x,
                                                           const float *__restrict__ wr,
                                                           double *__restrict__ part, int T,
                                                           int H, int E, int kslice) {
  constexpr int KC = RT_CHUNK;             // k values per chunk (256)
  __shared__ uint4 xs[RT_TOK * KC / 8];    // 64 rows x 512 B
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e0 = blockIdx.y * RT_EXP, s = blockIdx.z;
  const int kbeg = s * kslice;
  const int r16 = lane & 15, g = lane >> 4;
  const int e_row = e0 + wave * 16 + r16;
  const float *wrow = wr + (size_t)(e_row < E ? e_row : 0) * H;
  const int nfrag = (T + 15) >> 4;         // token fragments with real rows

  constexpr int NT = (PREC == 0) ? 3 : 2;
  double tot[4][4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[n][q] = 0.0;

  for (int kc = kbeg; kc < kbeg + kslice; kc += KC) {
    const int kn = min(KC, kbeg + kslice - kc);   // a multiple of 64
    // Weight: sub-step u covers k = kc + 32u + 8g .. +7 (8 floats per lane).
    float4 wv[16];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int kk = kc + (32 * u < kn ? 32 * u : 0) + g * 8;
      wv[2 * u] = *reinterpret_cast<const float4 *>(wrow + kk);
      wv[2 * u + 1] = *reinterpret_cast<const float4 *>(wrow + kk + 4);
    }
    // x chunk: row r, 16-byte chunk c (kn / 8 chunks per row).
    const int cpr = kn / 8;
    for (int i = tid; i < RT_TOK * cpr; i += 256) {
      const int r = i / cpr, c = i - r * cpr;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < T) v = *reinterpret_cast<const uint4 *>(x + (size_t)r * H + kc + c * 8);
      xs[r * (KC / 8) + (c ^ (r & 7))] = v;
    }
    __syncthreads();
    f32x4_t acc[NT][4];
#pragma unroll
    for (int a = 0; a < NT; ++a)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[a][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (32 * u < kn) {
        const float w8[8] = {wv[2 * u].x, wv[2 * u].y, wv[2 * u].z, wv[2 * u].w,
                             wv[2 * u + 1].x, wv[2 * u + 1].y, wv[2 * u + 1].z, wv[2 * u + 1].w};
        uint16_t th[8], tm[8], tl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (PREC == 0) {
            split3(w8[i], th[i], tm[i], tl[i]);
          } else {
            th[i] = f32_to_bf16(w8[i]);
            tm[i] = f32_to_bf16((w8[i] - bf16_to_f32(th[i])) * 256.0f);
          }
        }
        uint4 fa[NT];
        fa[0] = make_uint4(pack2(th[0], th[1]), pack2(th[2], th[3]), pack2(th[4], th[5]), pack2(th[6], th[7]));
        fa[1] = make_uint4(pack2(tm[0], tm[1]), pack2(tm[2], tm[3]), pack2(tm[4], tm[5]), pack2(tm[6], tm[7]));
        if (PREC == 0)
          fa[NT - 1] = make_uint4(pack2(tl[0], tl[1]), pack2(tl[2], tl[3]), pack2(tl[4], tl[5]), pack2(tl[6], tl[7]));
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          if (n < nfrag) {
            const int r = n * 16 + r16;
            const uint4 xb = xs[r * (KC / 8) + ((u * 4 + g) ^ (r & 7))];
#pragma unroll
            for (int a = 0; a < NT; ++a) Mma<bf16_t>::step(acc[a][n], fa[a], xb);
          }
        }
      }
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (PREC == 0)
          tot[n][q] += (double)acc[0][n][q] + ((double)acc[1][n][q] + (double)acc[2][n][q]);
        else
          tot[n][q] = __builtin_fma((double)acc[1][n][q], 1.0 / 256.0,
                                    tot[n][q] + (double)acc[0][n][q]);
      }
    }
    __syncthreads();   // xs is rewritten by the next chunk
  }

#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int t = n * 16 + r16;
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

// fp32 weight -> bf16 planes, 8 elements per thread.  PREC 0: hi, mid, lo
// (exact three-term split); PREC 1: hi and bf16(256 (w - hi)).
//
// Fragment-major layout, so that each of the planes kernel's weight loads is
// one contiguous 1 KB block per wavefront (8 whole cache lines, not 16
// half lines of 16 rows): for expert block b (16 experts; E padded to a
// multiple of 16, the padding rows repeating expert E-1), K step st (64
// values), plane p and half `sub` (32 values), 64 lanes of 16 bytes, lane
// 16 g + r holding W[16 b + r][64 st + 32 sub + 8 g + (0..7)], i.e. uint4
// index (((b * (H/64) + st) * NP + p) * 2 + sub) * 64 + lane.
template <int PREC>
__global__ __launch_bounds__(256) void router_split_kernel(const float *__restrict__ wr,
                                                           uint16_t *__restrict__ planes, int E,
                                                           int H, int E_pad) {
  constexpr int NP = (PREC == 0) ? 3 : 2;
  const int cpr = H / 8;                                    // 8-value chunks per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)E_pad * cpr) return;
  const int e = (int)(i / cpr), c = (int)(i - (int64_t)e * cpr);
  const float *src = wr + (size_t)min(e, E - 1) * H + c * 8;
  const float4 a = *reinterpret_cast<const float4 *>(src);
  const float4 b = *reinterpret_cast<const float4 *>(src + 4);
  const float wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint16_t th[8], tm[8], tl[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (PREC == 0) {
      split3(wv[j], th[j], tm[j], tl[j]);
    } else {
      th[j] = f32_to_bf16(wv[j]);
      tm[j] = f32_to_bf16((wv[j] - bf16_to_f32(th[j])) * 256.0f);
    }
  }
  // c * 8 = 64 st + 32 sub + 8 g
  const int st = c >> 3, sub = (c >> 2) & 1, g = c & 3;
  const size_t o = ((size_t)((e >> 4) * (H / 64) + st) * NP * 2 + sub) * 64 + g * 16 + (e & 15);
  uint4 *out = reinterpret_cast<uint4 *>(planes);
  out[o] = make_uint4(pack2(th[0], th[1]), pack2(th[2], th[3]), pack2(th[4], th[5]),
                      pack2(th[6], th[7]));
  out[o + 2 * 64] = make_uint4(pack2(tm[0], tm[1]), pack2(tm[2], tm[3]), pack2(tm[4], tm[5]),
                               pack2(tm[6], tm[7]));
  if (PREC == 0)
    out[o + 4 * 64] = make_uint4(pack2(tl[0], tl[1]), pack2(tl[2], tl[3]), pack2(tl[4], tl[5]),
                                 pack2(tl[6], tl[7]));
}

// Wavefronts (16 experts each) of a planes-kernel workgroup for E experts:
// every expert of the layer in one workgroup where E <= 192, so that a
// 64-token x tile is read once for all of them.
inline int planes_waves(int E) { return E <= 64 ? 4 : E <= 128 ? 8 : 12; }

// Router GEMM on pre-split bf16 planes.  A workgroup of NW wavefronts takes
// 64 tokens x 16 NW experts over one K-slice.  K steps of 64: the weight
// fragments of step st+1 are loaded while step st computes (two register
// sets), the x tile of step st+2 goes to registers (wavefronts 0-3) and is
// written to the idle LDS buffer at the end of step st+1.  Loads past the
// last step re-read it (in bounds, unused) so that no load is conditional,
// and a scheduling barrier keeps them at the top of the step.  The loop body
// is one fp64 fold period (4 steps), so the fold needs no branch.  Token rows
// past T re-read row T-1 and are not stored; experts past E re-read expert
// E-1 and are not stored.
//
// XCD-aware order: the three weight planes (E x H x 6 bytes: 4.7 MB at Hy3
// shape) exceed one XCD's L2, so the work items (slice, expert block, token
// tile) are numbered slice-major and each XCD takes a contiguous run of
// them (workgroup b runs on XCD b % 8): an XCD then reads only its slices'
// share of the planes, which stays in its L2 while the x tiles stream past.
template <int PREC, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void router_planes_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wp, double *__restrict__ part,
    int T, int H, int E, int kslice, int S) {
  constexpr int NP = (PREC == 0) ? 3 : 2;
  constexpr int XB = RT_TOK * 8;   // uint4 per LDS buffer
  constexpr int FOLD = RT_CHUNK / 64;
  __shared__ uint4 xs[2 * XB];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_tt = (T + RT_TOK - 1) / RT_TOK, n_eb = (E + 16 * NW - 1) / (16 * NW);
  const int n_items = n_tt * n_eb * S, per = (n_items + 7) / 8;
  const int item = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (item >= n_items) return;   // the grid is padded to a multiple of 8 x per
  const int combo = item / n_tt, tt = item - combo * n_tt;
  const int s = combo / n_eb, eb = combo - s * n_eb;
  const int t0 = tt * RT_TOK, e0 = eb * 16 * NW;
  const int kbeg = s * kslice;
  const bool xload = wave < 4;     // wavefronts 0-3 stage the x tile
  const int r16 = lane & 15, g = lane >> 4;
  // the wavefront's expert block (blocks past the last repeat it: not stored)
  const int blk = min((e0 >> 4) + wave, (E + 15) / 16 - 1);
  const uint4 *wfrag = reinterpret_cast<const uint4 *>(wp) +
                       (size_t)(blk * (H / 64) + kbeg / 64) * NP * 2 * 64 + lane;
  const int xrow = tid >> 3, xc = tid & 7;
  const uint16_t *xp0 = x + (size_t)min(t0 + xrow, T - 1) * H + kbeg + xc * 8;
  const uint16_t *xp1 = x + (size_t)min(t0 + xrow + 32, T - 1) * H + kbeg + xc * 8;
  const int xw0 = swz(xrow, xc), xw1 = swz(xrow + 32, xc);
  const int n = kslice / 64;

  f32x4_t ahi[4], alo[4];
  double tot[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ahi[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    alo[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) tot[j][q] = 0.0;
  }
  // Register sets A and B: weight fragments w<set><sub><plane>, x chunks x<set><0|1>.
  uint4 wA00, wA01, wA02, wA10, wA11, wA12, xA0, xA1;
  uint4 wB00, wB01, wB02, wB10, wB11, wB12, xB0, xB1;

#define HY3_W(st, sub, p) (wfrag[(uint32_t)((((st) * NP + (p)) * 2 + (sub)) * 64)])
#define HY3_LOADW(S, st)                                                               \
  {                                                                                    \
    const int st_ = (st);                                                              \
    w##S##00 = HY3_W(st_, 0, 0); w##S##01 = HY3_W(st_, 0, 1);                          \
    w##S##10 = HY3_W(st_, 1, 0); w##S##11 = HY3_W(st_, 1, 1);                          \
    if (NP == 3) { w##S##02 = HY3_W(st_, 0, 2); w##S##12 = HY3_W(st_, 1, 2); }         \
  }
#define HY3_LOADX(S, st)                                                               \
  if (xload) {                                                                         \
    const int st_ = (st);                                                              \
    x##S##0 = *reinterpret_cast<const uint4 *>(xp0 + st_ * 64);                        \
    x##S##1 = *reinterpret_cast<const uint4 *>(xp1 + st_ * 64);                        \
  }
#define HY3_SUB(S, sub, buf)                                                           \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                      \
    const uint4 xv = xs[(buf) * XB + swz(j * 16 + r16, (sub) * 4 + g)];                \
    Mma<bf16_t>::step(ahi[j], w##S##sub##0, xv);                                       \
    Mma<bf16_t>::step(alo[j], w##S##sub##1, xv);                                       \
    if (NP == 3) Mma<bf16_t>::step(alo[j], w##S##sub##2, xv);                          \
  }
// Step st with its weights in set C and the x of step st+1 in set N.
#define HY3_STEP(st, C, N, buf)                                                        \
  {                                                                                    \
    HY3_LOADW(N, min((st) + 1, n - 1));                                                \
    HY3_LOADX(C, min((st) + 2, n - 1));                                                \
    __builtin_amdgcn_sched_barrier(0);                                                 \
    HY3_SUB(C, 0, buf);                                                                \
    HY3_SUB(C, 1, buf);                                                                \
    if (xload) {                                                                       \
      xs[((buf) ^ 1) * XB + xw0] = x##N##0;                                            \
      xs[((buf) ^ 1) * XB + xw1] = x##N##1;                                            \
    }                                                                                  \
    __syncthreads();                                                                   \
  }
#define HY3_FOLD()                                                                     \
  _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                      \
    _Pragma("unroll") for (int q = 0; q < 4; ++q) {                                    \
      if (PREC == 0)                                                                   \
        tot[j][q] += (double)ahi[j][q] + (double)alo[j][q];                            \
      else                                                                             \
        tot[j][q] = __builtin_fma((double)alo[j][q], 1.0 / 256.0, tot[j][q] + (double)ahi[j][q]); \
    }                                                                                  \
    ahi[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};                                              \
    alo[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};                                              \
  }

  HY3_LOADW(A, 0);
  HY3_LOADX(A, 0);
  HY3_LOADX(B, min(1, n - 1));
  if (xload) {
    xs[xw0] = xA0;
    xs[xw1] = xA1;
  }
  __syncthreads();
  static_assert(FOLD == 4, "loop body is one fold period of 4 steps");
  int st = 0;
  for (; st + FOLD <= n; st += FOLD) {
    HY3_STEP(st, A, B, 0);
    HY3_STEP(st + 1, B, A, 1);
    HY3_STEP(st + 2, A, B, 0);
    HY3_STEP(st + 3, B, A, 1);
    HY3_FOLD();
  }
  if (st < n) {   // 1..3 remaining steps (kslice not a multiple of 256)
    HY3_STEP(st, A, B, 0);
    if (st + 1 < n) HY3_STEP(st + 1, B, A, 1);
    if (st + 2 < n) HY3_STEP(st + 2, A, B, 0);
    HY3_FOLD();
  }
#undef HY3_FOLD
#undef HY3_STEP
#undef HY3_SUB
#undef HY3_LOADX
#undef HY3_LOADW
#undef HY3_W

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = t0 + j * 16 + r16;
    if (t >= T) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + wave * 16 + 4 * g + q;
      if (e < E) part[((size_t)s * T + t) * E + e] = tot[j][q];
    }
  }
}

}  // namespace

bool router_use_planes(int64_t T, int dtype) { return dtype == DT_BF16 && T >= ROUTER_PLANES_MIN_T; }

int router_ksplit(int64_t T, int H, int E, int dtype) {
  // Enough workgroups to spread the weight read over the chip (the planes
  // kernel: about one workgroup of up to 12 wavefronts per CU; the others:
  // 512 of 4 wavefronts); each K-slice stays a multiple of 64 and at least
  // 128 long.
  const bool planes = router_use_planes(T, dtype);
  const int eb = planes ? 16 * planes_waves(E) : RT_EXP;
  const int64_t tiles = ((T + RT_TOK - 1) / RT_TOK) * ((E + eb - 1) / eb);
  const int64_t want = planes ? (planes_waves(E) == 4 ? 512 : 256) : 512;
  int S = 1;
  while (S < MAX_KSPLIT && tiles * S < want && (H / (2 * S)) >= 128 &&
         (H % (2 * S * 64)) == 0)
    S *= 2;
  return S;
}

size_t router_planes_bytes(int E, int H, int router_prec) {
  return (size_t)(router_prec == 0 ? 3 : 2) * ((E + 15) / 16 * 16) * H * 2;
}

hipError_t launch_router_split(const float *wr, int router_prec, uint16_t *planes, int E, int H,
                               hipStream_t stream) {
  const int E_pad = (E + 15) / 16 * 16;
  const dim3 sgrid((unsigned)(((int64_t)E_pad * H / 8 + 255) / 256));
  if (router_prec == 0)
    hipLaunchKernelGGL(router_split_kernel<0>, sgrid, dim3(256), 0, stream, wr, planes, E, H,
                       E_pad);
  else
    hipLaunchKernelGGL(router_split_kernel<1>, sgrid, dim3(256), 0, stream, wr, planes, E, H,
                       E_pad);
  return hipGetLastError();
}

hipError_t launch_router(const void *x, int dtype, int router_prec, const float *wr,
                         uint16_t *planes, const uint16_t *planes_in, double *part, int T, int H,
                         int E, int S, hipStream_t stream) {
  const int kslice = H / S;
  dim3 grid((T + RT_TOK - 1) / RT_TOK, (E + RT_EXP - 1) / RT_EXP, S);
  if (planes) {
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const int nw = planes_waves(E);
    const int64_t items = (int64_t)((T + RT_TOK - 1) / RT_TOK) *
                          ((E + 16 * nw - 1) / (16 * nw)) * S;
    const dim3 pgrid((unsigned)((items + 7) / 8 * 8));   // 8 equal XCD runs
    // the caller's offline split, else split once into the workspace
    const uint16_t *wp = planes_in;
    if (!wp) {
      const hipError_t e = launch_router_split(wr, router_prec, planes, E, H, stream);
      if (e != hipSuccess) return e;
      wp = planes;
    }
#define HY3_PLANES(P, NW)                                                              \
  hipLaunchKernelGGL((router_planes_kernel<P, NW>), pgrid, dim3(64 * NW), 0, stream, xb, wp, \
                     part, T, H, E, kslice, S)
    if (router_prec == 0) {
      if (nw == 4) HY3_PLANES(0, 4);
      else if (nw == 8) HY3_PLANES(0, 8);
      else HY3_PLANES(0, 12);
    } else {
      if (nw == 4) HY3_PLANES(1, 4);
      else if (nw == 8) HY3_PLANES(1, 8);
      else HY3_PLANES(1, 12);
    }
#undef HY3_PLANES
    return hipGetLastError();
  }
  if (dtype == DT_F32) {
    hipLaunchKernelGGL(router_f32_kernel, grid, dim3(256), 0, stream,
                       static_cast<const float *>(x), wr, part, T, H, E, kslice);
  } else if (T <= RT_TOK) {
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    if (router_prec == 0)
      hipLaunchKernelGGL(router_small_kernel<0>, grid, dim3(256), 0, stream, xb, wr, part, T, H,
                         E, kslice);
    else
      hipLaunchKernelGGL(router_small_kernel<1>, grid, dim3(256), 0, stream, xb, wr, part, T, H,
                         E, kslice);
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
