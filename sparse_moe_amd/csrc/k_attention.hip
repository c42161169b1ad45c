// Split-KV decode attention for GQA (head_dim 128, 8 query heads per KV
// head), following the Hy3 Preview inference case study, section "1.
// Attention dynamic scheduling": uniform tiles, a task map that shares the
// tiles out by the global tile count (hy3attn_plan, on the host), one
// workgroup per worker taking its tasks from the map, and a combine.
//
// HBM-bound: every cached key and value byte is read once.  A workgroup
// (4 wavefronts) walks a task's tokens in steps of 128, each wavefront a
// 32-token block, the next block's loads in flight while one is multiplied.
// The 8 query heads' scores and the P V product run on MFMA (see
// attn_split_mfma_kernel); the softmax keeps one running maximum per head
// and wavefront.  At the end of a task the 4 wavefronts' streams are merged
// in LDS and written as one split.  Scores are kept in log2 units (scaled by
// log2(e)/sqrt(128) after the dot product), so the softmax uses exp2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "hy3attn.h"

namespace hy3attn {

namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int D = HY3ATTN_HEAD_DIM;   // 128
constexpr int G = HY3ATTN_GROUP;      // 8 query heads per KV head
struct Partial {
  float *o;    // [n_tasks][G][D] unnormalised output
  float *ml;   // [n_tasks][2][G]: running maximum (log2 units), sum
};

__device__ __forceinline__ float exp2_or_zero(float x) { return x == -INFINITY ? 0.f : exp2f(x); }

// The split kernel.  Per wavefront, 32-token blocks of a task
// (the workgroup's 4 wavefronts take consecutive blocks of each 128-token
// step):
//  * scores: S^T[token][head] = K Q^T with MFMA 16x16x32 (bf16 in, float32
//    out), K the A operand loaded straight from memory (lane (m, g) takes
//    dims 32s + 8g .. +8 of token m of a 16-token tile: 16 rows x 64 bytes per
//    instruction, every row whole over the 4 K steps), Q^T the B operand held
//    for the task (columns 8..15 zero: 8 query heads per KV head).  Lane (n, g)
//    then holds the scores of head n for tokens 4g .. 4g+3 of each tile.
//  * softmax: one running maximum per head, common to the wavefront (the
//    block maximum crosses the 4 lane groups of a head with two shuffles);
//    each lane keeps a partial sum.
//  * P V: O[head][dim] += P[head][token] V[token][dim], again MFMA
//    16x16x32.  The contraction runs over the block's 32 tokens in the order
//    that puts lane (n, g)'s own 8 probabilities in its A operand (slot j:
//    token 4g + j of tile 0 for j < 4, token 4g + j - 4 of tile 1 after), so
//    P needs no data movement; the B operand gathers the same tokens' values
//    of one dimension from the wavefront's V tile in LDS (32 rows x 256
//    bytes, written by the wavefront itself).  P goes in as bf16 hi + lo
//    (two MFMAs on the same V operand), so it keeps ~16 significant bits and
//    the float32 partial sum l matches it.
// The unnormalised output, maximum and sum per task go to the same partials
// the combine kernel reads.
// A 16-byte load with the non-temporal hint: every cached value byte is
// read once.  (The V rows are loaded 4 tokens x 256 contiguous bytes per
// wavefront instruction; with the hint the split kernel ran 66 -> 77 % of HBM
// peak on one 131072-token request.  The same hint on the K loads, 16 tokens
// x 64 bytes per instruction, was slower.)
__device__ __forceinline__ uint4 load_nt(const uint16_t *p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ f32x4 mma_bf16(const uint4 &a, const uint4 &b, f32x4 c) {
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// The softmax and P V of one 32-token block, given its score tiles s0, s1
// (S^T of tokens tb + [0, 16) and tb + [16, 32)) and the block's V rows in
// this wavefront's LDS tile vs.
__device__ __forceinline__ void block_softmax_pv(const f32x4 &s0, const f32x4 &s1, int tb, int e,
                                                 float qscale, float &m, float &l, f32x4 (&o)[8],
                                                 const uint16_t *vs, int g4, int n16) {
  float sv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = tb + 16 * (j >> 2) + 4 * g4 + (j & 3);
    const float x = (j < 4 ? s0 : s1)[j & 3];
    sv[j] = tok < e ? x * qscale : -INFINITY;
  }
  float mb = sv[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) mb = fmaxf(mb, sv[j]);
  mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
  mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
  const float mn = fmaxf(m, mb);
  const float a = mn == -INFINITY ? 1.f : exp2_or_zero(m - mn);
  uint32_t ph[4], pl[4];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    const float p0 = mn == -INFINITY ? 0.f : exp2_or_zero(sv[j] - mn);
    const float p1 = mn == -INFINITY ? 0.f : exp2_or_zero(sv[j + 1] - mn);
    ps += p0 + p1;
    const uint32_t h0 = bf16_rne(p0), h1 = bf16_rne(p1);
    const float r0 = p0 - __uint_as_float(h0 << 16), r1 = p1 - __uint_as_float(h1 << 16);
    ph[j >> 1] = h0 | (h1 << 16);
    pl[j >> 1] = bf16_rne(r0) | (bf16_rne(r1) << 16);
  }
  l = l * a + ps;
  m = mn;
  // the O rows of this lane are heads 4 g4 + r: their rescale factors
  float ar[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) ar[r] = __shfl(a, 4 * g4 + r, 64);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    o[i][0] *= ar[0]; o[i][1] *= ar[1]; o[i][2] *= ar[2]; o[i][3] *= ar[3];
  }
  const uint4 pa_hi = make_uint4(ph[0], ph[1], ph[2], ph[3]);
  const uint4 pa_lo = make_uint4(pl[0], pl[1], pl[2], pl[3]);
  // B operand of dim block i: the tokens of slots j (rows 4 g4 + j, then
  // 16 + 4 g4 + j - 4) at dim 16 i + n16
  const uint16_t *c0 = vs + (4 * g4) * D + n16, *c1 = vs + (16 + 4 * g4) * D + n16;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 bv = make_uint4(
        (uint32_t)c0[0 * D + 16 * i] | ((uint32_t)c0[1 * D + 16 * i] << 16),
        (uint32_t)c0[2 * D + 16 * i] | ((uint32_t)c0[3 * D + 16 * i] << 16),
        (uint32_t)c1[0 * D + 16 * i] | ((uint32_t)c1[1 * D + 16 * i] << 16),
        (uint32_t)c1[2 * D + 16 * i] | ((uint32_t)c1[3 * D + 16 * i] << 16));
    o[i] = mma_bf16(pa_hi, bv, o[i]);
    o[i] = mma_bf16(pa_lo, bv, o[i]);
  }
}

__global__ __launch_bounds__(256, 2) void attn_split_mfma_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ kv_start, int B, int Hkv,
    int tile, const int32_t *__restrict__ tasks, int n_tasks,
    const int32_t *__restrict__ worker_begin, Partial part) {
  constexpr int BLK = 32;                  // tokens per wavefront block
  constexpr int STEP = 4 * BLK;            // tokens per workgroup step
  __shared__ uint4 vtile[4][BLK * D / 8];  // per wavefront: [32 tokens][128 dims] bf16
  __shared__ float mls[4][2][G];
  __shared__ float os[4][G][D];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g4 = lane >> 4;
  const int total = kv_start[B];
  const float qscale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
  const int t_beg = max(worker_begin[blockIdx.x], 0);
  const int t_end = min(worker_begin[blockIdx.x + 1], n_tasks);
  uint4 *vw = vtile[wave];
  const uint16_t *vs = reinterpret_cast<const uint16_t *>(vtile[wave]);
  for (int t = t_beg; t < t_end; ++t) {
    const int b = __builtin_amdgcn_readfirstlane(tasks[4 * t]);
    const int h = __builtin_amdgcn_readfirstlane(tasks[4 * t + 1]);
    const int t0 = __builtin_amdgcn_readfirstlane(tasks[4 * t + 2]);
    const int t1 = __builtin_amdgcn_readfirstlane(tasks[4 * t + 3]);
    const bool valid = b >= 0 && b < B && h >= 0 && h < Hkv && t0 >= 0 && t1 > t0;
    const int base = valid ? kv_start[b] : 0, L = valid ? kv_start[b + 1] - base : 0;
    const int64_t s64 = (int64_t)t0 * tile, e64 = min((int64_t)t1 * tile, (int64_t)L);
    const int s = base + (int)min(s64, (int64_t)L);
    const int e = base + (int)e64;
    if (!valid || e <= s) {   // a plan made for other lengths: an empty split, no loads
      const int g = tid >> 5, d4 = tid & 31;
      *reinterpret_cast<float4 *>(part.o + ((size_t)t * G + g) * D + 4 * d4) =
          make_float4(0.f, 0.f, 0.f, 0.f);
      if (d4 == 0) {
        part.ml[(size_t)t * 2 * G + g] = -INFINITY;
        part.ml[(size_t)t * 2 * G + G + g] = 0.f;
      }
      continue;
    }
    // Q^T operand: lane (head n16, K group g4), dims 32 st + 8 g4 .. +8
    uint4 qb[4];
#pragma unroll
    for (int st = 0; st < 4; ++st)
      qb[st] = n16 < G ? *reinterpret_cast<const uint4 *>(
                             q + ((size_t)b * (G * Hkv) + G * h + n16) * D + 32 * st + 8 * g4)
                       : make_uint4(0u, 0u, 0u, 0u);
    float m = -INFINITY, l = 0.f;    // head n16: common maximum, this lane's partial sum
    f32x4 o[8];                      // O[head 4 g4 + r][dim 16 i + n16]
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the KV head's rows: a uniform base plus 32-bit element offsets (the
    // caller's K and V hold fewer than 2^31 elements per KV head)
    const uint16_t *kh = k + (size_t)h * total * D;
    const uint16_t *vh = v + (size_t)h * total * D;
    // A block's loads: K operands of its 2 tiles x 4 K steps (lane (m, g):
    // token m of the tile, dims 32 st + 8 g), V rows (lane (row g, chunk n):
    // dims 8 n .. +8 of token 4 i + g); tokens past e re-read token e - 1 (in
    // bounds) and are masked.  Two sets of named registers: the next block's
    // loads are in flight while one is multiplied.
#define ATT_K(S, tt, st, tok) S##k##tt##st = *reinterpret_cast<const uint4 *>(kh + ((tok) * D + 32 * st + 8 * g4));
#define ATT_V(S, i)                                                                    \
  S##v##i = load_nt(vh + ((uint32_t)min(tb_ + 4 * i + g4, e - 1) * D + 8 * n16));
#define ATT_W(S, i) vw[(4 * i + g4) * 16 + n16] = S##v##i;
#define ATT_LOAD(S, cb)                                                                \
  {                                                                                    \
    const int tb_ = (cb) + BLK * wave;                                                 \
    const uint32_t ta_ = (uint32_t)min(tb_ + n16, e - 1);                              \
    const uint32_t tc_ = (uint32_t)min(tb_ + 16 + n16, e - 1);                         \
    ATT_K(S, 0, 0, ta_) ATT_K(S, 0, 1, ta_) ATT_K(S, 0, 2, ta_) ATT_K(S, 0, 3, ta_)    \
    ATT_K(S, 1, 0, tc_) ATT_K(S, 1, 1, tc_) ATT_K(S, 1, 2, tc_) ATT_K(S, 1, 3, tc_)    \
    ATT_V(S, 0) ATT_V(S, 1) ATT_V(S, 2) ATT_V(S, 3)                                    \
    ATT_V(S, 4) ATT_V(S, 5) ATT_V(S, 6) ATT_V(S, 7)                                    \
  }
#define ATT_COMPUTE(S, cb)                                                             \
  {                                                                                    \
    const int tb_ = (cb) + BLK * wave;                                                 \
    f32x4 s0_ = f32x4{0.f, 0.f, 0.f, 0.f}, s1_ = f32x4{0.f, 0.f, 0.f, 0.f};           \
    s0_ = mma_bf16(S##k00, qb[0], s0_); s0_ = mma_bf16(S##k01, qb[1], s0_);            \
    s0_ = mma_bf16(S##k02, qb[2], s0_); s0_ = mma_bf16(S##k03, qb[3], s0_);            \
    s1_ = mma_bf16(S##k10, qb[0], s1_); s1_ = mma_bf16(S##k11, qb[1], s1_);            \
    s1_ = mma_bf16(S##k12, qb[2], s1_); s1_ = mma_bf16(S##k13, qb[3], s1_);            \
    ATT_W(S, 0) ATT_W(S, 1) ATT_W(S, 2) ATT_W(S, 3)                                    \
    ATT_W(S, 4) ATT_W(S, 5) ATT_W(S, 6) ATT_W(S, 7)                                    \
    block_softmax_pv(s0_, s1_, tb_, e, qscale, m, l, o, vs, g4, n16);                  \
  }
    uint4 ak00, ak01, ak02, ak03, ak10, ak11, ak12, ak13, av0, av1, av2, av3, av4, av5, av6, av7;
    uint4 bk00, bk01, bk02, bk03, bk10, bk11, bk12, bk13, bv0, bv1, bv2, bv3, bv4, bv5, bv6, bv7;
    ATT_LOAD(a, s)
    for (int cb = s; cb < e; cb += 2 * STEP) {
      ATT_LOAD(b, cb + STEP)
      ATT_COMPUTE(a, cb)
      if (cb + STEP >= e) break;
      ATT_LOAD(a, cb + 2 * STEP)
      ATT_COMPUTE(b, cb + STEP)
    }
#undef ATT_COMPUTE
#undef ATT_LOAD
#undef ATT_W
#undef ATT_V
#undef ATT_K
    // the wavefront's sum of head n16 over its 4 lane groups
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (g4 < 2) {   // heads 0..7 of O
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) os[wave][4 * g4 + r][16 * i + n16] = o[i][r];
    }
    if (lane < G) {
      mls[wave][0][lane] = m;
      mls[wave][1][lane] = l;
    }
    __syncthreads();
    {   // thread (head g, dims 4 d4 .. 4 d4 + 3): merge the 4 wavefronts
      const int g = tid >> 5, d4 = tid & 31;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, mls[w][0][g]);
      float L2 = 0.f, O[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float a = M == -INFINITY ? 0.f : exp2_or_zero(mls[w][0][g] - M);
        L2 += mls[w][1][g] * a;
#pragma unroll
        for (int j = 0; j < 4; ++j) O[j] += os[w][g][4 * d4 + j] * a;
      }
      *reinterpret_cast<float4 *>(part.o + ((size_t)t * G + g) * D + 4 * d4) =
          make_float4(O[0], O[1], O[2], O[3]);
      if (d4 == 0) {
        part.ml[(size_t)t * 2 * G + g] = M;
        part.ml[(size_t)t * 2 * G + G + g] = L2;
      }
    }
    __syncthreads();   // LDS reused by the next task
  }
}

// One workgroup per (request, KV head) row and query head g: merge the row's
// splits.  Thread (split lane sp of 8, dims 4 d4 .. 4 d4 + 3) takes splits
// sp, sp + 8, ...; the maxima and the partial sums meet in LDS.
__global__ __launch_bounds__(256) void attn_combine_kernel(const int32_t *__restrict__ row_begin,
                                                           int n_tasks, Partial part, int Hkv,
                                                           uint16_t *__restrict__ out) {
  __shared__ float red[8][33][4];   // per split lane: 32 dim quads + the denominator
  __shared__ float mx[8];
  const int r = blockIdx.x / G, g = blockIdx.x - r * G, b = r / Hkv, h = r - b * Hkv;
  const int sp = threadIdx.x >> 5, d4 = threadIdx.x & 31;
  // the row's task range, clamped to the plan's tasks
  const int t0 = max(row_begin[r], 0), t1 = min(row_begin[r + 1], n_tasks);
  float M = -INFINITY;
  for (int t = t0 + sp; t < t1; t += 8) M = fmaxf(M, part.ml[(size_t)t * 2 * G + g]);
  if (d4 == 0) mx[sp] = M;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 8; ++i) M = fmaxf(M, mx[i]);
  float den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t = t0 + sp; t < t1; t += 8) {
    const float a = M == -INFINITY ? 0.f : exp2_or_zero(part.ml[(size_t)t * 2 * G + g] - M);
    den += part.ml[(size_t)t * 2 * G + G + g] * a;
    const float4 o = *reinterpret_cast<const float4 *>(part.o + ((size_t)t * G + g) * D + 4 * d4);
    num[0] += o.x * a; num[1] += o.y * a; num[2] += o.z * a; num[3] += o.w * a;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[sp][d4][j] = num[j];
  if (d4 == 0) red[sp][32][0] = den;
  __syncthreads();
  if (sp != 0) return;
  float tot_den = 0.f, tot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < 8; ++i) {   // in split-lane order: the same sums every call
    tot_den += red[i][32][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[j] += red[i][d4][j];
  }
  uint16_t res[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float x = tot_den > 0.f ? tot[j] / tot_den : 0.f;   // no tokens: zeros
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);                           // round to nearest even
    res[j] = (uint16_t)(u >> 16);
  }
  uint16_t *dst = out + ((size_t)b * (G * Hkv) + G * h + g) * D + 4 * d4;
  *reinterpret_cast<uint2 *>(dst) =
      make_uint2((uint32_t)res[0] | ((uint32_t)res[1] << 16), (uint32_t)res[2] | ((uint32_t)res[3] << 16));
}

}  // namespace

}  // namespace hy3attn

using namespace hy3attn;

extern "C" int64_t hy3attn_max_tasks(int B, int n_kv_heads, int n_workers) {
  return (int64_t)n_workers + (int64_t)B * n_kv_heads;
}

extern "C" size_t hy3attn_workspace_bytes(int64_t max_tasks) {
  const size_t o = (size_t)max_tasks * G * D * 4, ml = (size_t)max_tasks * 2 * G * 4;
  return (o + 255) / 256 * 256 + ml;
}

extern "C" int hy3attn_plan(const int32_t *kv_len, int B, int n_kv_heads, int tile,
                            int n_workers, int32_t *tasks, int64_t max_tasks,
                            int32_t *worker_begin, int32_t *row_begin, int64_t *n_tasks) {
  if (B < 0 || n_kv_heads < 1 || tile < 1 || n_workers < 1 || (B > 0 && !kv_len) || !tasks ||
      !worker_begin || !row_begin || !n_tasks)
    return HY3ATTN_ERR_INVALID;
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    if (kv_len[b] < 0) return HY3ATTN_ERR_INVALID;
    total += (int64_t)n_kv_heads * ((kv_len[b] + tile - 1) / tile);
  }
  const int64_t cap = total > 0 ? (total + n_workers - 1) / n_workers : 1;
  int64_t nt = 0, used = 0;
  int w = 0;
  worker_begin[0] = 0;
  for (int b = 0; b < B; ++b) {
    const int64_t rt = (kv_len[b] + tile - 1) / tile;
    for (int h = 0; h < n_kv_heads; ++h) {
      row_begin[b * n_kv_heads + h] = (int32_t)nt;
      for (int64_t t = 0; t < rt;) {
        const int64_t take = cap - used < rt - t ? cap - used : rt - t;
        if (nt >= max_tasks) return HY3ATTN_ERR_SPACE;
        tasks[4 * nt] = b;
        tasks[4 * nt + 1] = h;
        tasks[4 * nt + 2] = (int32_t)t;
        tasks[4 * nt + 3] = (int32_t)(t + take);
        ++nt;
        t += take;
        used += take;
        if (used == cap) {   // this worker is full
          worker_begin[++w] = (int32_t)nt;
          used = 0;
        }
      }
    }
  }
  row_begin[(int64_t)B * n_kv_heads] = (int32_t)nt;
  if (used) worker_begin[++w] = (int32_t)nt;
  while (w < n_workers) worker_begin[++w] = (int32_t)nt;
  *n_tasks = nt;
  return HY3ATTN_OK;
}

extern "C" int hy3attn_decode(const void *q, const void *k, const void *v, const int32_t *kv_start,
                              int B, int n_kv_heads, int tile, const int32_t *tasks,
                              int64_t n_tasks, const int32_t *worker_begin, int n_workers,
                              const int32_t *row_begin, int64_t n_rows, void *workspace,
                              size_t ws_bytes, void *out, void *stream) {
  if (B < 0 || n_kv_heads < 1 || tile < 1 || n_workers < 1 || n_tasks < 0 ||
      n_tasks > INT32_MAX)
    return HY3ATTN_ERR_INVALID;
  // the plan must have been made for this call's rows (request, KV head)
  if (n_rows != (int64_t)B * n_kv_heads) return HY3ATTN_ERR_INVALID;
  if (B == 0) return HY3ATTN_OK;
  if (!q || !k || !v || !kv_start || !tasks || !worker_begin || !row_begin || !out ||
      (n_tasks > 0 && !workspace))
    return HY3ATTN_ERR_INVALID;
  if (ws_bytes < hy3attn_workspace_bytes(n_tasks) || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return HY3ATTN_ERR_INVALID;
  // 16-byte vector loads of q, k and v rows, 8-byte stores of out
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
       reinterpret_cast<uintptr_t>(v)) & 15 || (reinterpret_cast<uintptr_t>(out) & 7))
    return HY3ATTN_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Partial part;
  const size_t o_bytes = ((size_t)n_tasks * G * D * 4 + 255) / 256 * 256;
  part.o = static_cast<float *>(workspace);
  part.ml = reinterpret_cast<float *>(static_cast<char *>(workspace) + o_bytes);
  if (n_tasks > 0)
    hipLaunchKernelGGL(attn_split_mfma_kernel, dim3(n_workers), dim3(256), 0, s,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), kv_start, B, n_kv_heads, tile, tasks,
                       (int)n_tasks, worker_begin, part);
  if (hipGetLastError() != hipSuccess) return HY3ATTN_ERR_HIP;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((int64_t)B * n_kv_heads * G)), dim3(256), 0,
                     s, row_begin, (int)n_tasks, part, n_kv_heads, static_cast<uint16_t *>(out));
  return hipGetLastError() == hipSuccess ? HY3ATTN_OK : HY3ATTN_ERR_HIP;
}
