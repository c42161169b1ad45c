// Split-KV decode attention for GQA (head_dim 128, 8 query heads per KV
// head), following the Hy3 Preview inference case study, section "1.
// Attention dynamic scheduling": uniform tiles, a task map that shares the
// tiles out by the global tile count (hy3attn_plan, on the host), one
// workgroup per worker taking its tasks from the map, and a combine.
//
// HBM-bound: every cached key and value byte is read once.  A workgroup
// (4 wavefronts) walks a task's tokens in chunks of 32, the next chunk's
// loads in flight while one is multiplied; lane (row r, chunk c)
// of a wavefront holds head-dims 8c .. 8c+7 of token 4 i + r of its step i,
// so one 16-byte load per lane covers 4 whole 256-byte key rows (1 KB
// contiguous).  The 8 query heads' scores of a token are summed over the 16
// lanes of its row with DPP moves (the sum lands in all 16 lanes), and each
// row keeps its own online softmax (running maximum m, sum l and the
// unnormalised output of its 8 dims for the 8 heads) over the tokens it
// sees.  At the end of a task the 16 row streams of the workgroup are merged
// (lane shuffles inside a wavefront, then LDS) and written as one split.
// Scores are kept in log2 units (q is pre-multiplied by log2(e)/sqrt(128)),
// so the softmax uses exp2.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "hy3attn.h"

namespace hy3attn {

namespace {

constexpr int D = HY3ATTN_HEAD_DIM;   // 128
constexpr int G = HY3ATTN_GROUP;      // 8 query heads per KV head
constexpr int STEPS = 2;              // token steps per chunk (4 tokens per wavefront step)
constexpr int CHUNK = 4 * 4 * STEPS;  // tokens per workgroup chunk: 4 waves x 4 rows x STEPS

struct Partial {
  float *o;    // [n_tasks][G][D] unnormalised output
  float *ml;   // [n_tasks][2][G]: running maximum (log2 units), sum
};

__device__ __forceinline__ void bf16x8_to_f32(const uint4 u, float *f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// x + x of lane CTRL(lane), for a DPP pattern inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF,
                                            0xF, false);
  return x + __int_as_float(y);
}
// Sum over the 16 lanes of a row, in all of them: neighbours, pairs, the
// mirrored half row, the mirrored row.
__device__ __forceinline__ float row16_sum(float x) {
  x = dpp_add<0xB1>(x);
  x = dpp_add<0x4E>(x);
  x = dpp_add<0x141>(x);
  return dpp_add<0x140>(x);
}

__device__ __forceinline__ float exp2_or_zero(float x) { return x == -INFINITY ? 0.f : exp2f(x); }

// Merge stream (m2, l2, o2) into (m, l, o) for one head.
__device__ __forceinline__ void merge(float &m, float &l, float (&o)[8], float m2, float l2,
                                      const float (&o2)[8]) {
  const float M = fmaxf(m, m2);
  const float a = M == -INFINITY ? 0.f : exp2_or_zero(m - M);
  const float b = M == -INFINITY ? 0.f : exp2_or_zero(m2 - M);
  l = l * a + l2 * b;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = o[i] * a + o2[i] * b;
  m = M;
}

__global__ __launch_bounds__(256, 2) void attn_split_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, const int32_t *__restrict__ kv_start, int B, int Hkv,
    int tile, const int32_t *__restrict__ tasks, int n_tasks,
    const int32_t *__restrict__ worker_begin, Partial part) {
  __shared__ float mls[4][2][G];       // per wavefront: m, l of the 8 heads
  __shared__ float os[4][G][D];        // per wavefront: unnormalised output
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane >> 4, c = lane & 15;          // token row of a step, dim chunk
  const int total = kv_start[B];
  const float qscale = 1.4426950408889634f / sqrtf((float)D);   // log2(e) / sqrt(d)
  // a worker's task range, clamped to the plan's tasks
  const int t_beg = max(worker_begin[blockIdx.x], 0);
  const int t_end = min(worker_begin[blockIdx.x + 1], n_tasks);
  for (int t = t_beg; t < t_end; ++t) {
    const int b = __builtin_amdgcn_readfirstlane(tasks[4 * t]);
    const int h = __builtin_amdgcn_readfirstlane(tasks[4 * t + 1]);
    const int t0 = __builtin_amdgcn_readfirstlane(tasks[4 * t + 2]);
    const int t1 = __builtin_amdgcn_readfirstlane(tasks[4 * t + 3]);
    // a task naming a request or KV head outside this call, or no tiles, is
    // an empty split: kv_start is read only for a request of this call
    const bool valid = b >= 0 && b < B && h >= 0 && h < Hkv && t0 >= 0 && t1 > t0;
    const int base = valid ? kv_start[b] : 0, L = valid ? kv_start[b + 1] - base : 0;
    const int64_t s64 = (int64_t)t0 * tile, e64 = min((int64_t)t1 * tile, (int64_t)L);
    const int s = base + (int)min(s64, (int64_t)L);       // first token of the split
    const int e = base + (int)e64;                        // end (> s for a plan of these lengths)
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
    // the lane's 8 dims of the 8 query heads, in log2 units
    float qv[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint4 u = *reinterpret_cast<const uint4 *>(q + ((size_t)b * (G * Hkv) + G * h + g) * D + 8 * c);
      bf16x8_to_f32(u, qv[g]);
#pragma unroll
      for (int i = 0; i < 8; ++i) qv[g][i] *= qscale;
    }
    float m[G], l[G], o[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) o[g][i] = 0.f;
    }
    const uint16_t *kh = k + (size_t)h * total * D + 8 * c;
    const uint16_t *vh = v + (size_t)h * total * D + 8 * c;
    // Two register sets: the next chunk's keys and values are in flight while
    // the current chunk is multiplied.  Tokens past e re-read token e - 1
    // (in bounds) and are masked.
    auto load = [&](uint4 (&ku)[STEPS], uint4 (&vu)[STEPS], int cb) {
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        const int tok = min(cb + wave * 4 * STEPS + 4 * i + row, e - 1);
        ku[i] = *reinterpret_cast<const uint4 *>(kh + (size_t)tok * D);
        vu[i] = *reinterpret_cast<const uint4 *>(vh + (size_t)tok * D);
      }
    };
    auto compute = [&](const uint4 (&ku)[STEPS], const uint4 (&vu)[STEPS], int cb) {
      float sc[STEPS][G];
#pragma unroll
      for (int i = 0; i < STEPS; ++i) {
        const bool ok = cb + wave * 4 * STEPS + 4 * i + row < e;
        float kf[8];
        bf16x8_to_f32(ku[i], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) acc = fmaf(qv[g][j], kf[j], acc);
          acc = row16_sum(acc);
          sc[i][g] = ok ? acc : -INFINITY;
        }
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mb = sc[0][g];
#pragma unroll
        for (int i = 1; i < STEPS; ++i) mb = fmaxf(mb, sc[i][g]);
        const float mn = fmaxf(m[g], mb);
        const float a = mn == -INFINITY ? 1.f : exp2_or_zero(m[g] - mn);
        float p[STEPS], ps = 0.f;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          p[i] = mn == -INFINITY ? 0.f : exp2_or_zero(sc[i][g] - mn);
          ps += p[i];
        }
        l[g] = l[g] * a + ps;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[g][j] *= a;
#pragma unroll
        for (int i = 0; i < STEPS; ++i) {
          float vf[8];
          bf16x8_to_f32(vu[i], vf);
#pragma unroll
          for (int j = 0; j < 8; ++j) o[g][j] = fmaf(p[i], vf[j], o[g][j]);
        }
        m[g] = mn;
      }
    };
    uint4 kA[STEPS], vA[STEPS], kB[STEPS], vB[STEPS];
    load(kA, vA, s);
    for (int cb = s; cb < e; cb += 2 * CHUNK) {
      load(kB, vB, cb + CHUNK);
      compute(kA, vA, cb);
      if (cb + CHUNK >= e) break;
      load(kA, vA, cb + 2 * CHUNK);
      compute(kB, vB, cb + CHUNK);
    }
    // merge the 4 row streams of the wavefront (lanes c, 16 + c, 32 + c, 48 + c)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float m2 = __shfl_xor(m[g], off, 64), l2 = __shfl_xor(l[g], off, 64);
        float o2[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o2[j] = __shfl_xor(o[g][j], off, 64);
        merge(m[g], l[g], o[g], m2, l2, o2);
      }
    }
    if (lane < 16) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int j = 0; j < 8; ++j) os[wave][g][8 * c + j] = o[g][j];
        if (c == 0) {
          mls[wave][0][g] = m[g];
          mls[wave][1][g] = l[g];
        }
      }
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
    hipLaunchKernelGGL(attn_split_kernel, dim3(n_workers), dim3(256), 0, s,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k),
                       static_cast<const uint16_t *>(v), kv_start, B, n_kv_heads, tile, tasks,
                       (int)n_tasks, worker_begin, part);
  if (hipGetLastError() != hipSuccess) return HY3ATTN_ERR_HIP;
  hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)((int64_t)B * n_kv_heads * G)), dim3(256), 0,
                     s, row_begin, (int)n_tasks, part, n_kv_heads, static_cast<uint16_t *>(out));
  return hipGetLastError() == hipSuccess ? HY3ATTN_OK : HY3ATTN_ERR_HIP;
}
