// Token -> expert permutation with a contiguous row range per expert.
//
// Follows the "routing and index preprocessing" stage of the FusedMoE chain
// (Hy3 Preview inference case, section 3 table): blocked counting in on-chip
// shared memory that reserves one contiguous output range per expert.  Here:
//
//  1. hist:    each wavefront counts the experts of one chunk of PERM_CHUNK
//              (token, pick) entries into its own LDS histogram.  Entries with
//              equal expert in a 64-wide step are grouped with a 9-ballot key
//              match, so the lowest lane of each group adds the group size
//              and no LDS atomics are needed.
//  2. scan:    one workgroup sums the chunk histograms per expert (turning them
//              into exclusive per-chunk prefixes), scans the group counts into
//              row offsets (group E = the shared expert, T rows), and writes
//              the row-tile list of the expert GEMMs, largest groups first for
//              the tile-grid paths (group order for the weight-streaming path,
//              whose work units do not depend on the tile order).
//     (Batches with at most four chunks run all three steps in one workgroup.)
//  3. scatter: each wavefront revisits its chunk in entry order and places
//              entry f = t*K + j at row offsets[e] + prefix + rank, where rank
//              counts earlier entries of the same expert.  The order within an
//              expert is therefore ascending (t, j): the permutation is stable
//              and deterministic.  Shared-expert rows are t = 0..T-1.
#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

constexpr int MAXG = 257;   // routed experts (<= 256) + the shared expert

// One wavefront counts the experts of chunk `chunk` into its LDS histogram.
__device__ __forceinline__ void hist_chunk(const int32_t *__restrict__ idx, int N, int chunk,
                                           int lane, int *cnt_w) {
  const int beg = chunk * PERM_CHUNK;
  const int end = min(N, beg + PERM_CHUNK);
  for (int base = beg; base < end; base += 64) {
    const int f = base + lane;
    const bool valid = f < end;
    const int e = valid ? idx[f] : 0;
    const uint64_t m = match_key(e, __ballot(valid));
    const bool leader = valid && ((m & lanemask_lt(lane)) == 0);
    if (leader) cnt_w[e] += __popcll(m);
  }
}

// One wavefront places the entries of chunk `chunk` in entry order; run_w[e]
// holds the next free row of expert e for this chunk.
__device__ __forceinline__ void scatter_chunk(const int32_t *__restrict__ idx, int N, int K,
                                              int chunk, int lane, int *run_w,
                                              int32_t *__restrict__ sorted_token,
                                              int32_t *__restrict__ pos_of) {
  const int beg = chunk * PERM_CHUNK;
  const int end = min(N, beg + PERM_CHUNK);
  for (int base = beg; base < end; base += 64) {
    const int f = base + lane;
    const bool valid = f < end;
    const int e = valid ? idx[f] : 0;
    const uint64_t m = match_key(e, __ballot(valid));
    const uint64_t below = m & lanemask_lt(lane);
    const int r0 = valid ? run_w[e] : 0;
    if (valid) {
      const int pos = r0 + __popcll(below);
      sorted_token[pos] = f / K;
      pos_of[f] = pos;
      if (below == 0) run_w[e] = r0 + __popcll(m);
    }
  }
}

__global__ __launch_bounds__(256) void perm_hist_kernel(const int32_t *__restrict__ idx, int N,
                                                        int E, int nchunks,
                                                        int32_t *__restrict__ hist) {
  __shared__ int cnt[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x * 4 + wave;
  for (int e = lane; e < 256; e += 64) cnt[wave][e] = 0;
  __syncthreads();
  if (chunk < nchunks) hist_chunk(idx, N, chunk, lane, cnt[wave]);
  __syncthreads();
  if (chunk < nchunks)
    for (int e = lane; e < E; e += 64) hist[(size_t)chunk * E + e] = cnt[wave][e];
}

// Exclusive scan of v[0..n) (n <= 1024) in LDS by 256 threads, 4 per thread.
__device__ void block_exclusive_scan(int *v, int n, int *total) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int loc[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = tid * 4 + i;
    loc[i] = (k < n) ? v[k] : 0;
    s += loc[i];
  }
  // inclusive scan of s across the wavefront
  int inc = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(inc, off, 64);
    if (lane >= off) inc += o;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int wbase = 0;
  for (int w = 0; w < wave; ++w) wbase += wsum[w];
  int run = wbase + inc - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = tid * 4 + i;
    if (k < n) v[k] = run;
    run += loc[i];
  }
  if (tid == 255) *total = run;
  __syncthreads();
}

// From per-group row counts cnt[0..E] (LDS, group E = shared expert) write
// counts, offsets and the row-tile list (largest groups first when
// sort_tiles, else in group order; with shared_last the shared expert's
// tiles come after every routed tile, whatever its size) and leave the row
// offsets in off[0..E+1] (LDS).  The list ends with the tile count and the
// count of routed tiles (the tiles before the shared expert's when
// shared_last).  Called by all 256 threads of one block.
__device__ void scan_groups(int *cnt, int *off, int E, int tile_rows, int max_tiles,
                            int sort_tiles, int shared_last, int32_t *__restrict__ counts,
                            int32_t *__restrict__ offsets, int32_t *__restrict__ tiles) {
  __shared__ __attribute__((aligned(16))) int ntile[MAXG + 3];   // padded to whole int4s
  __shared__ int order[MAXG], tstart[MAXG + 1];
  __shared__ int total_rows, total_tiles;
  const int tid = threadIdx.x;
  const int G = E + 1;
  for (int g = tid; g < G; g += 256) off[g] = cnt[g];
  __syncthreads();
  block_exclusive_scan(off, G, &total_rows);
  if (tid == 0) off[G] = total_rows;
  for (int g = tid; g < (G + 3) / 4 * 4; g += 256)
    ntile[g] = g < G ? (cnt[g] + tile_rows - 1) / tile_rows : -1;   // -1: never counted
  __syncthreads();
  // shared_last: the shared expert takes no part in the ranking (-1) and is
  // placed last; its count is restored below
  const int shared_tiles = ntile[E];
  __syncthreads();
  if (shared_last && sort_tiles && tid == 0) ntile[E] = -1;
  __syncthreads();
  // Rank of group g: groups with more tiles, or as many and a lower index.
  // Four counts per LDS read, several reads in flight.
  const int4 *nt4 = reinterpret_cast<const int4 *>(ntile);
  if (!sort_tiles) {
    for (int g = tid; g < G; g += 256) order[g] = g;
  } else for (int g = tid; g < G; g += 256) {
    if (shared_last && g == E) {
      order[E] = E;
      continue;
    }
    const int mine = ntile[g];
    int r = 0;
#pragma unroll 8
    for (int h4 = 0; h4 < (G + 3) / 4; ++h4) {
      const int4 o = nt4[h4];
      const int h = 4 * h4;
      r += (o.x > mine) || (o.x == mine && h < g);
      r += (o.y > mine) || (o.y == mine && h + 1 < g);
      r += (o.z > mine) || (o.z == mine && h + 2 < g);
      r += (o.w > mine) || (o.w == mine && h + 3 < g);
    }
    order[r] = g;
  }
  __syncthreads();
  if (tid == 0) ntile[E] = shared_tiles;
  __syncthreads();
  for (int r = tid; r < G; r += 256) tstart[r] = ntile[order[r]];
  __syncthreads();
  block_exclusive_scan(tstart, G, &total_tiles);
  for (int g = tid; g < G; g += 256) {
    counts[g] = cnt[g];
    offsets[g] = off[g];
  }
  if (tid == 0) offsets[G] = off[G];
  for (int r = tid; r < G; r += 256) {
    const int g = order[r];
    const int n = ntile[g];
    int ts = tstart[r];
    for (int i = 0; i < n && ts < max_tiles; ++i, ++ts) {
      tiles[2 * ts] = g;
      tiles[2 * ts + 1] = off[g] + i * tile_rows;
    }
  }
  if (tid == 0) {
    tiles[2 * max_tiles] = min(total_tiles, max_tiles);
    tiles[2 * max_tiles + 1] = min(shared_last ? total_tiles - shared_tiles : total_tiles, max_tiles);
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void perm_scan_kernel(int32_t *__restrict__ hist, int nchunks,
                                                        int E, int T_shared, int tile_rows,
                                                        int max_tiles, int sort_tiles,
                                                        int shared_last,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ tiles) {
  __shared__ int cnt[MAXG], off[MAXG + 1];
  const int tid = threadIdx.x;
  // Per-expert totals; the chunk histograms become exclusive prefixes.  The
  // counts of 16 chunks are loaded before any of them is rewritten, so there
  // is one memory round trip per 16 chunks rather than per chunk.
  for (int e = tid; e < E; e += 256) {
    int run = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        v[j] = c0 + j < nchunks ? hist[(size_t)(c0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (c0 + j < nchunks) hist[(size_t)(c0 + j) * E + e] = run;
        run += v[j];
      }
    }
    cnt[e] = run;
  }
  if (tid == 0) cnt[E] = T_shared;
  __syncthreads();
  scan_groups(cnt, off, E, tile_rows, max_tiles, sort_tiles, shared_last, counts, offsets, tiles);
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(
    const int32_t *__restrict__ idx, int N, int K, int E, int nchunks,
    const int32_t *__restrict__ hist, const int32_t *__restrict__ offsets, int T_shared,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ pos_of) {
  __shared__ int run[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x * 4 + wave;
  if (chunk < nchunks)
    for (int e = lane; e < E; e += 64) run[wave][e] = offsets[e] + hist[(size_t)chunk * E + e];
  __syncthreads();
  if (chunk < nchunks) scatter_chunk(idx, N, K, chunk, lane, run[wave], sorted_token, pos_of);
  // Shared-expert rows: identity.
  const int gtid = blockIdx.x * blockDim.x + threadIdx.x;
  const int base_sh = offsets[E];
  for (int t = gtid; t < T_shared; t += gridDim.x * blockDim.x) sorted_token[base_sh + t] = t;
}

// Whole permutation in one workgroup when there are at most 4 chunks
// (T*K <= 4 * PERM_CHUNK): one launch instead of three for small batches.
__global__ __launch_bounds__(256) void perm_small_kernel(const int32_t *__restrict__ idx, int N,
                                                         int K, int E, int nchunks, int T_shared,
                                                         int tile_rows, int max_tiles,
                                                         int sort_tiles, int shared_last,
                                                         int32_t *__restrict__ counts,
                                                         int32_t *__restrict__ offsets,
                                                         int32_t *__restrict__ tiles,
                                                         int32_t *__restrict__ sorted_token,
                                                         int32_t *__restrict__ pos_of) {
  __shared__ int cnt[4][256];
  __shared__ int tot[MAXG], off[MAXG + 1];
  __shared__ int32_t idx_s[4 * PERM_CHUNK];   // the picks, read twice below
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = lane; e < 256; e += 64) cnt[wave][e] = 0;
  for (int f = tid; f < N; f += 256) idx_s[f] = idx[f];
  __syncthreads();
  if (wave < nchunks) hist_chunk(idx_s, N, wave, lane, cnt[wave]);
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int run = 0;
    for (int w = 0; w < 4; ++w) {
      const int v = cnt[w][e];
      cnt[w][e] = run;
      run += v;
    }
    tot[e] = run;
  }
  if (tid == 0) tot[E] = T_shared;
  __syncthreads();
  scan_groups(tot, off, E, tile_rows, max_tiles, sort_tiles, shared_last, counts, offsets, tiles);
  for (int e = lane; e < E; e += 64) cnt[wave][e] += off[e];
  __syncthreads();
  if (wave < nchunks) scatter_chunk(idx_s, N, K, wave, lane, cnt[wave], sorted_token, pos_of);
  for (int t = tid; t < T_shared; t += 256) sorted_token[off[E] + t] = t;
}

}  // namespace

hipError_t launch_permute(const PermArgs &a, hipStream_t stream) {
  const int N = a.T * a.K;
  if (a.nchunks <= 4) {
    hipLaunchKernelGGL(perm_small_kernel, dim3(1), dim3(256), 0, stream, a.idx, N, a.K, a.E,
                       a.nchunks, a.T_shared, a.tile_rows, a.max_tiles, a.sort_tiles,
                       a.shared_last, a.counts,
                       a.offsets,
                       a.tiles, a.sorted_token, a.pos_of);
    return hipGetLastError();
  }
  const int blocks = (a.nchunks + 3) / 4;
  hipLaunchKernelGGL(perm_hist_kernel, dim3(blocks), dim3(256), 0, stream, a.idx, N, a.E,
                     a.nchunks, a.hist);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, stream, a.hist, a.nchunks, a.E,
                     a.T_shared, a.tile_rows, a.max_tiles, a.sort_tiles, a.shared_last, a.counts,
                     a.offsets,
                     a.tiles);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3(blocks), dim3(256), 0, stream, a.idx, N, a.K,
                     a.E, a.nchunks, a.hist, a.offsets, a.T_shared, a.sorted_token, a.pos_of);
  return hipGetLastError();
}

namespace {
__global__ __launch_bounds__(256) void shared_meta_kernel(int32_t *__restrict__ tiles,
                                                          int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ sorted_token,
                                                          int T, int N, int E, int tile_rows,
                                                          int max_tiles) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int n_sh = (T + tile_rows - 1) / tile_rows;
  if (i < n_sh) {
    tiles[2 * i] = E;
    tiles[2 * i + 1] = N + i * tile_rows;
  }
  if (i == 0) {
    tiles[2 * max_tiles] = n_sh;
    tiles[2 * max_tiles + 1] = 0;
  }
  if (i <= E) offsets[i] = N;
  if (i == E + 1) offsets[i] = N + T;
  if (i < T) sorted_token[N + i] = i;
}
}  // namespace

hipError_t launch_shared_meta(int32_t *tiles, int32_t *offsets, int32_t *sorted_token, int T,
                              int N, int E, int tile_rows, int max_tiles, hipStream_t stream) {
  const int n = T > E + 2 ? T : E + 2;
  hipLaunchKernelGGL(shared_meta_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, tiles,
                     offsets, sorted_token, T, N, E, tile_rows, max_tiles);
  return hipGetLastError();
}

}  // namespace hy3moe
