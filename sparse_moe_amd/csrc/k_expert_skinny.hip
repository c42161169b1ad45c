// Grouped expert GEMMs for few rows per expert (decode): weight streaming.
//
// At small T every routed expert sees one or two token copies, so the
// grouped GEMM has very low arithmetic intensity and is bound by the bytes
// of expert weights read from HBM (Hy3 Preview inference case, section on
// decode parallelism: small-batch MoE grouped GEMM is memory-bound).  This
// path reads every touched weight byte exactly once, straight from global
// memory into MFMA operand registers (no LDS round trip).
//
// Work unit = one wavefront's share of one group (routed expert or the shared
// expert, all of its <= 16*MT rows): 16 gate + 16 up weight rows (gate-up) or
// 32 output rows of W_down (down), over the whole K.  The grid is persistent:
// a fixed number of wavefronts strides over the units counted on the device,
// so no partially filled round of waves is left at the end.  Inside a unit,
// K is streamed in blocks of U 64-byte steps per row with two register sets,
// so one block of loads is in flight while the previous one feeds the MFMAs
// (8 steps = 24 loads per lane per block for one row fragment; fewer steps
// with more row fragments to stay within two wavefronts' registers per SIMD).
// The token rows (gathered through sorted_token for gate-up, contiguous h rows
// for down; padded by reloading a valid row) are the other MFMA operand.
#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

constexpr int UBASE = 8;          // 64-byte K steps per register set (one row fragment)
constexpr int WAVES_PER_SIMD = 2; // persistent grid occupancy

template <typename T, bool GATE_UP, int MT>
__device__ __forceinline__ void stream_unit(const ExpertArgs &a, int tile, int cb, int lane) {
  constexpr int U = UBASE / MT;   // 64-byte K steps per row per register set
  const int g = a.tiles[2 * tile];
  const int row0 = a.tiles[2 * tile + 1];
  const int grp_end = a.offsets[g + 1];
  const bool shared = (g == a.E);
  const int Ig = shared ? a.I_shared : a.I;
  const int Kdim = GATE_UP ? a.H : Ig;
  constexpr int EB = Elem<T>::kBytes;
  const int r16 = lane & 15, cg = lane >> 4;
  const int col0 = cb * (GATE_UP ? 16 : 32);
  if (col0 >= (GATE_UP ? Ig : a.H)) return;

  const char *w0p, *w1p;
  if (GATE_UP) {
    const T *gate = shared ? static_cast<const T *>(a.ws0)
                           : static_cast<const T *>(a.w0) + (size_t)g * a.I * a.H;
    const T *up = shared ? static_cast<const T *>(a.ws1)
                         : static_cast<const T *>(a.w1) + (size_t)g * a.I * a.H;
    w0p = reinterpret_cast<const char *>(gate + (size_t)(col0 + r16) * a.H) + cg * 16;
    w1p = reinterpret_cast<const char *>(up + (size_t)(col0 + r16) * a.H) + cg * 16;
  } else {
    const T *dn = shared ? static_cast<const T *>(a.ws0)
                         : static_cast<const T *>(a.w0) + (size_t)g * a.H * a.I;
    const int n0 = (col0 + r16 < a.H) ? col0 + r16 : col0;
    const int n1 = (col0 + 16 + r16 < a.H) ? col0 + 16 + r16 : col0;
    w0p = reinterpret_cast<const char *>(dn + (size_t)n0 * Ig) + cg * 16;
    w1p = reinterpret_cast<const char *>(dn + (size_t)n1 * Ig) + cg * 16;
  }
  const char *xp[MT];
  const T *act = static_cast<const T *>(a.act);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int trow = row0 + m * 16 + r16;
    if (trow >= grp_end) trow = row0;
    const size_t arow = GATE_UP ? (size_t)a.sorted_token[trow] * a.H : (size_t)trow * a.ldh;
    xp[m] = reinterpret_cast<const char *>(act + arow) + cg * 16;
  }

  f32x4_t acc[2][MT];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsub = Kdim * EB / 64;   // 64-byte steps per row (a multiple of 2)
  uint4 aw0[U], aw1[U], ax[U][MT];
  uint4 bw0[U], bw1[U], bx[U][MT];
#define HY3_LOAD(W0, W1, X, s0)                                                        \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                                      \
    const int o_ = ((s0) + u < nsub ? (s0) + u : nsub - 1) * 64;                       \
    W0[u] = *reinterpret_cast<const uint4 *>(w0p + o_);                                \
    W1[u] = *reinterpret_cast<const uint4 *>(w1p + o_);                                \
    _Pragma("unroll") for (int m = 0; m < MT; ++m)                                     \
        X[u][m] = *reinterpret_cast<const uint4 *>(xp[m] + o_);                        \
  }
#define HY3_MMA(W0, W1, X, s0)                                                         \
  _Pragma("unroll") for (int u = 0; u < U; ++u) {                                      \
    if ((s0) + u < nsub) {                                                             \
      _Pragma("unroll") for (int m = 0; m < MT; ++m) {                                 \
        Mma<T>::step(acc[0][m], W0[u], X[u][m]);                                       \
        Mma<T>::step(acc[1][m], W1[u], X[u][m]);                                       \
      }                                                                                \
    }                                                                                  \
  }
  // Steps past nsub re-read the last step (in bounds) and are not used.
  HY3_LOAD(aw0, aw1, ax, 0);
  for (int s = 0; s < nsub; s += 2 * U) {
    HY3_LOAD(bw0, bw1, bx, s + U);
    __builtin_amdgcn_sched_barrier(0);   // keep the next block's loads ahead
    HY3_MMA(aw0, aw1, ax, s);
    if (s + 2 * U < nsub) { HY3_LOAD(aw0, aw1, ax, s + 2 * U); }
    __builtin_amdgcn_sched_barrier(0);
    HY3_MMA(bw0, bw1, bx, s + U);
  }
#undef HY3_MMA
#undef HY3_LOAD

  // Lane holds D[col 4cg + q][token row 16m + r16].
  T *out = static_cast<T *>(a.out);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int trow = row0 + m * 16 + r16;
    if (trow >= grp_end) continue;
    if (GATE_UP) {
      const f32x4_t gv = acc[0][m], uv = acc[1][m];
      store4(out + (size_t)trow * a.ldh + col0 + 4 * cg, swiglu(gv[0], uv[0]),
             swiglu(gv[1], uv[1]), swiglu(gv[2], uv[2]), swiglu(gv[3], uv[3]));
    } else {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int n = col0 + f * 16 + 4 * cg;
        if (n >= a.H) continue;
        const f32x4_t v = acc[f][m];
        store4(out + (size_t)trow * a.H + n, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

template <typename T, bool GATE_UP, int MT>
__global__ __launch_bounds__(256, WAVES_PER_SIMD) void expert_stream_kernel(ExpertArgs a,
                                                                          int n_col_blocks) {
  const int lane = threadIdx.x & 63;
  // The wavefront index is uniform; readfirstlane makes that visible to the
  // compiler, so every unit-dependent guard below is a scalar branch.  (An
  // MFMA is a whole-wavefront operation: it must never sit under a per-lane
  // EXEC mask that is expected to switch it off.)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = a.tiles[2 * a.max_tiles] * n_col_blocks;
  const int total_waves = gridDim.x * 4;
  // Wavefront ids interleave the XCDs (block b runs on XCD b % 8), so the
  // units of one expert spread over all XCDs and HBM channels.
  for (int u = blockIdx.x * 4 + wave; u < n_units; u += total_waves) {
    const int tile = u / n_col_blocks;
    stream_unit<T, GATE_UP, MT>(a, tile, u - tile * n_col_blocks, lane);
  }
}

// Persistent grid: WAVES_PER_SIMD wavefronts per SIMD on the 256 CUs.
constexpr int STREAM_BLOCKS = 256 * WAVES_PER_SIMD;

template <typename T, int MT>
hipError_t launch_skinny_t(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  if (gate_up) {
    const int Imax = a.I > a.I_shared ? a.I : a.I_shared;
    const int ncb = (Imax + 15) / 16;
    hipLaunchKernelGGL((expert_stream_kernel<T, true, MT>), dim3(STREAM_BLOCKS), dim3(256), 0,
                       stream, a, ncb);
  } else {
    const int ncb = (a.H + 31) / 32;
    hipLaunchKernelGGL((expert_stream_kernel<T, false, MT>), dim3(STREAM_BLOCKS), dim3(256), 0,
                       stream, a, ncb);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_skinny(const ExpertArgs &a, bool gate_up, int T_tokens, hipStream_t stream) {
  if (T_tokens <= 16) return launch_skinny_t<T, 1>(a, gate_up, stream);
  if (T_tokens <= 32) return launch_skinny_t<T, 2>(a, gate_up, stream);
  return launch_skinny_t<T, 4>(a, gate_up, stream);
}

}  // namespace

int skinny_tile_rows(int T) { return T <= 16 ? 16 : (T <= 32 ? 32 : 64); }

hipError_t launch_tiled_gate_up(const ExpertArgs &a, int dtype, hipStream_t stream);
hipError_t launch_tiled_down(const ExpertArgs &a, int dtype, hipStream_t stream);
hipError_t launch_big_gate_up(const ExpertArgs &a, int dtype, hipStream_t stream);
hipError_t launch_big_down(const ExpertArgs &a, int dtype, hipStream_t stream);

hipError_t launch_gate_up(const ExpertArgs &a, int dtype, int T, int path, hipStream_t stream) {
  if (path == PATH_SKINNY)
    return dtype == DT_F32 ? launch_skinny<float>(a, true, T, stream)
                           : launch_skinny<bf16_t>(a, true, T, stream);
  if (path == PATH_BIG) return launch_big_gate_up(a, dtype, stream);
  return launch_tiled_gate_up(a, dtype, stream);
}

hipError_t launch_down(const ExpertArgs &a, int dtype, int T, int path, hipStream_t stream) {
  if (path == PATH_SKINNY)
    return dtype == DT_F32 ? launch_skinny<float>(a, false, T, stream)
                           : launch_skinny<bf16_t>(a, false, T, stream);
  if (path == PATH_BIG) return launch_big_down(a, dtype, stream);
  return launch_tiled_down(a, dtype, stream);
}

}  // namespace hy3moe
