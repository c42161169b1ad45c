// Grouped expert GEMMs for few rows per expert (decode): weight streaming.
//
// At small T every routed expert sees one or two token copies, so the
// grouped GEMM has very low arithmetic intensity and is bound by the bytes
// of expert weights read from HBM (Hy3 Preview inference case, section on
// decode parallelism: small-batch MoE grouped GEMM is memory-bound).  This
// path reads every touched weight byte exactly once, straight from global
// memory into MFMA operand registers (no LDS round trip), with many 16-byte
// loads in flight per wavefront.
//
// One workgroup = one group (routed expert or the shared expert) x one
// column block; one tile holds all rows of the group (T <= 16*MT).
// Each wavefront owns 16 gate + 16 up columns (gate-up) or 32 output columns
// (down); the token rows (<= 16*MT, zero-padded by reloading a valid row)
// are the MFMA B operand.  Same operand convention and fused SwiGLU epilogue
// as the tiled path.
#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

constexpr int U = 8;   // 64-byte K steps issued per loop iteration

template <typename T, bool GATE_UP, int MT>
__global__ __launch_bounds__(256) void expert_skinny_kernel(ExpertArgs a, int n_col_blocks) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_tiles = a.tiles[2 * a.max_tiles];
  const int tile = blockIdx.x / n_col_blocks;
  const int cb = blockIdx.x % n_col_blocks;
  if (tile >= n_tiles) return;
  const int g = a.tiles[2 * tile];
  const int row0 = a.tiles[2 * tile + 1];
  const int grp_end = a.offsets[g + 1];
  const bool shared = (g == a.E);
  const int Ig = shared ? a.I_shared : a.I;
  const int Kdim = GATE_UP ? a.H : Ig;
  constexpr int EB = Elem<T>::kBytes;
  const int r16 = lane & 15, cg = lane >> 4;

  int col0;
  if (GATE_UP) {
    col0 = cb * SKINNY_GU_COLS + wave * 16;
    if (col0 >= Ig) return;
  } else {
    col0 = cb * SKINNY_DN_COLS + wave * 32;
    if (col0 >= a.H) return;
  }

  const char *wptr[2];
  if (GATE_UP) {
    const T *gate = shared ? static_cast<const T *>(a.ws0)
                           : static_cast<const T *>(a.w0) + (size_t)g * a.I * a.H;
    const T *up = shared ? static_cast<const T *>(a.ws1)
                         : static_cast<const T *>(a.w1) + (size_t)g * a.I * a.H;
    wptr[0] = reinterpret_cast<const char *>(gate + (size_t)(col0 + r16) * a.H) + cg * 16;
    wptr[1] = reinterpret_cast<const char *>(up + (size_t)(col0 + r16) * a.H) + cg * 16;
  } else {
    const T *dn = shared ? static_cast<const T *>(a.ws0)
                         : static_cast<const T *>(a.w0) + (size_t)g * a.H * a.I;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      int n = col0 + f * 16 + r16;
      if (n >= a.H) n = col0;
      wptr[f] = reinterpret_cast<const char *>(dn + (size_t)n * Ig) + cg * 16;
    }
  }
  const char *xptr[MT];
  const T *act = static_cast<const T *>(a.act);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int trow = row0 + m * 16 + r16;
    if (trow >= grp_end) trow = row0;
    const size_t arow = GATE_UP ? (size_t)a.sorted_token[trow] * a.H : (size_t)trow * a.ldh;
    xptr[m] = reinterpret_cast<const char *>(act + arow) + cg * 16;
  }

  f32x4_t acc[2][MT];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nsub = Kdim * EB / 64;
  int s = 0;
  for (; s + U <= nsub; s += U) {
    uint4 wv[U][2], xv[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int off = (s + u) * 64;
      wv[u][0] = *reinterpret_cast<const uint4 *>(wptr[0] + off);
      wv[u][1] = *reinterpret_cast<const uint4 *>(wptr[1] + off);
#pragma unroll
      for (int m = 0; m < MT; ++m) xv[u][m] = *reinterpret_cast<const uint4 *>(xptr[m] + off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int m = 0; m < MT; ++m) Mma<T>::step(acc[f][m], wv[u][f], xv[u][m]);
  }
  for (; s < nsub; ++s) {
    const int off = s * 64;
    const uint4 w0 = *reinterpret_cast<const uint4 *>(wptr[0] + off);
    const uint4 w1 = *reinterpret_cast<const uint4 *>(wptr[1] + off);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const uint4 xb = *reinterpret_cast<const uint4 *>(xptr[m] + off);
      Mma<T>::step(acc[0][m], w0, xb);
      Mma<T>::step(acc[1][m], w1, xb);
    }
  }

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

template <typename T, int MT>
hipError_t launch_skinny_t(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  if (gate_up) {
    const int Imax = a.I > a.I_shared ? a.I : a.I_shared;
    const int ncb = (Imax + SKINNY_GU_COLS - 1) / SKINNY_GU_COLS;
    hipLaunchKernelGGL((expert_skinny_kernel<T, true, MT>), dim3(a.max_tiles * ncb), dim3(256),
                       0, stream, a, ncb);
  } else {
    const int ncb = (a.H + SKINNY_DN_COLS - 1) / SKINNY_DN_COLS;
    hipLaunchKernelGGL((expert_skinny_kernel<T, false, MT>), dim3(a.max_tiles * ncb), dim3(256),
                       0, stream, a, ncb);
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
