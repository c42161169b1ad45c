// Grouped expert GEMMs for many rows per expert (prefill): bf16/fp32 MFMA,
// LDS double buffering, one workgroup per (row tile, column tile).
//
// Gate-up (FusedMoE chain, Hy3 Preview inference case section 3: the gate-up
// GEMM reads the original input rows through the route index, with no
// explicit gather pass):  for group g and expert-major rows r,
//     a = x[sorted_token[r]]   (gathered while the tile is loaded)
//     h[r][c] = silu(a . W_gate[g][c]) * (a . W_up[g][c])
// The B tile holds 64 gate rows and the same 64 up rows, interleaved by 32,
// so each wavefront ends up with the gate and up accumulators of the same
// columns in the same lanes and applies SwiGLU in registers.
//
// Down ("written compactly per expert so that accesses stay sequential"):
//     y[r][n] = h[r] . W_down[g][n]
// h rows of one group are contiguous, so the row operand is a plain stripe.
//
// Tile: 128 weight rows x 128 token rows x 128 bytes of K per stage, 4
// wavefronts in 2 x 2, each owning a 64 x 64 block (4 x 4 MFMA tiles of
// 16 x 16).  The weight rows are the MFMA A operand and the token rows the B
// operand, so each lane ends with 4 consecutive output columns of one row.
// Group E is the shared expert (its own weight pointers and width I_shared).
//
// MXFP4 weights (F4): each thread loads the 4 code bytes (8 E2M1 weights) of
// its chunk and the E8M0 scale of the 32-weight block it lies in, and
// decodes them with the scale exactly to 8 bf16 before the LDS write.
//
// FP8 E4M3 weights (F8): each thread loads the 8 code bytes of its chunk,
// decodes them exactly to 8 bf16 before the LDS write, and the per-matrix
// scale multiplies the accumulators in the epilogue; the rest is unchanged.
#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

constexpr int BR = 128;          // weight rows per tile
constexpr int BT = 128;          // token rows per tile (== TILED_ROWS)
constexpr int KB = 128;          // bytes of K per stage (8 chunks of 16 B)
constexpr int CHUNKS = KB / 16;  // 8

__device__ __forceinline__ int swz(int row, int chunk) { return row * CHUNKS + (chunk ^ (row & 7)); }

// BRANCH names the instantiation only (0: routed experts or every group, 1:
// the shared expert's own launches).
template <typename T, bool GATE_UP, int WF, int BRANCH>
__global__ __launch_bounds__(256, 2) void expert_tiled_kernel(ExpertArgs a, int n_col_tiles) {
  constexpr bool F8 = WF == WF_FP8, F4 = WF == WF_MXFP4;
  __shared__ uint4 lds[2][(BR + BT) * CHUNKS];   // 2 x 32 KB

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tbase, n_tiles;   // this launch's slice of the tile list (grp_sel)
  tile_slice(a, a.tiles, tbase, n_tiles);
  a.tiles += 2 * tbase;
  const int tile = blockIdx.x / n_col_tiles;
  const int ct = blockIdx.x % n_col_tiles;
  if (tile >= n_tiles) return;

  const int g = a.tiles[2 * tile];
  const int row0 = a.tiles[2 * tile + 1];           // first expert-major row of the tile
  const int grp_end = a.offsets[g + 1];
  const bool shared = (g == a.E);
  const int Ig = shared ? a.I_shared : a.I;
  const int Kdim = GATE_UP ? a.H : Ig;               // reduction length (elements)
  constexpr int EB = Elem<T>::kBytes;
  constexpr int EPC = Elem<T>::kPerChunk;
  constexpr int WCH = F4 ? 4 : (F8 ? 8 : 16);        // weight bytes per 16-byte LDS chunk
  // bytes of a weight row of K elements
  auto rowb = [](int K) { return F4 ? (size_t)K / 2 : (size_t)K * (F8 ? 1 : EB); };

  // Columns of this tile.
  const int col0 = ct * (GATE_UP ? TILED_GU_COLS : TILED_DN_COLS);
  if (GATE_UP && col0 >= Ig) return;

  // ---- per-thread load descriptors: 4 weight rows + 4 token rows, 1 chunk each ----
  const int lrow = tid >> 3, lch = tid & 7;     // row 0..31 within a pass, chunk 0..7
  const char *wptr[4];
  const char *xptr[4];
  const uint8_t *sptr[4];   // MXFP4: scale byte of the chunk's block at stage 0
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = p * 32 + lrow;   // LDS weight row 0..127
    const char *base;
    int wr;                        // weight row
    const uint8_t *sbase = nullptr;
    if (GATE_UP) {
      const int half = r >> 6, rr = r & 63;
      const bool up = rr >= 32;
      wr = col0 + half * 32 + (rr & 31);
      base = shared ? static_cast<const char *>(up ? a.ws1 : a.ws0)
                    : static_cast<const char *>(up ? a.w1 : a.w0) + (size_t)g * a.I * rowb(a.H);
      if (F4) sbase = shared ? (up ? a.mxs1 : a.mxs0)
                             : (up ? a.mx1 : a.mx0) + (size_t)g * a.I * (a.H / 32);
    } else {
      base = shared ? static_cast<const char *>(a.ws0)
                    : static_cast<const char *>(a.w0) + (size_t)g * a.H * rowb(a.I);
      wr = (col0 + r < a.H) ? col0 + r : col0;   // column tail: reload a valid row
      if (F4) sbase = shared ? a.mxs0 : a.mx0 + (size_t)g * a.H * (a.I / 32);
    }
    wptr[p] = base + (size_t)wr * rowb(Kdim) + lch * WCH;
    // the chunk's K values lch * 8 + [0, 8) lie in block lch / 4 of a stage
    if (F4) sptr[p] = sbase + (size_t)wr * (Kdim / 32) + (lch >> 2);

    int trow = row0 + r;                       // expert-major row of this token slot
    if (trow >= grp_end) trow = row0;          // ragged tail: reload a valid row
    const T *act = static_cast<const T *>(a.act);
    size_t arow;
    if (GATE_UP) arow = (size_t)a.sorted_token[trow] * a.H;
    else arow = (size_t)trow * a.ldh;
    xptr[p] = reinterpret_cast<const char *>(act + arow) + lch * 16;
  }

  uint4 wreg[4], xreg[4];
  uint2 wq[4];                     // FP8: the chunk's 8 code bytes
  uint32_t wq4[4], ws4[4];         // MXFP4: the chunk's 4 code bytes and its scale code
  // kbyte: byte offset of the stage in a bf16 (or fp32) row; FP8 weight rows
  // advance by half of it.
#define HY3_GLOAD(kbyte)                                                   \
  _Pragma("unroll") for (int p = 0; p < 4; ++p) {                          \
    if constexpr (F4) {                                                    \
      wq4[p] = *reinterpret_cast<const uint32_t *>(wptr[p] + (kbyte) / 4); \
      ws4[p] = sptr[p][(kbyte) / 64];                                      \
    } else if constexpr (F8)                                               \
      wq[p] = *reinterpret_cast<const uint2 *>(wptr[p] + (kbyte) / 2);     \
    else wreg[p] = *reinterpret_cast<const uint4 *>(wptr[p] + (kbyte));    \
    xreg[p] = *reinterpret_cast<const uint4 *>(xptr[p] + (kbyte));         \
  }
#define HY3_LSTORE(buf)                                                    \
  _Pragma("unroll") for (int p = 0; p < 4; ++p) {                          \
    const int r = p * 32 + lrow;                                           \
    if constexpr (F4)                                                      \
      lds[buf][swz(r, lch)] = fp4x8_to_bf16(wq4[p], e8m0_to_f32(ws4[p]));  \
    else if constexpr (F8) lds[buf][swz(r, lch)] = e4m3x8_to_bf16(wq[p]);  \
    else lds[buf][swz(r, lch)] = wreg[p];                                  \
    lds[buf][BR * CHUNKS + swz(r, lch)] = xreg[p];                         \
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int wr_ = wave >> 1;      // weight-row block of this wavefront (0/1)
  const int wt_ = wave & 1;       // token-row block (0/1)
  const int r16 = lane & 15, cg = lane >> 4;
  const int nk = Kdim * EB / KB;

  HY3_GLOAD(0);
  HY3_LSTORE(0);
  __syncthreads();
  int cur = 0;
  for (int ks = 0; ks < nk; ++ks) {
    // Prefetch the next stage; the last iteration re-reads stage 0 (in bounds)
    // into the buffer nobody reads again, which keeps the loop branch-free.
    const int knext = (ks + 1 < nk) ? (ks + 1) * KB : 0;
    HY3_GLOAD(knext);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int ch = sub * 4 + cg;
      uint4 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = lds[cur][swz(wr_ * 64 + i * 16 + r16, ch)];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = lds[cur][BR * CHUNKS + swz(wt_ * 64 + j * 16 + r16, ch)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mma<T>::step(acc[i][j], af[i], bfr[j]);
    }
    HY3_LSTORE(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }
#undef HY3_GLOAD
#undef HY3_LSTORE
  (void)EPC;

  // ---- epilogue: lane holds D[weight row 16i + 4cg + q][token row 16j + r16] ----
  T *out = static_cast<T *>(a.out);
  // FP8: scale of the gate (or down) matrix and of the up matrix
  float s0 = 1.0f, s1 = 1.0f, hs = 1.0f;   // hs: activation scale of h (a8)
  if (F8) {
    s0 = shared ? *a.ssc0 : a.sc0[g];
    if (GATE_UP) s1 = shared ? *a.ssc1 : a.sc1[g];
    if (a.a8) {   // the token rows hold E4M3 values of x / xs (gate-up) or h / hs[g]
      const float as = GATE_UP ? *a.xs : a.hs[g];
      s0 *= as;
      s1 *= as;
      hs = a.hs[g];
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int trow = row0 + wt_ * 64 + j * 16 + r16;
    if (trow >= grp_end) continue;
    if (GATE_UP) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // weight rows wr_*64 + 16i + .. are gate cols col0 + 32*wr_ + 16i + ..;
        // rows +32 are the matching up cols.
        const int c = col0 + wr_ * 32 + i * 16 + 4 * cg;
        const f32x4_t gv = acc[i][j] * s0, uv = acc[i + 2][j] * s1;
        if (F8 && a.a8)   // bf16 h quantised with its static scale, stored as bf16 values
          *reinterpret_cast<uint2 *>(out + (size_t)trow * a.ldh + c) = e4m3x4_to_bf16(
              quant_e4m3x4_bf16(swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]),
                                swiglu(gv[2], uv[2]), swiglu(gv[3], uv[3]), hs));
        else
          store4(out + (size_t)trow * a.ldh + c, swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]),
                 swiglu(gv[2], uv[2]), swiglu(gv[3], uv[3]));
      }
    } else {
      // y: fp16 for bf16 layers (float32 for float32 layers)
      typename YElem<T>::type *y = static_cast<typename YElem<T>::type *>(a.out);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = col0 + wr_ * 64 + i * 16 + 4 * cg;
        if (n >= a.H) continue;
        const f32x4_t v = acc[i][j] * s0;
        store4(y + (size_t)trow * a.H + n, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

}  // namespace

template <typename T, int WF, int BRANCH>
static hipError_t launch_tiled_b(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  if (gate_up) {
    const int Imax = a.I > a.I_shared ? a.I : a.I_shared;
    const int nct = Imax / TILED_GU_COLS;
    hipLaunchKernelGGL((expert_tiled_kernel<T, true, WF, BRANCH>), dim3(a.max_tiles * nct), dim3(256),
                       0, stream, a, nct);
  } else {
    const int nct = (a.H + TILED_DN_COLS - 1) / TILED_DN_COLS;
    hipLaunchKernelGGL((expert_tiled_kernel<T, false, WF, BRANCH>), dim3(a.max_tiles * nct), dim3(256),
                       0, stream, a, nct);
  }
  return hipGetLastError();
}

template <typename T, int WF>
static hipError_t launch_tiled(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  return a.grp_sel == GRP_SHARED ? launch_tiled_b<T, WF, 1>(a, gate_up, stream)
                                 : launch_tiled_b<T, WF, 0>(a, gate_up, stream);
}

hipError_t launch_tiled_gate_up(const ExpertArgs &a, int dtype, hipStream_t stream) {
  return dtype == DT_F32 ? launch_tiled<float, WF_DTYPE>(a, true, stream)
         : a.w_fp4       ? launch_tiled<bf16_t, WF_MXFP4>(a, true, stream)
         : a.w_fp8       ? launch_tiled<bf16_t, WF_FP8>(a, true, stream)
                         : launch_tiled<bf16_t, WF_DTYPE>(a, true, stream);
}
hipError_t launch_tiled_down(const ExpertArgs &a, int dtype, hipStream_t stream) {
  return dtype == DT_F32 ? launch_tiled<float, WF_DTYPE>(a, false, stream)
         : a.w_fp4       ? launch_tiled<bf16_t, WF_MXFP4>(a, false, stream)
         : a.w_fp8       ? launch_tiled<bf16_t, WF_FP8>(a, false, stream)
                         : launch_tiled<bf16_t, WF_DTYPE>(a, false, stream);
}

}  // namespace hy3moe
