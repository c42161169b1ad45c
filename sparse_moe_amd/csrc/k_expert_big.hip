// Grouped expert GEMMs for many rows per expert (prefill), large tiles.
//
// Same operation as the 128x128 tiled path (gate-up with x rows gathered
// through the route index at load time and SwiGLU in registers; down over the
// contiguous h rows of each expert), laid out for gfx950:
//
//  * 256 weight rows x 256 token rows per workgroup, 8 wavefronts (two per
//    SIMD) in 2 x 4, each owning 128 weight rows x 64 token rows (8 x 4 MFMA
//    16x16x32 tiles, 128 fp32 accumulators per lane).
//  * K is staged 128 bytes per row at a time (64 bf16): one stage is 4M MACs
//    (~2000 MFMA cycles per CU at peak).  Global loads go to one of two
//    register sets two stages ahead; each stage is written to the idle LDS
//    buffer one stage ahead; one barrier per stage.
//    LDS rows use the swizzle chunk ^ (row & 7), which makes the 16-byte
//    operand reads of 8 consecutive rows and the wavefront's writes
//    conflict-free, and every LDS access a base register plus an immediate.
//  * The instruction order of a stage is pinned (see stage_schedule): the
//    global loads go out spread over the whole stage and the LDS writes over
//    its second half, so a load has about a stage and a half to land.
//  * Global addresses are a uniform base per matrix plus 32-bit per-thread
//    offsets.
//  * One workgroup per CU, each looping over tiles.  Consecutive logical
//    tiles run on the same XCD (dispatch is round-robin over the 8 XCDs) with
//    an equal share of the real tiles per XCD, and logical tiles are ordered
//    in bands of 4 row tiles x all column tiles with the row tile fastest: an
//    XCD's 32 tiles in flight share 4 token-row blocks and 8 weight-row blocks
//    in its L2.  The next tile's first two K stages are loaded while the
//    finished tile's epilogue runs.
// Group E is the shared expert (its own weights and width I_shared).
//
// MXFP4 weights (F4): a thread loads the 4 code bytes (8 E2M1 weights) of
// its chunk and the E8M0 scale of the chunk's 32-weight block, and decodes
// them with the scale exactly to 8 bf16 when it writes the chunk to LDS.
//
// FP8 E4M3 weights (F8): a thread loads the 8 code bytes of its weight chunk,
// decodes them exactly to 8 bf16 when it writes the chunk to LDS, and the
// per-matrix scale multiplies the accumulators in the epilogue.
//
// Static FP8 activations (A8, W8A8): both operands are E4M3 bytes, so a
// 128-byte stage row holds 128 K values and one 16x16x128 FP8 MFMA replaces
// the two 16x16x32 bf16 ones of a fragment pair: the LDS layout, the reads
// (chunks c and 4 + c of the lane's row, the same K positions for both
// operands) and the 16-element output fragments stay as they are.  The
// gate-up epilogue quantises h with the group's static scale and stores
// bytes; the down epilogue scales by weight scale x activation scale.
#include <type_traits>

#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

constexpr int BW = 256;          // weight rows per tile
constexpr int BTK = 256;         // token rows per tile (== BIG_ROWS)
constexpr int RB = 128;          // bytes of K per row per stage
constexpr int CH = RB / 16;      // 16-byte chunks per row per stage (8)
constexpr int ROWS = BW + BTK;   // LDS rows per stage
constexpr int BAND = 4;          // row tiles per band of the tile order

// One group of the stage's instruction order: G global loads, 4 MFMAs, R LDS
// operand reads, W LDS writes (scheduling-group masks: 0x020 global reads,
// 0x008 MFMA, 0x100 LDS reads, 0x200 LDS writes).
template <int G, int R, int W>
__device__ __forceinline__ void sched_group() {
  if constexpr (G > 0) __builtin_amdgcn_sched_group_barrier(0x020, G, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  if constexpr (R > 0) __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
  if constexpr (W > 0) __builtin_amdgcn_sched_group_barrier(0x200, W, 0);
}

// Order of one bf16 stage per wavefront: 64 MFMAs in two k-halves of 8 groups
// of 4 (one A fragment against the 4 B fragments), the 24 operand reads two
// groups ahead of their MFMAs (6 at the start of each half), one of the 8
// global loads (stage k + 2) every 8 MFMAs, and the 8 LDS writes (stage k + 1)
// one per group of the second half.  Left to itself the compiler sinks the
// global loads to the end of the stage and hoists the LDS writes that wait
// for the previous loads into the middle of the next stage, which leaves a
// load about half a stage to land.
__device__ __forceinline__ void stage_schedule() {
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
  sched_group<1, 1, 0>(); sched_group<0, 1, 0>(); sched_group<1, 1, 0>(); sched_group<0, 1, 0>();
  sched_group<1, 1, 0>(); sched_group<0, 1, 0>(); sched_group<1, 0, 0>(); sched_group<0, 0, 0>();
  __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
  sched_group<1, 1, 1>(); sched_group<0, 1, 1>(); sched_group<1, 1, 1>(); sched_group<0, 1, 1>();
  sched_group<1, 1, 1>(); sched_group<0, 1, 1>(); sched_group<1, 0, 1>(); sched_group<0, 0, 1>();
}

// A global-memory pointer that is the same in every lane of the wavefront,
// moved to scalar registers (rebuilt as a global-address-space pointer, so
// that loads through it stay global loads).
__device__ __forceinline__ const char *wave_uniform(const char *p) {
  typedef const __attribute__((address_space(1))) char gchar_t;
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char *)(gchar_t *)(((uint64_t)hi << 32) | lo);
}

// A tile of the list: its group, rows and output columns.
struct BigTile {
  int g, row0, grp_end, Ig, col0, nk;
};

// Logical tile r of this XCD's run (see the kernel); false if it is padding.
template <typename T, bool GATE_UP, bool A8>
__device__ __forceinline__ bool big_tile_at(const ExpertArgs &a, int n_tiles, int n_col_tiles,
                                            int per, int xcd, int r, BigTile &t) {
  constexpr int EB = A8 ? 1 : Elem<T>::kBytes;   // bytes per K element of a stage row
  const int band_sz = BAND * n_col_tiles;
  const int L = xcd * per + r;
  const int band = L / band_sz, within = L - band * band_sz;
  const int ct = within / BAND;
  const int rt = band * BAND + (within - ct * BAND);
  if (rt >= n_tiles) return false;
  t.g = a.tiles[2 * rt];
  t.row0 = a.tiles[2 * rt + 1];
  t.grp_end = a.offsets[t.g + 1];
  t.Ig = (t.g == a.E) ? a.I_shared : a.I;
  t.col0 = ct * (GATE_UP ? BW / 2 : BW);
  t.nk = (GATE_UP ? a.H : t.Ig) * EB / RB;
  return !(GATE_UP && t.col0 >= t.Ig);
}

// Load descriptors of tile t: thread loads chunk lc of rows lr + 64 p, p = 0..3,
// of the weight block and of the token block.  Gate-up weight rows: each
// block of 64 rows [64q, 64q+64) holds gate cols col0 + 32q + [0, 32) and then
// the up cols of the same columns, so lr < 32 loads gate rows, lr >= 32 up rows.
// Global addresses: a base pointer plus 32-bit offsets (every matrix < 4 GiB).
template <typename T, bool GATE_UP, int WF, bool A8>
__device__ __forceinline__ void big_tile_loads(const ExpertArgs &a, const BigTile &t, int lr,
                                               int lc, const char *&wb, const char *&xb,
                                               uint32_t *woff, uint32_t *xoff,
                                               const uint8_t *&sb) {
  constexpr bool F8 = WF == WF_FP8, F4 = WF == WF_MXFP4;
  constexpr int EB = A8 ? 1 : Elem<T>::kBytes; // bytes per token-row element
  // bytes of a weight row of K elements, and per 16-byte LDS chunk
  auto rowb = [](int K) { return F4 ? (uint32_t)K / 2 : (uint32_t)K * (F8 ? 1 : Elem<T>::kBytes); };
  constexpr int WCH = F4 ? 4 : ((F8 && !A8) ? 8 : 16);
  const bool shared = (t.g == a.E);
  if (GATE_UP) {
    const bool up = lr >= 32;
    wb = shared ? static_cast<const char *>(up ? a.ws1 : a.ws0)
                : static_cast<const char *>(up ? a.w1 : a.w0) + (size_t)t.g * a.I * rowb(a.H);
    if (F4) sb = shared ? (up ? a.mxs1 : a.mxs0) : (up ? a.mx1 : a.mx0) + (size_t)t.g * a.I * (a.H / 32);
    if constexpr (F4)
      sb = reinterpret_cast<const uint8_t *>(wave_uniform(reinterpret_cast<const char *>(sb)));
    // A wavefront stages 8 consecutive rows lr (lr = tid / 8), all gate or
    // all up: the base is wave-uniform, held in scalar registers for A8.
    if constexpr (A8 || F4) wb = wave_uniform(wb);
    xb = static_cast<const char *>(a.act);
  } else {
    wb = shared ? static_cast<const char *>(a.ws0)
                : static_cast<const char *>(a.w0) + (size_t)t.g * a.H * rowb(a.I);
    if (F4) sb = shared ? a.mxs0 : a.mx0 + (size_t)t.g * a.H * (a.I / 32);
    xb = static_cast<const char *>(a.act) + (size_t)t.row0 * a.ldh * EB;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = p * 64 + lr;
    if (GATE_UP) {
      int wrow = t.col0 + p * 32 + (lr & 31);
      if (wrow >= t.Ig) wrow = t.col0;         // column tail (Ig % 128 == 64)
      woff[p] = (uint32_t)wrow * rowb(a.H) + lc * WCH;
    } else {
      const int wrow = (t.col0 + r < a.H) ? t.col0 + r : t.col0;
      woff[p] = (uint32_t)wrow * rowb(t.Ig) + lc * WCH;
    }
    int trow = t.row0 + r;
    if (trow >= t.grp_end) trow = t.row0;      // ragged tail: reload a valid row
    if (GATE_UP) xoff[p] = (uint32_t)a.sorted_token[trow] * (uint32_t)(a.H * EB) + lc * 16;
    else xoff[p] = (uint32_t)(trow - t.row0) * (uint32_t)(a.ldh * EB) + lc * 16;
  }
}

// A8 gate-up epilogue: h = SwiGLU of the scaled accumulators, rounded to
// bf16 (the layer's activation tensor) and quantised with the group's static
// scale hsc; 128 E4M3 bytes per token row are staged in LDS
// (16-byte chunks swizzled by row) and stored as whole chunks.
__device__ __forceinline__ void big_epilogue_h8(const ExpertArgs &a, const BigTile &t,
                                                const f32x4_t (&acc)[8][4], uint4 *lds, int tid,
                                                float s0, float s1, float hsc) {
  const int lane = tid & 63, wave = tid >> 6;
  const int wr_ = wave >> 2, wt_ = wave & 3, r16 = lane & 15, cg = lane >> 4;
  constexpr int OC = BW / 2 / 16;   // 16-byte chunks per staged row (8)
  char *stg = reinterpret_cast<char *>(lds);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wt_ * 64 + j * 16 + r16;
    char *row = stg + r * OC * 16;
    // fragment pairs as in the bf16 epilogue: gate frag gi, up frag gi + 2
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int gi = (i >> 1) * 4 + (i & 1);
      const int c = wr_ * 64 + (i >> 1) * 32 + (i & 1) * 16 + 4 * cg;
      const f32x4_t gv = acc[gi][j] * s0, uv = acc[gi + 2][j] * s1;
      const uint32_t q = quant_e4m3x4_bf16(swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]),
                                           swiglu(gv[2], uv[2]), swiglu(gv[3], uv[3]), hsc);
      *reinterpret_cast<uint32_t *>(row + (((c >> 4) ^ (r & 7)) << 4) + (c & 15)) = q;
    }
  }
  __syncthreads();
  uint8_t *out = static_cast<uint8_t *>(a.out);
#pragma unroll
  for (int m = 0; m < 256 * OC / 512; ++m) {
    const int q = tid + 512 * m;
    const int r = q / OC, ch = q % OC;
    const int c = t.col0 + ch * 16;
    if (t.row0 + r < t.grp_end && c < t.Ig) {
      const uint4 v = lds[r * OC + (ch ^ (r & 7))];
      uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)(t.row0 + r) * a.ldh + c);
      __builtin_nontemporal_store(v.x, &dst->x);
      __builtin_nontemporal_store(v.y, &dst->y);
      __builtin_nontemporal_store(v.z, &dst->z);
      __builtin_nontemporal_store(v.w, &dst->w);
    }
  }
}

// Epilogue of a tile: lane holds D[weight row 16i + 4cg + q][token row 16j + r16]
// of wavefront (wr_, wt_).  tid is the thread index.
template <typename T, bool GATE_UP, int WF, bool A8>
__device__ __forceinline__ void big_epilogue(const ExpertArgs &a, const BigTile &t,
                                             const f32x4_t (&acc)[8][4], uint4 *lds, int tid) {
  // FP8: scale of the gate (or down) matrix and of the up matrix (A8: times
  // the activation scale of the GEMM's input)
  constexpr bool F8 = WF == WF_FP8;
  float s0 = 1.0f, s1 = 1.0f;
  if (F8) {
    const bool shared = (t.g == a.E);
    s0 = shared ? *a.ssc0 : a.sc0[t.g];
    if (GATE_UP) s1 = shared ? *a.ssc1 : a.sc1[t.g];
  }
  if (A8) {
    const float as = GATE_UP ? *a.xs : a.hs[t.g];
    s0 *= as;
    s1 *= as;
  }
  if constexpr (A8 && GATE_UP) {
    big_epilogue_h8(a, t, acc, lds, tid, s0, s1, a.hs[t.g]);
    return;
  }
  const int lane = tid & 63, wave = tid >> 6;
  const int wr_ = wave >> 2, wt_ = wave & 3, r16 = lane & 15, cg = lane >> 4;
  T *out = static_cast<T *>(a.out);
  if constexpr (sizeof(T) == 2) {
    // Through LDS (free after the loop's last barrier): each lane writes its
    // 4-column pieces into bf16 token rows (16-byte chunks swizzled by row),
    // then each thread stores whole 16-byte chunks, so a wavefront writes two
    // full output rows per instruction instead of 32-byte pieces of 16 rows.
    constexpr int OC = GATE_UP ? BW / 2 / 8 : BW / 8;   // 16-byte chunks per tile row
    char *stg = reinterpret_cast<char *>(lds);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wt_ * 64 + j * 16 + r16;
      char *row = stg + r * OC * 16;
      if (GATE_UP) {
        // wavefront wr_ holds weight rows 128 wr_ + [0, 128): frags i = 0,1 are
        // gate cols 64 wr_ + [0, 32), i = 2,3 their up cols, i = 4,5 gate cols
        // 64 wr_ + [32, 64), i = 6,7 their up cols.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int gi = (i >> 1) * 4 + (i & 1);
          const int c = wr_ * 64 + (i >> 1) * 32 + (i & 1) * 16 + 4 * cg;
          const f32x4_t gv = acc[gi][j] * s0, uv = acc[gi + 2][j] * s1;
          uint2 v;
          v.x = pack_bf16x2(swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]));
          v.y = pack_bf16x2(swiglu(gv[2], uv[2]), swiglu(gv[3], uv[3]));
          *reinterpret_cast<uint2 *>(row + (((c >> 3) ^ (r & 7)) << 4) + (c & 7) * 2) = v;
        }
      } else {
        // y: fp16 (11 significant bits), rounded once more by the combine
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int c = wr_ * 128 + i * 16 + 4 * cg;
          const f32x4_t v4 = acc[i][j] * s0;
          uint2 v;
          v.x = pack_f16x2(v4[0], v4[1]);
          v.y = pack_f16x2(v4[2], v4[3]);
          *reinterpret_cast<uint2 *>(row + (((c >> 3) ^ (r & 7)) << 4) + (c & 7) * 2) = v;
        }
      }
    }
    __syncthreads();
    const int width = GATE_UP ? t.Ig : a.H;           // output columns of this matrix
    const size_t ldo = GATE_UP ? (size_t)a.ldh : (size_t)a.H;
    if constexpr (WF == WF_W4A8 && GATE_UP) {
      // W4A8: the staged bf16 h quantised to MXFP8 per 32 columns.  A row's
      // 16 chunks go to 16 consecutive threads, so the 4 chunks of a block
      // are in 4 adjacent lanes; out receives the codes (rows of ldh bytes)
      // and out_sc the block scales.
      uint8_t *hq = static_cast<uint8_t *>(a.out);
#pragma unroll
      for (int m = 0; m < 256 * OC / 512; ++m) {
        const int q = tid + 512 * m;
        const int r = q / OC, ch = q % OC;
        const int c = t.col0 + ch * 8;
        const uint4 u = lds[r * OC + (ch ^ (r & 7))];
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
        float v[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          v[2 * k] = __uint_as_float(w4[k] << 16);
          v[2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
        }
        uint32_t code;
        const uint2 cq = mxfp8_quant8(v, code);   // all lanes: it exchanges maxima
        if (t.row0 + r < t.grp_end && c < width) {
          uint2 *dst = reinterpret_cast<uint2 *>(hq + (size_t)(t.row0 + r) * ldo + c);
          __builtin_nontemporal_store(cq.x, &dst->x);
          __builtin_nontemporal_store(cq.y, &dst->y);
          if ((tid & 3) == 0)
            a.out_sc[(size_t)(t.row0 + r) * (ldo / 32) + (c >> 5)] = (uint8_t)code;
        }
      }
      return;
    }
#pragma unroll
    for (int m = 0; m < 256 * OC / 512; ++m) {
      const int q = tid + 512 * m;
      const int r = q / OC, ch = q % OC;
      const int c = t.col0 + ch * 8;
      if (t.row0 + r < t.grp_end && c < width) {
        const uint4 v = lds[r * OC + (ch ^ (r & 7))];
        uint4 *dst = reinterpret_cast<uint4 *>(out + (size_t)(t.row0 + r) * ldo + c);
        // written once, read by the next kernel: non-temporal
        __builtin_nontemporal_store(v.x, &dst->x);
        __builtin_nontemporal_store(v.y, &dst->y);
        __builtin_nontemporal_store(v.z, &dst->z);
        __builtin_nontemporal_store(v.w, &dst->w);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int trow = t.row0 + wt_ * 64 + j * 16 + r16;
      if (trow >= t.grp_end) continue;
      if (GATE_UP) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int gi = (i >> 1) * 4 + (i & 1);
          const int c = t.col0 + wr_ * 64 + (i >> 1) * 32 + (i & 1) * 16 + 4 * cg;
          if (c >= t.Ig) continue;
          const f32x4_t gv = acc[gi][j] * s0, uv = acc[gi + 2][j] * s1;
          store4(out + (size_t)trow * a.ldh + c, swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]),
                 swiglu(gv[2], uv[2]), swiglu(gv[3], uv[3]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int n = t.col0 + wr_ * 128 + i * 16 + 4 * cg;
          if (n >= a.H) continue;
          const f32x4_t v = acc[i][j] * s0;
          store4(out + (size_t)trow * a.H + n, v[0], v[1], v[2], v[3]);
        }
      }
    }
  }
}

// LDS form of a staged weight chunk: as loaded, decoded from E4M3 codes, or
// decoded from E2M1 codes with their block's E8M0 scale s (used by MXFP4 only).
__device__ __forceinline__ uint4 weight_chunk(const uint4 &v, uint32_t) { return v; }
__device__ __forceinline__ uint4 weight_chunk(const uint2 &q, uint32_t) { return e4m3x8_to_bf16(q); }
__device__ __forceinline__ uint4 weight_chunk(uint32_t q, uint32_t s) {
  return fp4x8_to_bf16(q, e8m0_to_f32(s));
}

// Order of one A8 stage per wavefront: the 8 B reads and the first A
// fragment's 2 reads up front, then 8 groups, each of: one piece of stage
// k + 1 from registers to LDS, the same registers reloaded with that piece
// of stage k + 2, 4 MFMAs (one A fragment against the 4 B fragments) and
// the next A fragment's 2 reads.  One register set suffices and every load has
// a whole iteration to land.  The next A fragment is read after the MFMAs
// that use the current one, so its registers are reused; the reads land
// while those MFMAs execute.
__device__ __forceinline__ void stage_schedule_a8() {
  __builtin_amdgcn_sched_group_barrier(0x100, 10, 0);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    if (i < 7) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// BRANCH names the instantiation only (0: routed experts or every group, 1:
// the shared expert's own launches), so that profiles list them apart.
template <typename T, bool GATE_UP, int WF, bool A8, int BRANCH>
__global__ __launch_bounds__(512, 1) void expert_big_kernel(ExpertArgs a, int n_col_tiles) {
  constexpr bool F8 = WF == WF_FP8, F4 = WF == WF_MXFP4;
  __shared__ uint4 lds[2 * ROWS * CH];   // 2 x 64 KB

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // XCD-aware order.  Dispatch is round-robin over the 8 XCDs (workgroup b runs
  // on XCD b % 8); each XCD takes a contiguous run of `per` logical tiles
  // (`per` from the device-side tile count, so every XCD gets an equal share of
  // real tiles), and its workgroups walk that run with a stride of their count.
  int tbase, n_tiles;   // this launch's slice of the tile list (grp_sel)
  tile_slice(a, a.tiles, tbase, n_tiles);
  a.tiles += 2 * tbase;
  const int per = ((n_tiles + BAND - 1) / BAND * (BAND * n_col_tiles) + 7) >> 3;
  const int xcd = blockIdx.x & 7, nb = gridDim.x >> 3;
  int r = blockIdx.x >> 3;
  BigTile cur;
  while (r < per && !big_tile_at<T, GATE_UP, A8>(a, n_tiles, n_col_tiles, per, xcd, r, cur))
    r += nb;
  if (r >= per) return;

  const int lr = tid >> 3, lc = tid & 7;
  const char *wb, *xb;
  uint32_t woff[4], xoff[4];
  const uint8_t *sb = nullptr;   // MXFP4: scale bytes of the weight rows
  big_tile_loads<T, GATE_UP, WF, A8>(a, cur, lr, lc, wb, xb, woff, xoff, sb);

  const int wr_ = wave >> 2, wt_ = wave & 3;
  const int r16 = lane & 15, cg = lane >> 4;
  // LDS addresses (uint4 units).  Rows 16i + r16 and 64p + lr have the same
  // swizzle term for every i and p, so each access is a base plus an immediate.
  const int rd_a = (wr_ * 128 + r16) * CH;
  const int rd_b = (BW + wt_ * 64 + r16) * CH;
  const int sw0 = cg ^ (r16 & 7), sw1 = (4 + cg) ^ (r16 & 7);
  const int wr_l = lr * CH + (lc ^ (lr & 7));

  // Two register stage sets: stage s is loaded into set s % 2 at the start of
  // iteration s - 2 and written to LDS at the end of iteration s - 1, so the
  // global latency is covered by two iterations of MFMA work.
  // Weight chunks: 16 bytes, or the 8 E4M3 code bytes of 8 weights (FP8).
  // MXFP4: the 4 code bytes of 8 weights, and their block's scale code.
  typedef typename std::conditional<
      F4, uint32_t, typename std::conditional<F8 && !A8, uint2, uint4>::type>::type wchunk_t;
  wchunk_t aw0, aw1, aw2, aw3, bw0, bw1, bw2, bw3;
  uint32_t as0 = 0, as1 = 0, as2 = 0, as3 = 0, bs0 = 0, bs1 = 0, bs2 = 0, bs3 = 0;
  uint4 ax0, ax1, ax2, ax3;   // set 0
  uint4 bx0, bx1, bx2, bx3;   // set 1
#define HY3_GLOAD(S, kst)                                                              \
  {                                                                                    \
    const uint32_t kb_ = (uint32_t)(kst) * RB;                                         \
    /* weight bytes: W8A16 half, MXFP4 a quarter of the bf16 stage */                 \
    const uint32_t kw_ = F4 ? kb_ / 4 : ((F8 && !A8) ? kb_ / 2 : kb_);                 \
    /* MXFP4: the scale of a chunk is byte woff / 16 of its row's scales (a row  */  \
    /* of K/2 code bytes has K/32 scale bytes; chunk lc holds K lc*8 + [0, 8)) */      \
    if constexpr (F4) {                                                                \
      S##s0 = sb[(woff[0] >> 4) + kb_ / 64]; S##s1 = sb[(woff[1] >> 4) + kb_ / 64];    \
      S##s2 = sb[(woff[2] >> 4) + kb_ / 64]; S##s3 = sb[(woff[3] >> 4) + kb_ / 64];    \
    }                                                                                  \
    S##w0 = *reinterpret_cast<const wchunk_t *>(wb + (kw_ + woff[0]));                 \
    S##w1 = *reinterpret_cast<const wchunk_t *>(wb + (kw_ + woff[1]));                 \
    S##w2 = *reinterpret_cast<const wchunk_t *>(wb + (kw_ + woff[2]));                 \
    S##w3 = *reinterpret_cast<const wchunk_t *>(wb + (kw_ + woff[3]));                 \
    S##x0 = *reinterpret_cast<const uint4 *>(xb + (kb_ + xoff[0]));                    \
    S##x1 = *reinterpret_cast<const uint4 *>(xb + (kb_ + xoff[1]));                    \
    S##x2 = *reinterpret_cast<const uint4 *>(xb + (kb_ + xoff[2]));                    \
    S##x3 = *reinterpret_cast<const uint4 *>(xb + (kb_ + xoff[3]));                    \
  }
#define HY3_LSTORE(S, buf)                                                             \
  {                                                                                    \
    uint4 *d_ = lds + (buf) * ROWS * CH + wr_l;                                        \
    d_[0 * 64 * CH] = weight_chunk(S##w0, S##s0);                                      \
    d_[1 * 64 * CH] = weight_chunk(S##w1, S##s1);                                      \
    d_[2 * 64 * CH] = weight_chunk(S##w2, S##s2);                                      \
    d_[3 * 64 * CH] = weight_chunk(S##w3, S##s3);                                      \
    d_[(BW + 0 * 64) * CH] = S##x0; d_[(BW + 1 * 64) * CH] = S##x1;                    \
    d_[(BW + 2 * 64) * CH] = S##x2; d_[(BW + 3 * 64) * CH] = S##x3;                    \
  }
#define HY3_COMPUTE(buf)                                                               \
  {                                                                                    \
    const uint4 *base_ = lds + (buf) * ROWS * CH;                                      \
    _Pragma("unroll") for (int sub = 0; sub < 2; ++sub) {                              \
      const int swz = sub ? sw1 : sw0;                                                 \
      uint4 bf_[4];                                                                    \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                    \
          bf_[j] = base_[rd_b + j * 16 * CH + swz];                                    \
      _Pragma("unroll") for (int i = 0; i < 8; ++i) {                                  \
        const uint4 af_ = base_[rd_a + i * 16 * CH + swz];                             \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) Mma<T>::step(acc[i][j], af_, bf_[j]); \
      }                                                                                \
    }                                                                                  \
  }
// Iteration k: prefetch stage k+2 into set S (its stage k went to LDS at the
// end of iteration k-1), compute buffer B, write set SN (stage k+1) to the
// other buffer.  Past the end the prefetch re-reads stage 0 and the store
// fills a buffer that is not read again: the body stays branch-free.
#define HY3_ITER(k, S, B, SN)                                                          \
  {                                                                                    \
    HY3_GLOAD(S, ((k) + 2 < cur.nk) ? (k) + 2 : 0);                                        \
    HY3_COMPUTE(B);                                                                    \
    HY3_LSTORE(SN, (B) ^ 1);                                                           \
    if constexpr (sizeof(T) == 2) stage_schedule();                                    \
    __syncthreads();                                                                   \
  }

  // A8: one register set st0..st7 of a stage (weight pieces 0-3, token
  // pieces 4-7), refilled piece by piece as it is written to LDS (see
  // stage_schedule_a8).  Named variables, not an array: an array indexed
  // across the unrolled groups is left in scratch memory.
  uint4 st0, st1, st2, st3, st4, st5, st6, st7;
#define HY3_A8_LOAD(p, kst)                                                            \
  st##p = *reinterpret_cast<const uint4 *>(((p) < 4 ? wb : xb) +                      \
                                           ((uint32_t)(kst) * RB +                     \
                                            ((p) < 4 ? woff[(p) & 3] : xoff[(p) & 3])));
#define HY3_A8_STORE(p, buf)                                                           \
  lds[(buf) * ROWS * CH + wr_l + ((p) < 4 ? (p) * 64 * CH : (BW + ((p) - 4) * 64) * CH)] = st##p;
#define HY3_A8_LOAD_ALL(kst)                                                           \
  HY3_A8_LOAD(0, kst) HY3_A8_LOAD(1, kst) HY3_A8_LOAD(2, kst) HY3_A8_LOAD(3, kst)       \
  HY3_A8_LOAD(4, kst) HY3_A8_LOAD(5, kst) HY3_A8_LOAD(6, kst) HY3_A8_LOAD(7, kst)
#define HY3_A8_STORE_ALL(buf)                                                          \
  HY3_A8_STORE(0, buf) HY3_A8_STORE(1, buf) HY3_A8_STORE(2, buf) HY3_A8_STORE(3, buf)   \
  HY3_A8_STORE(4, buf) HY3_A8_STORE(5, buf) HY3_A8_STORE(6, buf) HY3_A8_STORE(7, buf)
// Group i of an iteration: piece i of stage k + 1 to LDS, piece i of stage
// k + 2 into its registers, A fragment i against the 4 B fragments, then
// the next A fragment's reads.
#define HY3_A8_GROUP(i, B)                                                             \
  HY3_A8_STORE(i, (B) ^ 1)                                                             \
  HY3_A8_LOAD(i, kn_)                                                                  \
  _Pragma("unroll") for (int j = 0; j < 4; ++j)                                        \
      mma_fp8(acc[i][j], a0_, a1_, b0_[j], b1_[j]);                                    \
  if ((i) < 7) {                                                                       \
    a0_ = base_[rd_a + ((i) + 1) * 16 * CH + sw0];                                     \
    a1_ = base_[rd_a + ((i) + 1) * 16 * CH + sw1];                                     \
  }
// Iteration k: compute buffer B, write stage k + 1 to the other buffer and
// load stage k + 2 (past the end: stage 0 again, written to a buffer that is
// not read any more).
#define HY3_A8_ITER(k, B)                                                              \
  {                                                                                    \
    const uint4 *base_ = lds + (B) * ROWS * CH;                                        \
    const int kn_ = ((k) + 2 < cur.nk) ? (k) + 2 : 0;                                  \
    uint4 b0_[4], b1_[4];                                                              \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                    \
      b0_[j] = base_[rd_b + j * 16 * CH + sw0];                                        \
      b1_[j] = base_[rd_b + j * 16 * CH + sw1];                                        \
    }                                                                                  \
    uint4 a0_ = base_[rd_a + sw0], a1_ = base_[rd_a + sw1];                            \
    HY3_A8_GROUP(0, B) HY3_A8_GROUP(1, B) HY3_A8_GROUP(2, B) HY3_A8_GROUP(3, B)         \
    HY3_A8_GROUP(4, B) HY3_A8_GROUP(5, B) HY3_A8_GROUP(6, B) HY3_A8_GROUP(7, B)         \
    stage_schedule_a8();                                                               \
    __syncthreads();                                                                   \
  }

  if constexpr (A8) {
    HY3_A8_LOAD_ALL(0)
    HY3_A8_STORE_ALL(0)
    HY3_A8_LOAD_ALL((1 < cur.nk) ? 1 : 0)
  } else {
    HY3_GLOAD(a, 0);
    HY3_GLOAD(b, (1 < cur.nk) ? 1 : 0);
    HY3_LSTORE(a, 0);
  }
  __syncthreads();
  f32x4_t acc[8][4];
  // Persistent over this workgroup's tiles.  Between two tiles the next
  // tile's first two K stages are issued before the finished tile's
  // epilogue, so their latency overlaps the epilogue and its stores.
  for (;;) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);
    const int nk = cur.nk;
    int k = 0;
    if constexpr (A8) {
      for (; k + 2 <= nk; k += 2) {
        HY3_A8_ITER(k, 0);
        HY3_A8_ITER(k + 1, 1);
      }
      if (k < nk) HY3_A8_ITER(k, 0);
    } else {
      for (; k + 2 <= nk; k += 2) {
        HY3_ITER(k, a, 0, b);
        HY3_ITER(k + 1, b, 1, a);
      }
      if (k < nk) HY3_ITER(k, a, 0, b);
    }

    BigTile nxt;
    int rn = r + nb;
    while (rn < per && !big_tile_at<T, GATE_UP, A8>(a, n_tiles, n_col_tiles, per, xcd, rn, nxt))
      rn += nb;
    const bool has_next = rn < per;
    // The address arithmetic below uses fresh copies of the thread index, so
    // that the compiler recomputes it per tile instead of hoisting it out of
    // the tile loop and holding it in registers through the main loop.
    if (has_next) {   // the finished tile's load descriptors are free
      int tid_n = tid;
      asm volatile("" : "+v"(tid_n));
      big_tile_loads<T, GATE_UP, WF, A8>(a, nxt, tid_n >> 3, tid_n & 7, wb, xb, woff, xoff, sb);
      if constexpr (A8) {
        HY3_A8_LOAD_ALL(0)
      } else {
        HY3_GLOAD(a, 0);
        HY3_GLOAD(b, (1 < nxt.nk) ? 1 : 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    int tid_e = tid;
    asm volatile("" : "+v"(tid_e));
    big_epilogue<T, GATE_UP, WF, A8>(a, cur, acc, lds, tid_e);
    __builtin_amdgcn_sched_barrier(0);
    if (!has_next) break;
    __syncthreads();   // the epilogue's LDS reads are done
    if constexpr (A8) {
      HY3_A8_STORE_ALL(0)
      HY3_A8_LOAD_ALL((1 < nxt.nk) ? 1 : 0)
    } else {
      HY3_LSTORE(a, 0);
    }
    __syncthreads();
    cur = nxt;
    r = rn;
  }
#undef HY3_A8_ITER
#undef HY3_A8_GROUP
#undef HY3_A8_STORE_ALL
#undef HY3_A8_LOAD_ALL
#undef HY3_A8_STORE
#undef HY3_A8_LOAD
#undef HY3_ITER
#undef HY3_COMPUTE
#undef HY3_LSTORE
#undef HY3_GLOAD

}

// W4A8 tiles (MXFP4 weights x dynamic MXFP8 tokens): block-scaled FP4 x FP8
// MFMAs, 128 K values per stage.  Per stage and buffer the LDS holds the
// 256 weight rows as 64-byte code rows (4 chunks, unswizzled: a wavefront's
// A reads -- chunk g of 16 consecutive rows -- cover 1 KB contiguously),
// the 256 token rows as 128-byte code rows (swizzled as in the A8 tiles),
// and one dword of scales per row (blocks 0..3 of the stage).  With the
// measured layout of the instruction, lane (g, r) takes chunk g of its
// weight row and chunks g and 4 + g of its token row, with scale byte g of
// each row.  Each thread stages 2 weight chunks, 4 token chunks and one
// scale dword per stage, refilled piece by piece as in the A8 tiles.
constexpr int W4_WCH = 4;                 // 16-byte chunks per staged weight row
constexpr int W4_TOK = BW * W4_WCH;       // token region (uint4 units)
constexpr int W4_SC = W4_TOK + BTK * CH;  // scale region: 512 dwords (weights, then tokens)

template <bool GATE_UP, int BRANCH>
__global__ __launch_bounds__(512, 1) void expert_big_w4a8_kernel(ExpertArgs a, int n_col_tiles) {
  __shared__ uint4 lds[2 * ROWS * CH];   // 2 x 64 KB: buffers of 50 KB, and the epilogue's staging
  static_assert(W4_SC + (BW + BTK) / 4 <= ROWS * CH, "W4A8 stage buffer");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int tbase, n_tiles;   // this launch's slice of the tile list (grp_sel)
  tile_slice(a, a.tiles, tbase, n_tiles);
  a.tiles += 2 * tbase;
  const int per = ((n_tiles + BAND - 1) / BAND * (BAND * n_col_tiles) + 7) >> 3;
  const int xcd = blockIdx.x & 7, nb = gridDim.x >> 3;
  int r = blockIdx.x >> 3;
  BigTile cur;
  while (r < per && !big_tile_at<bf16_t, GATE_UP, true>(a, n_tiles, n_col_tiles, per, xcd, r, cur))
    r += nb;
  if (r >= per) return;

  // ---- load descriptors of a tile (recomputed per tile) ----
  const char *wb, *xb;
  const uint8_t *sp;               // this thread's scale row (weight row or token row)
  uint32_t woff[2], xoff[4];
  auto tile_loads = [&](const BigTile &t, int tq) {
    const bool shared = (t.g == a.E);
    const int K = GATE_UP ? a.H : t.Ig;
    const int lrow = tq >> 2;      // weight rows lrow and lrow + 128, chunk tq & 3
    if (GATE_UP) {
      const bool up = (lrow & 63) >= 32;   // the same for both rows; uniform per wavefront
      wb = shared ? static_cast<const char *>(up ? a.ws1 : a.ws0)
                  : static_cast<const char *>(up ? a.w1 : a.w0) + (size_t)t.g * a.I * (a.H / 2);
    } else {
      wb = shared ? static_cast<const char *>(a.ws0)
                  : static_cast<const char *>(a.w0) + (size_t)t.g * a.H * (a.I / 2);
    }
    wb = wave_uniform(wb);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int row = lrow + 128 * p;
      int wrow;
      if (GATE_UP) {
        wrow = t.col0 + (row >> 6) * 32 + (row & 31);
        if (wrow >= t.Ig) wrow = t.col0;
      } else {
        wrow = (t.col0 + row < a.H) ? t.col0 + row : t.col0;
      }
      woff[p] = (uint32_t)wrow * (uint32_t)(K / 2) + (tq & 3) * 16;
    }
    const int lr = tq >> 3, lc = tq & 7;
    xb = static_cast<const char *>(a.act) + (GATE_UP ? 0 : (size_t)t.row0 * a.ldh);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      int trow = t.row0 + p * 64 + lr;
      if (trow >= t.grp_end) trow = t.row0;
      xoff[p] = GATE_UP ? (uint32_t)a.sorted_token[trow] * (uint32_t)a.H + lc * 16
                        : (uint32_t)(trow - t.row0) * (uint32_t)a.ldh + lc * 16;
    }
    // scale dword: threads 0..255 the weight row tq, threads 256..511 token row tq - 256
    if (tq < 256) {
      const int row = tq;
      int wrow;
      const uint8_t *sb;
      if (GATE_UP) {
        const bool up = (row & 63) >= 32;
        sb = shared ? (up ? a.mxs1 : a.mxs0) : (up ? a.mx1 : a.mx0) + (size_t)t.g * a.I * (a.H / 32);
        wrow = t.col0 + (row >> 6) * 32 + (row & 31);
        if (wrow >= t.Ig) wrow = t.col0;
      } else {
        sb = shared ? a.mxs0 : a.mx0 + (size_t)t.g * a.H * (a.I / 32);
        wrow = (t.col0 + row < a.H) ? t.col0 + row : t.col0;
      }
      sp = sb + (size_t)wrow * (K / 32);
    } else {
      int trow = t.row0 + (tq - 256);
      if (trow >= t.grp_end) trow = t.row0;
      sp = a.act_sc + (GATE_UP ? (size_t)a.sorted_token[trow] * (a.H / 32)
                               : (size_t)trow * (a.ldh / 32));
    }
  };
  tile_loads(cur, tid);

  const int wr_ = wave >> 2, wt_ = wave & 3;
  const int r16 = lane & 15, cg = lane >> 4;
  const int rd_a = (wr_ * 128 + r16) * W4_WCH + cg;                // + 16 i * W4_WCH per fragment
  const int rd_b = W4_TOK + (wt_ * 64 + r16) * CH;                 // token rows, as in the A8 tiles
  const int sw0 = cg ^ (r16 & 7), sw1 = (4 + cg) ^ (r16 & 7);
  const int rs_a = (W4_SC * 16) + (wr_ * 128 + r16) * 4 + cg;      // scale bytes (byte offsets)
  const int rs_b = (W4_SC * 16) + (BW + wt_ * 64 + r16) * 4 + cg;
  const int lr = tid >> 3, lc = tid & 7;
  const int wl0 = (tid >> 2) * W4_WCH + (tid & 3);                 // weight chunk slots
  const int wl1 = ((tid >> 2) + 128) * W4_WCH + (tid & 3);
  const int xl = W4_TOK + lr * CH + (lc ^ (lr & 7));               // token chunk slot, + 64 CH per piece

  uint4 st0, st1, st2, st3, st4, st5;
  uint32_t st6;
#define HY3_W4_LOADW(p, kst)                                                           \
  { st##p = *reinterpret_cast<const uint4 *>(wb + ((uint32_t)(kst) * 64 + woff[(p) & 1])); }
#define HY3_W4_LOADX(p, kst)                                                           \
  { st##p = *reinterpret_cast<const uint4 *>(xb + ((uint32_t)(kst) * 128 + xoff[((p) - 2) & 3])); }
#define HY3_W4_LOADS(kst) { st6 = *reinterpret_cast<const uint32_t *>(sp + (kst) * 4); }
#define HY3_W4_STORE(p, buf)                                                           \
  {                                                                                    \
    uint4 *b_ = lds + (buf) * ROWS * CH;                                               \
    if ((p) == 0) b_[wl0] = st0;                                                       \
    else if ((p) == 1) b_[wl1] = st1;                                                  \
    else if ((p) < 6) b_[xl + ((p) - 2) * 64 * CH] = HY3_W4_PIECE(p);                   \
    else reinterpret_cast<uint32_t *>(b_ + W4_SC)[tid] = st6;                          \
  }
#define HY3_W4_PIECE(p) ((p) == 2 ? st2 : (p) == 3 ? st3 : (p) == 4 ? st4 : st5)
#define HY3_W4_LOAD_ALL(kst)                                                           \
  { HY3_W4_LOADW(0, kst) HY3_W4_LOADW(1, kst) HY3_W4_LOADX(2, kst) HY3_W4_LOADX(3, kst) \
    HY3_W4_LOADX(4, kst) HY3_W4_LOADX(5, kst) HY3_W4_LOADS(kst) }
#define HY3_W4_STORE_ALL(buf)                                                          \
  { HY3_W4_STORE(0, buf) HY3_W4_STORE(1, buf) HY3_W4_STORE(2, buf) HY3_W4_STORE(3, buf) \
    HY3_W4_STORE(4, buf) HY3_W4_STORE(5, buf) HY3_W4_STORE(6, buf) }
// Group i: staging piece i (i < 7) of stage k + 1 to LDS and the same piece
// of stage k + 2 into its registers, weight fragment i against the 4 token
// fragments, then the next weight fragment and its scale.
#define HY3_W4_GROUP(i, B)                                                             \
  if ((i) == 0) { HY3_W4_STORE(0, (B) ^ 1) HY3_W4_LOADW(0, kn_) }                      \
  else if ((i) == 1) { HY3_W4_STORE(1, (B) ^ 1) HY3_W4_LOADW(1, kn_) }                 \
  else if ((i) == 2) { HY3_W4_STORE(2, (B) ^ 1) HY3_W4_LOADX(2, kn_) }                 \
  else if ((i) == 3) { HY3_W4_STORE(3, (B) ^ 1) HY3_W4_LOADX(3, kn_) }                 \
  else if ((i) == 4) { HY3_W4_STORE(4, (B) ^ 1) HY3_W4_LOADX(4, kn_) }                 \
  else if ((i) == 5) { HY3_W4_STORE(5, (B) ^ 1) HY3_W4_LOADX(5, kn_) }                 \
  else if ((i) == 6) { HY3_W4_STORE(6, (B) ^ 1) HY3_W4_LOADS(kn_) }                    \
  _Pragma("unroll") for (int j = 0; j < 4; ++j)                                        \
      mma_fp4_fp8(acc[i][j], a_, sa_, b0_[j], b1_[j], sb_[j]);                          \
  if ((i) < 7) {                                                                       \
    a_ = base_[rd_a + ((i) + 1) * 16 * W4_WCH];                                        \
    sa_ = sbase_[rs_a + ((i) + 1) * 16 * 4];                                           \
  }
#define HY3_W4_ITER(k, B)                                                              \
  {                                                                                    \
    const uint4 *base_ = lds + (B) * ROWS * CH;                                        \
    const uint8_t *sbase_ = reinterpret_cast<const uint8_t *>(base_);                  \
    const int kn_ = ((k) + 2 < cur.nk) ? (k) + 2 : 0;                                  \
    uint4 b0_[4], b1_[4];                                                              \
    uint32_t sb_[4];                                                                   \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                    \
      b0_[j] = base_[rd_b + j * 16 * CH + sw0];                                        \
      b1_[j] = base_[rd_b + j * 16 * CH + sw1];                                        \
      sb_[j] = sbase_[rs_b + j * 16 * 4];                                              \
    }                                                                                  \
    uint4 a_ = base_[rd_a];                                                            \
    uint32_t sa_ = sbase_[rs_a];                                                       \
    HY3_W4_GROUP(0, B) HY3_W4_GROUP(1, B) HY3_W4_GROUP(2, B) HY3_W4_GROUP(3, B)         \
    HY3_W4_GROUP(4, B) HY3_W4_GROUP(5, B) HY3_W4_GROUP(6, B) HY3_W4_GROUP(7, B)         \
    __syncthreads();                                                                   \
  }

  HY3_W4_LOAD_ALL(0)
  HY3_W4_STORE_ALL(0)
  HY3_W4_LOAD_ALL((1 < cur.nk) ? 1 : 0)
  __syncthreads();
  f32x4_t acc[8][4];
  for (;;) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);
    const int nk = cur.nk;
    int k = 0;
    for (; k + 2 <= nk; k += 2) {
      HY3_W4_ITER(k, 0);
      HY3_W4_ITER(k + 1, 1);
    }
    if (k < nk) HY3_W4_ITER(k, 0);

    BigTile nxt;
    int rn = r + nb;
    while (rn < per && !big_tile_at<bf16_t, GATE_UP, true>(a, n_tiles, n_col_tiles, per, xcd, rn, nxt))
      rn += nb;
    const bool has_next = rn < per;
    if (has_next) {
      int tid_n = tid;
      asm volatile("" : "+v"(tid_n));
      tile_loads(nxt, tid_n);
      HY3_W4_LOAD_ALL(0)
    }
    __builtin_amdgcn_sched_barrier(0);
    int tid_e = tid;
    asm volatile("" : "+v"(tid_e));
    big_epilogue<bf16_t, GATE_UP, WF_W4A8, false>(a, cur, acc, lds, tid_e);
    __builtin_amdgcn_sched_barrier(0);
    if (!has_next) break;
    __syncthreads();
    HY3_W4_STORE_ALL(0)
    HY3_W4_LOAD_ALL((1 < nxt.nk) ? 1 : 0)
    __syncthreads();
    cur = nxt;
    r = rn;
  }
#undef HY3_W4_ITER
#undef HY3_W4_GROUP
#undef HY3_W4_STORE_ALL
#undef HY3_W4_LOAD_ALL
#undef HY3_W4_PIECE
#undef HY3_W4_STORE
#undef HY3_W4_LOADS
#undef HY3_W4_LOADX
#undef HY3_W4_LOADW
}

template <typename T, int WF, bool A8, int BRANCH>
hipError_t launch_big_b(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  int nct;
  if (gate_up) {
    const int Imax = a.I > a.I_shared ? a.I : a.I_shared;
    nct = (Imax + BW / 2 - 1) / (BW / 2);
  } else {
    nct = (a.H + BW - 1) / BW;
  }
  // Logical tiles: bands of BAND row tiles x nct columns; the grid covers the
  // upper bound of row tiles, padded to a multiple of the 8 XCDs.
  const int bands = (a.max_tiles + BAND - 1) / BAND;
  const long logical = (long)bands * BAND * nct;
  // One workgroup per CU (the LDS of a workgroup fills most of a CU); each
  // walks its XCD's tiles.
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const long cap = n_cu >= 8 ? n_cu / 8 * 8 : 8;
  const long want = (logical + 7) / 8 * 8;
  const dim3 grid((unsigned)(want < cap ? want : cap));
  if constexpr (WF == WF_W4A8) {
    if (gate_up)
      hipLaunchKernelGGL((expert_big_w4a8_kernel<true, BRANCH>), grid, dim3(512), 0, stream, a, nct);
    else
      hipLaunchKernelGGL((expert_big_w4a8_kernel<false, BRANCH>), grid, dim3(512), 0, stream, a, nct);
  } else {
    if (gate_up)
      hipLaunchKernelGGL((expert_big_kernel<T, true, WF, A8, BRANCH>), grid, dim3(512), 0, stream, a, nct);
    else
      hipLaunchKernelGGL((expert_big_kernel<T, false, WF, A8, BRANCH>), grid, dim3(512), 0, stream, a, nct);
  }
  return hipGetLastError();
}

template <typename T, int WF, bool A8>
hipError_t launch_big_t(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  return a.grp_sel == GRP_SHARED ? launch_big_b<T, WF, A8, 1>(a, gate_up, stream)
                                 : launch_big_b<T, WF, A8, 0>(a, gate_up, stream);
}

}  // namespace

hipError_t launch_big_gate_up(const ExpertArgs &a, int dtype, hipStream_t stream) {
  return dtype == DT_F32 ? launch_big_t<float, WF_DTYPE, false>(a, true, stream)
         : a.amx         ? launch_big_t<bf16_t, WF_W4A8, false>(a, true, stream)
         : a.a8          ? launch_big_t<bf16_t, WF_FP8, true>(a, true, stream)
         : a.w_fp4       ? launch_big_t<bf16_t, WF_MXFP4, false>(a, true, stream)
         : a.w_fp8       ? launch_big_t<bf16_t, WF_FP8, false>(a, true, stream)
                         : launch_big_t<bf16_t, WF_DTYPE, false>(a, true, stream);
}
hipError_t launch_big_down(const ExpertArgs &a, int dtype, hipStream_t stream) {
  return dtype == DT_F32 ? launch_big_t<float, WF_DTYPE, false>(a, false, stream)
         : a.amx         ? launch_big_t<bf16_t, WF_W4A8, false>(a, false, stream)
         : a.a8          ? launch_big_t<bf16_t, WF_FP8, true>(a, false, stream)
         : a.w_fp4       ? launch_big_t<bf16_t, WF_MXFP4, false>(a, false, stream)
         : a.w_fp8       ? launch_big_t<bf16_t, WF_FP8, false>(a, false, stream)
                         : launch_big_t<bf16_t, WF_DTYPE, false>(a, false, stream);
}

}  // namespace hy3moe
