// Grouped expert GEMMs for few rows per expert (decode): weight streaming.
//
// At small T every routed expert sees one or two token copies, so the
// grouped GEMM has very low arithmetic intensity and is bound by the bytes
// of expert weights read from HBM (Hy3 Preview inference case, section on
// decode parallelism: small-batch MoE grouped GEMM is memory-bound).  This
// path reads every touched weight byte exactly once, from global memory
// into registers: in the MFMA operand layout itself, or (the grouped loads,
// TR below) in wider row pieces that a per-wavefront LDS buffer turns into
// that layout.
//
// Work unit = one wavefront's share of one 16-row tile of a group (routed
// expert or the shared expert; a group of more rows has several tiles): 16
// gate + 16 up weight rows (gate-up) or 32 output rows of W_down (down), over
// the whole K.  The grid is persistent: a fixed number of wavefronts (fewer
// when that evens out the rounds) strides over the units counted on the
// device.  Inside a unit,
// K is streamed in blocks of U 64-byte steps per row with two register sets,
// so one block of loads is in flight while the previous one feeds the MFMAs
// (for bf16, 8 steps = 24 loads per lane per block; fewer for the formats
// whose steps need more registers, to stay within two wavefronts' registers
// per SIMD).
// The token rows (gathered through sorted_token for gate-up, contiguous h rows
// for down; padded by reloading a valid row) are the other MFMA operand.
//
// FP8 E4M3 weights (one byte per element, one float32 scale per matrix): a
// 64-byte step then holds 64 K values per row.  Lane (r16, g) loads bytes
// [16g, 16g + 16) of the step and decodes them exactly to two bf16 fragments
// (K values 16g + [0, 8) and 16g + [8, 16)), and loads the matching 2 x 16
// bytes of each token row; the two MFMAs of a step pair them up.  The scale
// multiplies the float32 accumulators before SwiGLU / the store.  Half the
// weight bytes per K value is the point: this path is bound by them.
//
// MXFP4 weights (E2M1 codes, two per byte, one E8M0 scale per 32 weights of
// a row): a 64-byte step holds 128 K values.  Lane (r16, g) loads bytes
// [16g, 16g + 16), K values 32g + [0, 32) -- exactly one scale block, whose
// scale byte it also loads -- and decodes them, scale applied, to four bf16
// fragments (v_cvt_scalef32_pk_bf16_fp4, exact); the token rows supply the
// matching 64 bytes, and four MFMAs per weight fragment take a step.
//
// W4A8 (MXFP4 weights, token rows as dynamic MXFP8: E4M3 codes with one E8M0
// scale per 32): one block-scaled v_mfma_f32_16x16x128_f8f6f4 (FP4 A, FP8 B)
// takes a step of a weight fragment -- no decode, and half the token bytes
// of bf16.  Measured operand layout of that instruction with an FP4 A: lane
// group g of A holds 32 FP4 values whose K positions (in B's byte order,
// B lane group g' byte q = position 32g' + q) are two runs of 16:
// 64 (g & 1) + 16 (g >> 1) + [0, 16) and that + 32; and the E8M0 scale in
// lane group c, on either side, covers exactly A lane group c's 32
// positions.  So A lane g takes weight block g of the step (16 contiguous
// bytes, its own scale), and B lane g takes token bytes [16g, 16g + 16) and
// [64 + 16g, 64 + 16g + 16) of the step with token block g's scale.
//
// W8A8 (FP8 weights, static FP8 token rows as E4M3 codes; H, I and I_shared
// multiples of 128): two consecutive 64-byte steps of a weight fragment are
// one v_mfma_f32_16x16x128_f8f6f4 (FP8 x FP8).  Lane (r16, g) supplies bytes
// [16g, 16g + 16) of each of the two steps on both sides (weights and token
// codes), so A and B pair up byte for byte; the weight scale times the
// activation scale multiplies the accumulators.  Half the token bytes of the
// bf16 values, a quarter of the MFMAs, no decode.  The gate-up epilogue
// stores h as E4M3 codes for the down GEMM.
#include <type_traits>

#include "common.cuh"
#include "internal.h"

namespace hy3moe {

namespace {

constexpr int UBASE = 8;          // 64-byte K steps per register set (bf16 weights)
constexpr int WAVES_PER_SIMD = 2; // persistent grid occupancy
// Token rows of a unit: one 16-row MFMA fragment (the tiles of this path hold
// 16 rows).
constexpr int MT = 1;

// 64-byte steps per register set: bf16 weights UBASE; FP8 weights 6 (each
// step also holds two token chunks); W8A8 8 (one chunk of codes per step;
// even, as two steps make one MFMA); MXFP4 3 (four token chunks per step);
// W4A8 4.  With the grouped weight loads (TRG steps per group) a multiple of
// the group: FP8 takes 4 in groups of four, MXFP4 2 in groups of two, or 4
// when its token chunks are read at multiply time (XD, below).
template <int WF, int TRG = 0, bool XD = false>
constexpr int steps_per_set() {
  return TRG == 4 && WF == WF_FP8 ? 4
         : TRG == 2 && WF == WF_MXFP4 ? (XD ? 4 : 2)
         : WF == WF_W8A8  ? 8   // even: pairs of steps
         : WF == WF_FP8   ? 6
         : WF == WF_MXFP4 ? 3
         : WF == WF_W4A8  ? 4
                          : UBASE;
}
// XD: the token chunks of a step are read from the LDS copy of x when the
// step is multiplied, not with its weights one register set ahead.  For
// MXFP4 weights with bf16 tokens (four chunks per step) that frees the
// registers for a second group of grouped loads per set (Hy3 decode
// gate-up 116 -> 109 us); for the other formats, whose steps hold one or
// two chunks, it measured the same or slower.
template <bool XL, int WF>
constexpr bool tokens_at_multiply() { return XL && WF == WF_MXFP4; }
// 16-byte token chunks per 64-byte weight step.
template <int WF>
constexpr int token_chunks() {
  return WF == WF_MXFP4 ? 4 : ((WF == WF_FP8 || WF == WF_W4A8) ? 2 : 1);
}
// Token rows of E4M3 codes (one byte per K value).
template <int WF>
constexpr bool token_codes() { return WF == WF_W4A8 || WF == WF_W8A8; }

// Where a unit's operands are (per lane) and what its epilogue needs.
struct UnitSrc {
  const char *w0p, *w1p;   // the two 16-row weight fragments (gate/up, or two down blocks)
  const char *xp[MT];      // token rows (gathered x for gate-up, h rows for down)
  uint32_t xlo[MT];        // XL: byte offsets of the lane's token chunks in the LDS copy of x
  const uint8_t *s0p, *s1p;  // MXFP4: the lane's scale bytes of the two fragments
  const uint8_t *xsp[MT];    // W4A8: the lane's scale bytes of the token rows
  bool vs;                   // MXFP4, W4A8: scale rows allow 16-byte loads of 4 steps
  int nsub;                // 64-byte K steps per row
  int nf;                  // fragments streamed (2; 1 for half of a down unit)
  int rowb;                // TR: bytes per weight row (the stride of the grouped loads)
};
struct UnitOut {
  int row0, grp_end, col0, nsub, nf;
  float sc0, sc1;          // FP8 weights: scales of fragment 0 / 1's matrix
                           // (times the input's activation scale with a8)
  float hs;                // a8 gate-up: activation scale of the group's h
  uint32_t xlo;            // XD: byte offset of the lane's token chunks in the LDS copy of x
};

// XL (gate-up, where the copy and the wavefronts' buffers fit: T <= 16 for
// bf16 x at H = 4096, about 32 for E4M3 codes): the workgroup copies every
// token row of x into LDS once, and the token operand of each step is read
// from there, so the
// global loads carry only weights (the load path, not HBM, bounded the FP8
// and MXFP4 weights, whose token chunks per weight byte are 2x and 4x
// bf16's).  Rows of the copy are padded by 16 bytes, which spreads the 16
// gathered rows of a wavefront read over the banks.
__host__ __device__ constexpr int x_lds_stride(int row_bytes) { return row_bytes + 16; }

// TR (grouped weight loads; every K row of the launch a multiple of the
// group's 64 TRG bytes): a weight load covers 16 / TRG rows x 64 TRG
// contiguous bytes (TRG = 4: four rows x 256 B; TRG = 2: eight rows x 128 B)
// instead of sixteen rows x 64 bytes, with a non-temporal hint; a streaming
// read in those forms ran ~10 % faster than the MFMA-shaped one at the rows
// of 1.5-4 KB of these GEMMs.  Load j of a group of TRG 64-byte steps holds
// row (16 / TRG) j + l / (4 TRG), bytes [16 (l % 4 TRG), +16) of the group's
// 64 TRG; the wavefront's LDS buffer (1 KB x TRG) turns the group into the
// MFMA layout (step s: row l % 16, bytes [64 s + 16 (l / 16), +16)).  Chunk
// c of row r sits in slot 4 TRG r + (c ^ (r % 4 TRG)), so the passes are
// free of bank conflicts (TRG = 4) or two-way (TRG = 2).  LDS operations of
// one wavefront complete in order; the wavefront-scope fences keep the
// compiler from reordering them across the passes.
__host__ __device__ constexpr int tr_wave_bytes(int trg) { return 1024 * trg; }

__device__ __forceinline__ uint4 load_nt16(const char *p) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int U, int TRG>
__device__ __forceinline__ void transpose_groups(uint4 (&W)[U], uint4 *lb, int lane) {
  static_assert(TRG == 2 || TRG == 4, "groups of two or four steps");
  static_assert(U % TRG == 0, "whole groups per register set");
  constexpr int CPR = 4 * TRG;      // 16-byte chunks per row of a group
  constexpr int RPL = 16 / TRG;     // rows per load
#pragma unroll
  for (int q = 0; q < U / TRG; ++q) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int j = 0; j < TRG; ++j) {
      const int r = RPL * j + lane / CPR, c = lane % CPR;
      lb[CPR * r + (c ^ (r % CPR))] = W[TRG * q + j];
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int st = 0; st < TRG; ++st) {
      const int r = lane & 15, c = 4 * st + (lane >> 4);
      W[TRG * q + st] = lb[CPR * r + (c ^ (r % CPR))];
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Unit u (tile u / n_col_blocks, column block u % n_col_blocks) of this
// kernel; returns false if the column block lies past the group's width.
// half = 1 or 2: only the first or the second 16-row fragment of a down unit.
template <typename T, bool GATE_UP, int WF, bool XL, int TRG>
__device__ __forceinline__ bool unit_of(const ExpertArgs &a, int u, int n_col_blocks, int lane,
                                        UnitSrc &src, UnitOut &o, int half = 0) {
  constexpr bool F8 = WF == WF_FP8 || WF == WF_W8A8, F4 = WF == WF_MXFP4 || WF == WF_W4A8;
  constexpr bool MXA = WF == WF_W4A8, CODES = token_codes<WF>();
  constexpr int EB = Elem<T>::kBytes;
  // bytes per weight row of K elements (MXFP4: half a byte per element)
  auto rowb = [](int K) { return F4 ? K / 2 : K * (F8 ? 1 : EB); };
  const int tile = u / n_col_blocks, cb = u - tile * n_col_blocks;
  // uniform per wavefront (u is); readfirstlane keeps the values, read from
  // LDS, in scalar registers, so the branches on them stay scalar
  const int g = __builtin_amdgcn_readfirstlane(a.tiles[2 * tile]);
  o.row0 = __builtin_amdgcn_readfirstlane(a.tiles[2 * tile + 1]);
  o.grp_end = __builtin_amdgcn_readfirstlane(a.offsets[g + 1]);
  const bool shared = (g == a.E);
  const int Ig = shared ? a.I_shared : a.I;
  o.col0 = cb * (GATE_UP ? 16 : 32) + (half == 2 ? 16 : 0);
  o.nsub = rowb(GATE_UP ? a.H : Ig) / 64;
  o.nf = half ? 1 : 2;
  if (o.col0 >= (GATE_UP ? Ig : a.H)) return false;
  src.nsub = o.nsub;
  src.nf = o.nf;
  const int r16 = lane & 15, cg = lane >> 4;
  if (GATE_UP) {
    const char *gate = shared ? static_cast<const char *>(a.ws0)
                              : static_cast<const char *>(a.w0) + (size_t)g * a.I * rowb(a.H);
    const char *up = shared ? static_cast<const char *>(a.ws1)
                            : static_cast<const char *>(a.w1) + (size_t)g * a.I * rowb(a.H);
    // TR: row l / (4 TRG) of a grouped load, bytes [16 (l % 4 TRG), +16) of
    // the row's 64 TRG
    const int lr = TRG ? lane / (4 * TRG) : r16, lc = TRG ? lane % (4 * TRG) : cg;
    src.w0p = gate + (size_t)(o.col0 + lr) * rowb(a.H) + lc * 16;
    src.w1p = up + (size_t)(o.col0 + lr) * rowb(a.H) + lc * 16;
    src.rowb = rowb(a.H);
    if (F4) {   // scale rows of H / 32 bytes; the lane's block is step * 4 + cg
      const int sr = a.H / 32;
      const uint8_t *sg = shared ? a.mxs0 : a.mx0 + (size_t)g * a.I * sr;
      const uint8_t *su = shared ? a.mxs1 : a.mx1 + (size_t)g * a.I * sr;
      src.s0p = sg + (size_t)(o.col0 + r16) * sr + cg;
      src.s1p = su + (size_t)(o.col0 + r16) * sr + cg;
    }
  } else {
    const char *dn = shared ? static_cast<const char *>(a.ws0)
                            : static_cast<const char *>(a.w0) + (size_t)g * a.H * rowb(a.I);
    const int n0 = (o.col0 + r16 < a.H) ? o.col0 + r16 : o.col0;
    const int n1 = (o.col0 + 16 + r16 < a.H) ? o.col0 + 16 + r16 : o.col0;
    if (TRG) {   // H % 64 == 0: the fragments' rows all exist
      src.w0p = dn + (size_t)(o.col0 + lane / (4 * TRG)) * rowb(Ig) + lane % (4 * TRG) * 16;
      src.w1p = src.w0p + (size_t)16 * rowb(Ig);
    } else {
      src.w0p = dn + (size_t)n0 * rowb(Ig) + cg * 16;
      src.w1p = dn + (size_t)n1 * rowb(Ig) + cg * 16;
    }
    src.rowb = rowb(Ig);
    if (F4) {
      const int sr = Ig / 32;
      const uint8_t *sd = shared ? a.mxs0 : a.mx0 + (size_t)g * a.H * (a.I / 32);
      src.s0p = sd + (size_t)n0 * sr + cg;
      src.s1p = sd + (size_t)n1 * sr + cg;
    }
  }
  if (o.nf == 1) {   // one fragment: the second's loads re-read the first (cache hits), so
    src.w1p = src.w0p;   // that the load sequence, and with it the compiler's waits on
    src.s1p = src.s0p;   // the in-order load counter, does not depend on nf
  }
  if (F8) {
    o.sc0 = shared ? *a.ssc0 : a.sc0[g];
    o.sc1 = GATE_UP ? (shared ? *a.ssc1 : a.sc1[g]) : o.sc0;
    if (a.a8) {   // the token rows hold E4M3 values of x / xs (gate-up) or h / hs[g]
      const float as = GATE_UP ? *a.xs : a.hs[g];
      o.sc0 *= as;
      o.sc1 *= as;
      o.hs = a.hs[g];
    }
  }
  const T *act = static_cast<const T *>(a.act);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    int trow = o.row0 + m * 16 + r16;
    if (trow >= o.grp_end) trow = o.row0;
    const size_t arow = GATE_UP ? (size_t)a.sorted_token[trow] * a.H : (size_t)trow * a.ldh;
    // bf16 weights: chunk g of each 64-byte step; FP8: bytes [32g, 32g+32) of
    // each 128-byte step of the token row; MXFP4: bytes [64g, 64g+64) of each
    // 256-byte step (the K values of the lane's codes); W4A8: code bytes
    // [32g, 32g+32) of each 128-byte step, and block scale step * 4 + g
    if (XL)   // the token's row of the LDS copy, the lane's chunk of a step
      o.xlo = src.xlo[m] = (uint32_t)a.sorted_token[trow] * (uint32_t)x_lds_stride(a.H * (CODES ? 1 : EB)) +
                   cg * 16 * (MXA ? 1 : token_chunks<WF>());
    if (WF == WF_W8A8) {   // code bytes [16g, 16g + 16) of each 64-byte step
      src.xp[m] = static_cast<const char *>(a.act) + arow + cg * 16;
    } else if (MXA) {   // bytes [16g, 16g + 16) and [64 + 16g, ...) of each 128-byte step
      src.xp[m] = static_cast<const char *>(a.act) + arow + cg * 16;
      src.xsp[m] = a.act_sc + arow / 32 + cg;
      // K % 512 == 0: weight scale rows of K/32 bytes are 16-byte multiples,
      // and so are the token scale rows (x: K = H; h: rows of ldh / 32)
      src.vs = (o.nsub & 3) == 0 && (GATE_UP || a.ldh % 512 == 0);
    } else if (WF == WF_MXFP4) {
      src.xp[m] = reinterpret_cast<const char *>(act + arow) + cg * 16 * token_chunks<WF>();
      src.vs = (o.nsub & 3) == 0;   // the weight scale rows (K / 32 bytes), as for W4A8
    } else {
      src.xp[m] = reinterpret_cast<const char *>(act + arow) + cg * 16 * token_chunks<WF>();
    }
  }
  return true;
}

// Work item k >= k0 of wavefront w (of nw): item k is unit w + k * nw.  For
// down, when the units left after the full rounds number at most nw / 2, each
// of them is split into its two 16-row fragments for twice as many
// wavefronts, so the last round costs half a unit.  Returns the item index
// (kmax when there is none) and fills src / o.
template <typename T, bool GATE_UP, int WF, bool XL, int TRG>
__device__ __forceinline__ int next_item(const ExpertArgs &a, int k, int w, int nw, int n_units,
                                         int n_col_blocks, int lane, UnitSrc &src,
                                         UnitOut &o) {
  const int full = n_units / nw, tail = n_units - full * nw;
  const bool split = !GATE_UP && 2 * tail <= nw;
  const int kmax = full + 1;
  for (; k < kmax; ++k) {
    if (k < full || !split) {
      const int u = w + k * nw;
      if (u >= n_units) return kmax;
      if (unit_of<T, GATE_UP, WF, XL, TRG>(a, u, n_col_blocks, lane, src, o)) return k;
    } else {
      if (w >= 2 * tail) return kmax;
      if (unit_of<T, GATE_UP, WF, XL, TRG>(a, full * nw + (w >> 1), n_col_blocks, lane, src, o,
                                      1 + (w & 1)))
        return k;
    }
  }
  return kmax;
}

template <typename T, bool GATE_UP, int WF>
__device__ __forceinline__ void unit_epilogue(const ExpertArgs &a, const UnitOut &o,
                                              f32x4_t (&acc)[2][MT], int lane) {
  constexpr bool F8 = WF == WF_FP8 || WF == WF_W8A8;
  const float s0 = F8 ? o.sc0 : 1.0f, s1 = F8 ? o.sc1 : 1.0f;
  const int r16 = lane & 15, cg = lane >> 4;
  // Lane holds D[col 4cg + q][token row 16m + r16].
  T *out = static_cast<T *>(a.out);
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int trow = o.row0 + m * 16 + r16;
    if (trow >= o.grp_end) continue;
    if (GATE_UP) {
      const f32x4_t gv = acc[0][m] * s0, uv = acc[1][m] * s1;
      T *dst = out + (size_t)trow * a.ldh + o.col0 + 4 * cg;
      if (WF == WF_W8A8)   // bf16 h quantised with its static scale: 4 code bytes
        *reinterpret_cast<uint32_t *>(static_cast<uint8_t *>(a.out) + (size_t)trow * a.ldh +
                                      o.col0 + 4 * cg) =
            quant_e4m3x4_bf16(swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]), swiglu(gv[2], uv[2]),
                              swiglu(gv[3], uv[3]), o.hs);
      else if (F8 && a.a8)   // bf16 h quantised with its static scale, stored as bf16 values
        *reinterpret_cast<uint2 *>(dst) = e4m3x4_to_bf16(
            quant_e4m3x4_bf16(swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]), swiglu(gv[2], uv[2]),
                              swiglu(gv[3], uv[3]), o.hs));
      else
        store4(dst, swiglu(gv[0], uv[0]), swiglu(gv[1], uv[1]), swiglu(gv[2], uv[2]),
               swiglu(gv[3], uv[3]));
    } else {
      // y: fp16 for bf16 layers (float32 for float32 layers)
      typename YElem<T>::type *y = static_cast<typename YElem<T>::type *>(a.out);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int n = o.col0 + f * 16 + 4 * cg;
        if (f >= o.nf || n >= a.H) continue;
        const f32x4_t v = acc[f][m] * (f ? s1 : s0);
        store4(y + (size_t)trow * a.H + n, v[0], v[1], v[2], v[3]);
      }
    }
  }
}

// Floats of the per-group scales a workgroup stages (FP8 weights; reserved
// for every format).
__host__ __device__ constexpr int scale_lds_floats(int E) { return 3 * (E + 1) + 1; }

// LDS bytes of the unit metadata a workgroup stages (see the kernel).
inline size_t meta_lds_bytes(const ExpertArgs &a, bool gate_up) {
  return 4 * ((size_t)2 * a.max_tiles + 2 + a.E + 2 + (gate_up ? a.n_rows : 0) +
              scale_lds_floats(a.E));
}

// Threads per workgroup: 256 (two workgroups per CU), or 512 with the LDS
// copy of x (one per CU holding it), two wavefronts per SIMD either way.
template <bool XL> constexpr int stream_threads() { return XL ? 512 : 256; }

// BRANCH names the instantiation only: 0 for the routed experts (or every
// group), 1 for the shared expert's own launches, which profiles then list
// apart.
template <typename T, bool GATE_UP, int WF, bool XL, int TRG, int BRANCH>
__global__ __launch_bounds__(stream_threads<XL>(), WAVES_PER_SIMD) void expert_stream_kernel(
    ExpertArgs a_in, int n_col_blocks) {
  constexpr bool F8 = WF == WF_FP8, F4 = WF == WF_MXFP4, MXA = WF == WF_W4A8;
  constexpr bool A8C = WF == WF_W8A8, CODES = token_codes<WF>();
  constexpr bool TR = TRG > 0;
  constexpr int NT = stream_threads<XL>(), WPB = NT / 64;
  // The unit metadata -- tile list, group offsets and (gate-up) the sorted
  // token ids -- is staged in LDS once per workgroup, so that the set-up of a
  // wavefront's next unit reads LDS instead of a chain of dependent global
  // loads, which held back the unit's first weight loads at every change.
  // Each thread issues its loads of a round together and then writes them
  // (one memory round trip per round, not one per word or chunk).
  extern __shared__ int32_t meta[];
  const int n_t = 2 * a_in.max_tiles + 2, n_o = a_in.E + 2;
  const int n_m = n_t + n_o + (GATE_UP ? a_in.n_rows : 0);
  constexpr int MB = 4;   // words per thread per round
  for (int base = 0; base < n_m; base += NT * MB) {
    // past the end a thread copies the last word again (no branch: a branch
    // per word would have its load sunk into it)
    int32_t v[MB];
    int at[MB];
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int i = min(base + j * NT + (int)threadIdx.x, n_m - 1);
      // word i of the concatenation: select the array and its first word
      const bool in_t = i < n_t, in_o = i < n_t + n_o;
      const int32_t *arr = in_t ? a_in.tiles : (in_o ? a_in.offsets : a_in.sorted_token);
      const int first = in_t ? 0 : (in_o ? n_t : n_t + n_o);
      v[j] = arr[i - first];
      at[j] = i;
    }
#pragma unroll
    for (int j = 0; j < MB; ++j) meta[at[j]] = v[j];
  }
  // FP8 weights: the scales of every group of this launch (weights, and with
  // a8 the activations) follow, so that a unit's set-up issues no global
  // load: the wavefront would wait there for all of its streaming loads, as
  // the wait counter is in order.  Layout: sc0[E+1] (group E: the shared
  // expert), sc1[E+1], hs[E+1], xs.
  constexpr bool FSC = F8 || A8C;
  const int n_sc = scale_lds_floats(a_in.E);
  float *scl = reinterpret_cast<float *>(meta + n_m);
  if constexpr (FSC) {
    const int E = a_in.E;
    const bool routed = a_in.grp_sel != GRP_SHARED;
    const bool shared = a_in.grp_sel != GRP_ROUTED && a_in.I_shared > 0;
    for (int i = threadIdx.x; i <= E; i += NT) {
      float s0 = 0.f, s1 = 0.f, h = 0.f;
      if (i < E ? routed : shared) {   // pointers of groups outside the launch may be null
        s0 = i < E ? a_in.sc0[i] : *a_in.ssc0;
        if (GATE_UP) s1 = i < E ? a_in.sc1[i] : *a_in.ssc1;
        if (a_in.a8) h = a_in.hs[i];
      }
      scl[i] = s0;
      scl[E + 1 + i] = s1;
      scl[2 * (E + 1) + i] = h;
    }
    if (threadIdx.x == 0) scl[3 * (E + 1)] = a_in.a8 ? *a_in.xs : 0.f;
  }
  // XL: every token row of x, 16-byte chunks, after the metadata (16-byte
  // aligned), XB chunks per thread per round
  const int meta_n = (n_m + n_sc + 3) & ~3;
  const char *xl = reinterpret_cast<const char *>(meta + meta_n);
  if constexpr (XL) {
    const int rb = a_in.H * (CODES ? 1 : Elem<T>::kBytes), cpr = rb / 16;
    const int rs = x_lds_stride(rb);
    const int n_x = a_in.n_tok * cpr;
    char *dst = reinterpret_cast<char *>(meta + meta_n);
    const char *src_x = static_cast<const char *>(a_in.act);
    constexpr int XB = 8;
    for (int base = 0; base < n_x; base += NT * XB) {
      // Past the end a thread copies the last chunk again (the same bytes to
      // the same place): no branch, so the loads are not sunk into one each.
      uint4 v[XB];
      int at[XB];
#pragma unroll
      for (int j = 0; j < XB; ++j) {
        const int i = min(base + j * NT + (int)threadIdx.x, n_x - 1);
        const int t = i / cpr, c = i - t * cpr;
        v[j] = *reinterpret_cast<const uint4 *>(src_x + (size_t)t * rb + c * 16);
        at[j] = t * rs + c * 16;
      }
#pragma unroll
      for (int j = 0; j < XB; ++j) *reinterpret_cast<uint4 *>(dst + at[j]) = v[j];
    }
  }
  // TR: each wavefront's transposition buffer after the x copy
  const int x_bytes = XL ? a_in.n_tok * x_lds_stride(a_in.H * (CODES ? 1 : Elem<T>::kBytes)) : 0;
  uint4 *lb = reinterpret_cast<uint4 *>(reinterpret_cast<char *>(meta + meta_n) + x_bytes +
                                        (threadIdx.x >> 6) * tr_wave_bytes(TRG));
  (void)lb;
  __syncthreads();
  ExpertArgs a = a_in;
  int tbase, n_tiles;   // this launch's slice of the tile list (grp_sel)
  tile_slice(a_in, meta, tbase, n_tiles);
  a.tiles = meta + 2 * tbase;
  a.offsets = meta + n_t;
  a.sorted_token = meta + n_t + n_o;
  if constexpr (FSC) {
    a.sc0 = scl;
    a.sc1 = scl + (a_in.E + 1);
    a.ssc0 = scl + a_in.E;
    a.ssc1 = scl + (a_in.E + 1) + a_in.E;
    a.hs = scl + 2 * (a_in.E + 1);
    a.xs = scl + 3 * (a_in.E + 1);
  }
  constexpr bool XD = tokens_at_multiply<XL, WF>();
  constexpr int U = steps_per_set<WF, TRG, XD>();   // 64-byte K steps per row per register set
  constexpr int XN = token_chunks<WF>();       // 16-byte token chunks per step
  constexpr bool SC4 = (F4 || MXA) && U % 4 == 0;   // block scales of 4 steps per load
  const int lane = threadIdx.x & 63;
  // The wavefront index is uniform; readfirstlane makes that visible to the
  // compiler, so every unit-dependent guard below is a scalar branch.  (An
  // MFMA is a whole-wavefront operation: it must never sit under a per-lane
  // EXEC mask that is expected to switch it off.)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_units = __builtin_amdgcn_readfirstlane(n_tiles) * n_col_blocks;
  // When the last of two or more rounds of units would leave more than a
  // quarter of the wavefronts idle, the units stride over fewer wavefronts,
  // so that every round is (nearly) full: R = ceil(n / nw) rounds over
  // ceil(n / R) wavefronts; the others exit.  Hy3 decode gate-up with FP8,
  // MXFP4 and W4A8 weights (last rounds 52-61 % full): 2.5-3 % faster; with
  // the last round fuller (bf16, W8A8 gate-up) the whole grid was as fast or
  // faster.
  int nw = gridDim.x * WPB;
  {
    const int R = (n_units + nw - 1) / nw, tail = n_units - (R - 1) * nw;
    if (R >= 2 && 4 * tail < 3 * nw) nw = (n_units + R - 1) / R;
  }
  const int w = blockIdx.x * WPB + wave;
  if (w >= nw) return;
  const int kmax = n_units / nw + 1;
  // Wavefront ids interleave the XCDs (block b runs on XCD b % 8), so the
  // units of one expert spread over all XCDs and HBM channels.
  UnitSrc src;    // item whose blocks are being loaded
  UnitOut om, ol;     // item being multiplied, item being loaded
  int k_ld = next_item<T, GATE_UP, WF, XL, TRG>(a, 0, w, nw, n_units, n_col_blocks, lane, src, ol);
  if (k_ld >= kmax) return;
  int k_mm = k_ld;
  om = ol;
  int s_ld = 0, s_mm = 0;   // next K step to load / to multiply, in their units

  f32x4_t acc[2][MT];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 aw0[U], aw1[U], ax[U][MT][XN];
  uint4 bw0[U], bw1[U], bx[U][MT][XN];
  uint32_t as0[U], as1[U], bs0[U], bs1[U];   // MXFP4: the lane's block scale codes
  uint32_t axs[U][MT], bxs[U][MT];           // W4A8: the token rows' block scale codes
  // Load the next block of the loading unit into set W0/W1/X, then move the
  // loading position on (to the next unit at the end of this one).  Steps past
  // nsub re-read the last step (in bounds) and are not used.
  // MXFP4 and W4A8 weights, 4 steps per register set: the scales of steps
  // st .. st + 3 (all four lane groups) are 16 contiguous bytes of a scale
  // row when the unit's K is a multiple of 512 (then st % 4 == 0 and st + 3 <
  // nsub, or st >= nsub; the rows are 16-byte aligned): one load per row
  // instead of four byte loads per lane (MXFP4 Hy3 decode gate-up 109 -> 90
  // us).  The lane's byte of step st + v is byte g of word v, shifted to byte
  // 0 (the MFMA reads byte 0 of the scale register; the MXFP4 decode takes
  // the byte alone).  Otherwise byte loads.
#define HY3_SCALES4(S0, S1, XS, u, st)                                                 \
  {                                                                                    \
    const int sh_ = 8 * (lane >> 4);                                                   \
    constexpr uint32_t sm_ = MXA ? 0xFFFFFFFFu : 0xFFu;                                \
    if (src.vs) {                                                                      \
      /* past the end: a valid group of 4 steps, not used */                          \
      const int s4_ = (st) < src.nsub ? (st) : src.nsub - 4;                           \
      const uint4 w0_ = *reinterpret_cast<const uint4 *>(src.s0p - (lane >> 4) + s4_ * 4); \
      S0[(u) + 0] = (w0_.x >> sh_) & sm_; S0[(u) + 1] = (w0_.y >> sh_) & sm_;          \
      S0[(u) + 2] = (w0_.z >> sh_) & sm_; S0[(u) + 3] = (w0_.w >> sh_) & sm_;          \
      {                                                                                \
        const uint4 w1_ = *reinterpret_cast<const uint4 *>(src.s1p - (lane >> 4) + s4_ * 4); \
        S1[(u) + 0] = (w1_.x >> sh_) & sm_; S1[(u) + 1] = (w1_.y >> sh_) & sm_;        \
        S1[(u) + 2] = (w1_.z >> sh_) & sm_; S1[(u) + 3] = (w1_.w >> sh_) & sm_;        \
      }                                                                                \
      if constexpr (MXA) _Pragma("unroll") for (int m = 0; m < MT; ++m) {              \
        const uint4 x_ = *reinterpret_cast<const uint4 *>(src.xsp[m] - (lane >> 4) + s4_ * 4); \
        XS[(u) + 0][m] = x_.x >> sh_; XS[(u) + 1][m] = x_.y >> sh_;                    \
        XS[(u) + 2][m] = x_.z >> sh_; XS[(u) + 3][m] = x_.w >> sh_;                    \
      }                                                                                \
    } else {                                                                           \
      _Pragma("unroll") for (int v = 0; v < 4; ++v) {                                  \
        const int sv_ = (st) + v < src.nsub ? (st) + v : src.nsub - 1;                 \
        S0[(u) + v] = src.s0p[sv_ * 4];                                                \
        S1[(u) + v] = src.s1p[sv_ * 4];                                                \
        if constexpr (MXA) _Pragma("unroll") for (int m = 0; m < MT; ++m) XS[(u) + v][m] = src.xsp[m][sv_ * 4]; \
      }                                                                                \
    }                                                                                  \
  }
#define HY3_LOAD(W0, W1, X, S0, S1, XS)                                                \
  {                                                                                    \
    _Pragma("unroll") for (int u = 0; u < U; ++u) {                                    \
      const int st_ = s_ld + u < src.nsub ? s_ld + u : src.nsub - 1;                  \
      if constexpr (TR) {   /* load j of a group: rows (16 / TRG) j .. */             \
        const int g_ = s_ld + (u & ~(TRG - 1)) < src.nsub ? s_ld + (u & ~(TRG - 1))   \
                                                          : src.nsub - TRG;             \
        const size_t o_ = (size_t)g_ * 64 + (size_t)(16 / TRG * (u & (TRG - 1))) * src.rowb; \
        W0[u] = load_nt16(src.w0p + o_);                                               \
        W1[u] = load_nt16(src.w1p + o_);                                               \
      } else {                                                                         \
        const int o_ = st_ * 64;                                                       \
        W0[u] = *reinterpret_cast<const uint4 *>(src.w0p + o_);                        \
        W1[u] = *reinterpret_cast<const uint4 *>(src.w1p + o_);                        \
      }                                                                                \
      if constexpr ((F4 || MXA) && !SC4) {                                             \
        S0[u] = src.s0p[st_ * 4];                                                      \
        S1[u] = src.s1p[st_ * 4];                                                      \
      }                                                                                \
      if constexpr (MXA && !SC4) {                                                     \
        _Pragma("unroll") for (int m = 0; m < MT; ++m) XS[u][m] = src.xsp[m][st_ * 4]; \
      }                                                                                \
      if constexpr (SC4) {                                                             \
        if (u % 4 == 0) HY3_SCALES4(S0, S1, XS, u, s_ld + u);                          \
      }                                                                                \
      if constexpr (!XD)                                                               \
      _Pragma("unroll") for (int m = 0; m < MT; ++m)                                   \
        _Pragma("unroll") for (int h = 0; h < XN; ++h)                                 \
          X[u][m][h] = XL ? *reinterpret_cast<const uint4 *>(xl + src.xlo[m] +          \
                                                             st_ * 64 * XN +           \
                                                             h * (MXA ? 64 : 16))      \
                          : *reinterpret_cast<const uint4 *>(src.xp[m] + st_ * 64 * XN + \
                                                             h * (MXA ? 64 : 16));     \
    }                                                                                  \
    s_ld += U;                                                                         \
    if (s_ld >= src.nsub) {                                                            \
      k_ld = next_item<T, GATE_UP, WF, XL, TRG>(a, k_ld + 1, w, nw, n_units, n_col_blocks,   \
                                           lane, src, ol);                             \
      s_ld = 0;                                                                        \
    }                                                                                  \
  }
  // Multiply one block of the multiplying unit; at its end, write the unit
  // and move on.  `more` turns false after the last unit.
#define HY3_MMA(W0, W1, X, S0, S1, XS)                                                 \
  {                                                                                    \
    if constexpr (XD) {   /* this block's token chunks, from LDS */                 \
      _Pragma("unroll") for (int u = 0; u < U; ++u) {                                  \
        const int sx_ = s_mm + u < om.nsub ? s_mm + u : om.nsub - 1;                   \
        _Pragma("unroll") for (int h = 0; h < XN; ++h)                                 \
          X[u][0][h] = *reinterpret_cast<const uint4 *>(xl + om.xlo + sx_ * 64 * XN +  \
                                                        h * (MXA ? 64 : 16));           \
      }                                                                                \
    }                                                                                  \
    if constexpr (TR) {                                                                \
      transpose_groups<U, TRG>(W0, lb, lane);                                          \
      transpose_groups<U, TRG>(W1, lb, lane);                                          \
    }                                                                                  \
    _Pragma("unroll") for (int u = 0; u < U; ++u) {                                    \
      if (s_mm + u < om.nsub) {                                                        \
        if constexpr (A8C) {                                                           \
          /* steps u and u + 1 (nsub and U are even) form one 128-K MFMA */           \
          if ((u & 1) == 0) {                                                          \
            _Pragma("unroll") for (int m = 0; m < MT; ++m) {                           \
              mma_fp8(acc[0][m], W0[u], W0[u + 1], X[u][m][0], X[u + 1][m][0]);       \
              if (om.nf == 2)                                                          \
                mma_fp8(acc[1][m], W1[u], W1[u + 1], X[u][m][0], X[u + 1][m][0]);     \
            }                                                                          \
          }                                                                            \
        } else if constexpr (MXA) {                                                    \
          _Pragma("unroll") for (int m = 0; m < MT; ++m) {                             \
            mma_fp4_fp8(acc[0][m], W0[u], S0[u], X[u][m][0], X[u][m][1], XS[u][m]);    \
            if (om.nf == 2)                                                            \
              mma_fp4_fp8(acc[1][m], W1[u], S1[u], X[u][m][0], X[u][m][1], XS[u][m]);  \
          }                                                                            \
        } else if constexpr (F4) {                                                     \
          const float sc0_ = e8m0_to_f32(S0[u]);                                       \
          const uint4 q0_ = W0[u];                                                     \
          const uint4 f0_[4] = {fp4x8_to_bf16(q0_.x, sc0_), fp4x8_to_bf16(q0_.y, sc0_), \
                                fp4x8_to_bf16(q0_.z, sc0_), fp4x8_to_bf16(q0_.w, sc0_)}; \
          _Pragma("unroll") for (int m = 0; m < MT; ++m)                               \
            _Pragma("unroll") for (int f = 0; f < 4; ++f)                              \
              Mma<T>::step(acc[0][m], f0_[f], X[u][m][f]);                             \
          if (om.nf == 2) {                                                            \
            const float sc1_ = e8m0_to_f32(S1[u]);                                     \
            const uint4 q1_ = W1[u];                                                   \
            const uint4 f1_[4] = {fp4x8_to_bf16(q1_.x, sc1_), fp4x8_to_bf16(q1_.y, sc1_), \
                                  fp4x8_to_bf16(q1_.z, sc1_), fp4x8_to_bf16(q1_.w, sc1_)}; \
            _Pragma("unroll") for (int m = 0; m < MT; ++m)                             \
              _Pragma("unroll") for (int f = 0; f < 4; ++f)                            \
                Mma<T>::step(acc[1][m], f1_[f], X[u][m][f]);                           \
          }                                                                            \
        } else if constexpr (F8) {                                                     \
          uint4 l0_, h0_, l1_, h1_;                                                    \
          e4m3x16_to_bf16(W0[u], l0_, h0_);                                            \
          if (om.nf == 2) e4m3x16_to_bf16(W1[u], l1_, h1_);                            \
          _Pragma("unroll") for (int m = 0; m < MT; ++m) {                             \
            Mma<T>::step(acc[0][m], l0_, X[u][m][0]);                                  \
            Mma<T>::step(acc[0][m], h0_, X[u][m][XN - 1]);                             \
            if (om.nf == 2) {                                                          \
              Mma<T>::step(acc[1][m], l1_, X[u][m][0]);                                \
              Mma<T>::step(acc[1][m], h1_, X[u][m][XN - 1]);                           \
            }                                                                          \
          }                                                                            \
        } else {                                                                       \
          _Pragma("unroll") for (int m = 0; m < MT; ++m) {                             \
            Mma<T>::step(acc[0][m], W0[u], X[u][m][0]);                                \
            if (om.nf == 2) Mma<T>::step(acc[1][m], W1[u], X[u][m][0]);                \
          }                                                                            \
        }                                                                              \
      }                                                                                \
    }                                                                                  \
    s_mm += U;                                                                         \
    if (s_mm >= om.nsub) {                                                             \
      unit_epilogue<T, GATE_UP, WF>(a, om, acc, lane);                             \
      _Pragma("unroll") for (int f = 0; f < 2; ++f)                                    \
        _Pragma("unroll") for (int m = 0; m < MT; ++m) acc[f][m] = f32x4_t{0.f, 0.f, 0.f, 0.f}; \
      k_mm = next_item<T, GATE_UP, WF, XL, TRG>(a, k_mm + 1, w, nw, n_units, n_col_blocks,   \
                                           lane, src_dummy, om);                       \
      s_mm = 0;                                                                        \
      more = k_mm < kmax;                                                              \
    }                                                                                  \
  }
  UnitSrc src_dummy;   // next_unit also fills operand pointers; the multiply side ignores them
  bool more = true;
  HY3_LOAD(aw0, aw1, ax, as0, as1, axs);
  while (more) {
    if (k_ld < kmax) HY3_LOAD(bw0, bw1, bx, bs0, bs1, bxs);
    __builtin_amdgcn_sched_barrier(0);   // keep the next block's loads ahead
    HY3_MMA(aw0, aw1, ax, as0, as1, axs);
    if (!more) break;
    if (k_ld < kmax) HY3_LOAD(aw0, aw1, ax, as0, as1, axs);
    __builtin_amdgcn_sched_barrier(0);
    HY3_MMA(bw0, bw1, bx, bs0, bs1, bxs);
  }
#undef HY3_MMA
#undef HY3_LOAD
#undef HY3_SCALES4
}

// Persistent grid: WAVES_PER_SIMD wavefronts per SIMD on the 256 CUs.
constexpr int STREAM_BLOCKS = 256 * WAVES_PER_SIMD;
constexpr size_t STREAM_XL_LDS_MAX = 160 * 1024;   // LDS of one workgroup (one per CU)

// LDS bytes of the x copy (rows padded), or 0 when the gate-up GEMM of this
// batch does not stage x (the copy and the unit metadata do not fit).
template <typename T, int WF>
size_t x_lds_bytes(const ExpertArgs &a) {
  const int rb = a.H * (token_codes<WF>() ? 1 : Elem<T>::kBytes);
  const size_t meta = (meta_lds_bytes(a, true) + 15) / 16 * 16;
  const size_t x = (size_t)a.n_tok * x_lds_stride(rb);
  return meta + x <= STREAM_XL_LDS_MAX ? x : 0;
}

// Bytes per weight row of K elements.
template <typename T, int WF>
constexpr int weight_row_bytes(int K) {
  return (WF == WF_MXFP4 || WF == WF_W4A8) ? K / 2
         : (WF == WF_FP8 || WF == WF_W8A8) ? K
                                           : K * Elem<T>::kBytes;
}

// Group size of the grouped weight loads for a format (0: none): four
// 64-byte steps where the register sets hold whole groups of four without
// spilling, else two.  FP8 takes four steps per set; MXFP4 weights with bf16
// tokens take groups of two (at four they spill; the grouped loads with two
// steps per set beat the MFMA-shaped ones with three: Hy3 decode 0.254 ->
// 0.202 ms), two groups per set when the tokens are read at multiply time.
template <typename T, int WF>
constexpr int tr_group() {
  if (std::is_same<T, float>::value) return 0;
  return WF == WF_MXFP4 ? 2 : 4;
}
// Every weight row of the launch a multiple of a group's 64 trg bytes.
template <typename T, int WF>
bool tr_rows(const ExpertArgs &a, bool gate_up, int trg) {
  auto ok = [trg](int K) { return weight_row_bytes<T, WF>(K) % (64 * trg) == 0; };
  if (gate_up) return ok(a.H);
  return (a.grp_sel == GRP_SHARED || ok(a.I)) &&
         (a.grp_sel == GRP_ROUTED || a.I_shared == 0 || ok(a.I_shared));
}

template <typename T, int WF, int TRG, int BRANCH>
hipError_t launch_skinny_tr(const ExpertArgs &a, bool gate_up, size_t xb, hipStream_t stream) {
  const size_t meta = (meta_lds_bytes(a, gate_up) + 15) / 16 * 16;
  if (gate_up) {
    const int Imax = a.I > a.I_shared ? a.I : a.I_shared;
    const int ncb = (Imax + 15) / 16;
    if (xb)   // one 512-thread workgroup per CU, x in LDS
      hipLaunchKernelGGL((expert_stream_kernel<T, true, WF, true, TRG, BRANCH>),
                         dim3(STREAM_BLOCKS / 2), dim3(512), meta + xb + 8 * tr_wave_bytes(TRG),
                         stream, a, ncb);
    else
      hipLaunchKernelGGL((expert_stream_kernel<T, true, WF, false, TRG, BRANCH>),
                         dim3(STREAM_BLOCKS), dim3(256), meta + 4 * tr_wave_bytes(TRG), stream, a,
                         ncb);
  } else {
    const int ncb = (a.H + 31) / 32;
    hipLaunchKernelGGL((expert_stream_kernel<T, false, WF, false, TRG, BRANCH>),
                       dim3(STREAM_BLOCKS), dim3(256), meta + 4 * tr_wave_bytes(TRG), stream, a,
                       ncb);
  }
  return hipGetLastError();
}

template <typename T, int WF, int BRANCH>
hipError_t launch_skinny_b(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  const size_t xb = gate_up ? x_lds_bytes<T, WF>(a) : 0;
  constexpr int G = tr_group<T, WF>();
  if constexpr (G > 0) {
    // The grouped loads with the LDS copy of x when it leaves room for the
    // 8 wavefronts' buffers; groups of two steps (half the buffer) when only
    // those leave room; else the grouped loads with the
    // tokens from global memory (measured faster than the copy without them
    // for bf16 x at H = 4096).
    const size_t meta = (meta_lds_bytes(a, gate_up) + 15) / 16 * 16;
    auto room = [&](int trg) {
      return !xb || meta + xb + 8 * (size_t)tr_wave_bytes(trg) <= STREAM_XL_LDS_MAX;
    };
    if (tr_rows<T, WF>(a, gate_up, G) && room(G))
      return launch_skinny_tr<T, WF, G, BRANCH>(a, gate_up, xb, stream);
    if constexpr (G == 4) {
      if (xb && tr_rows<T, WF>(a, gate_up, 2) && room(2))
        return launch_skinny_tr<T, WF, 2, BRANCH>(a, gate_up, xb, stream);
    }
    if (tr_rows<T, WF>(a, gate_up, G))
      return launch_skinny_tr<T, WF, G, BRANCH>(a, gate_up, 0, stream);
  }
  return launch_skinny_tr<T, WF, 0, BRANCH>(a, gate_up, xb, stream);
}

// Every batch of this path runs units of one 16-row token fragment: the
// tile list holds tiles of SKINNY_ROWS rows, and a group of more rows has
// several, each of which streams the group's weights again (their units of
// one column block run in the same round of the persistent grid, so the
// repeated rows are mostly cache hits).  Tiles of 32 and 64 rows with two
// and four fragments per unit, which read the weights once, were slower:
// their register sets held fewer steps and their padding fragments cost
// full token loads for routed experts of a few rows (Hy3 decode T=64
// 0.915 -> 0.805 ms, T=32 0.661 -> 0.652 ms).
template <typename T, int WF>
hipError_t launch_skinny(const ExpertArgs &a, bool gate_up, hipStream_t stream) {
  return a.grp_sel == GRP_SHARED ? launch_skinny_b<T, WF, 1>(a, gate_up, stream)
                                 : launch_skinny_b<T, WF, 0>(a, gate_up, stream);
}

}  // namespace

hipError_t launch_tiled_gate_up(const ExpertArgs &a, int dtype, hipStream_t stream);
hipError_t launch_tiled_down(const ExpertArgs &a, int dtype, hipStream_t stream);
hipError_t launch_big_gate_up(const ExpertArgs &a, int dtype, hipStream_t stream);
hipError_t launch_big_down(const ExpertArgs &a, int dtype, hipStream_t stream);

hipError_t launch_gate_up(const ExpertArgs &a, int dtype, int path, hipStream_t stream) {
  if (path == PATH_SKINNY)
    return dtype == DT_F32 ? launch_skinny<float, WF_DTYPE>(a, true, stream)
           : a.amx         ? launch_skinny<bf16_t, WF_W4A8>(a, true, stream)
           : a.w_fp4       ? launch_skinny<bf16_t, WF_MXFP4>(a, true, stream)
           : a.w_fp8 && a.a8 && a.a8_codes ? launch_skinny<bf16_t, WF_W8A8>(a, true, stream)
           : a.w_fp8       ? launch_skinny<bf16_t, WF_FP8>(a, true, stream)
                           : launch_skinny<bf16_t, WF_DTYPE>(a, true, stream);
  if (path == PATH_BIG) return launch_big_gate_up(a, dtype, stream);
  return launch_tiled_gate_up(a, dtype, stream);
}

hipError_t launch_down(const ExpertArgs &a, int dtype, int path, hipStream_t stream) {
  if (path == PATH_SKINNY)
    return dtype == DT_F32 ? launch_skinny<float, WF_DTYPE>(a, false, stream)
           : a.amx         ? launch_skinny<bf16_t, WF_W4A8>(a, false, stream)
           : a.w_fp4       ? launch_skinny<bf16_t, WF_MXFP4>(a, false, stream)
           : a.w_fp8 && a.a8 && a.a8_codes ? launch_skinny<bf16_t, WF_W8A8>(a, false, stream)
           : a.w_fp8       ? launch_skinny<bf16_t, WF_FP8>(a, false, stream)
                           : launch_skinny<bf16_t, WF_DTYPE>(a, false, stream);
  if (path == PATH_BIG) return launch_big_down(a, dtype, stream);
  return launch_tiled_down(a, dtype, stream);
}

}  // namespace hy3moe
