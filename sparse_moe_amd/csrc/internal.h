// Host-side launchers of the MoE kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hy3moe {

enum { DT_F32 = 0, DT_BF16 = 1 };
// Storage of the expert weights inside the GEMM kernels.
// WF_W4A8: MXFP4 weights with dynamic MXFP8 token rows (E4M3 codes and one
// E8M0 scale per 32), multiplied by block-scaled FP4 x FP8 MFMAs.
// WF_W8A8: FP8 weights with static FP8 token rows as E4M3 codes, multiplied
// by FP8 x FP8 MFMAs (the weight-streaming path; the large-tile path has its
// own A8 kernels).
enum { WF_DTYPE = 0, WF_FP8 = 1, WF_MXFP4 = 2, WF_W4A8 = 3, WF_W8A8 = 4 };

// Row-tile shapes of the expert GEMMs.
constexpr int TILED_ROWS = 128;     // rows (token copies) per tile, large-T path
constexpr int TILED_GU_COLS = 64;   // h columns per gate-up tile (64 gate + 64 up rows)
constexpr int TILED_DN_COLS = 128;  // y columns per down tile
constexpr int SKINNY_MAX_T = 64;    // at or below this T the weight-streaming path runs
constexpr int SKINNY_ROWS = 16;     // rows per tile of the weight-streaming path
constexpr int SKINNY_GU_COLS = 64;  // h columns per skinny gate-up workgroup
constexpr int SKINNY_DN_COLS = 128; // y columns per skinny down workgroup
constexpr int PERM_CHUNK = 1024;    // (token, pick) entries per wavefront in the permutation
constexpr int MAX_KSPLIT = 16;      // router K-slices (partial logit sets)
constexpr int BIG_ROWS = 256;       // rows per tile of the large-tile path
constexpr int BIG_MIN_AVG_ROWS = 192;  // mean routed rows per expert that selects it

enum { GRP_ALL = 0, GRP_ROUTED = 1, GRP_SHARED = 2 };

// Which expert-GEMM path runs for a batch (the tile list is built for it).
enum { PATH_SKINNY = 0, PATH_TILED = 1, PATH_BIG = 2 };
// big_ok = false keeps batches off the large-tile path (static FP8
// activations there need H, I and I_shared to be multiples of 128).
inline int expert_path(int64_t T, int K, int E, bool big_ok = true) {
  if (T <= SKINNY_MAX_T) return PATH_SKINNY;
  if (big_ok && T * K >= (int64_t)BIG_MIN_AVG_ROWS * E) return PATH_BIG;
  return PATH_TILED;
}

// Router -------------------------------------------------------------------
constexpr int ROUTER_PLANES_MIN_T = 1024;  // bf16 batches this large pre-split the weight
bool router_use_planes(int64_t T, int dtype);
int router_ksplit(int64_t T, int H, int E, int dtype);
// planes: workspace for the bf16 weight planes [3][E][H], or null (split on the fly).
// planes_in: the caller's planes from hy3moe_router_split (same E, H and
// router_prec), used instead of splitting into `planes` when that path runs.
hipError_t launch_router(const void *x, int dtype, int router_prec, const float *w_router,
                         uint16_t *planes, const uint16_t *planes_in, double *part, int T, int H,
                         int E, int S, hipStream_t stream);
// Planes bytes for E experts of H values: NP bf16 planes (3 for the exact
// split, 2 for the two-term one), E padded to a multiple of 16.
size_t router_planes_bytes(int E, int H, int router_prec);
// The split alone: fp32 w_router [E][H] -> planes (router_planes_bytes).
hipError_t launch_router_split(const float *w_router, int router_prec, uint16_t *planes, int E,
                               int H, hipStream_t stream);

// Score + top-K select ------------------------------------------------------
// An activation quantisation the select launch may host in workgroups of
// its own (it needs neither the route nor the select): mode QH_NONE, QH_E4M3
// (static FP8 of n elements of x, n % 8 == 0; carrier 1 writes the codes'
// bf16 values) or QH_MXFP8 (dynamic MXFP8 of n bf16 values in rows of a
// multiple of 32; codes and scales, or carrier 1 the bf16 values).
enum { QH_NONE = 0, QH_E4M3 = 1, QH_MXFP8 = 2 };
struct HostedQuant {
  int mode = QH_NONE;
  const void *x = nullptr;
  int dtype = DT_BF16;
  int64_t n = 0;
  const float *scale = nullptr;
  void *q = nullptr;
  uint8_t *scales = nullptr;
  int carrier = 0;
};
hipError_t launch_select(const double *part, int S, int T, int E, int K, const float *bias,
                         int route_mode, float scale, float renorm_eps, int32_t *idx,
                         float *weight, hipStream_t stream, const HostedQuant &hq = HostedQuant());

// Permutation ---------------------------------------------------------------
struct PermArgs {
  const int32_t *idx;     // [T*K]
  int32_t *hist;          // [nchunks][E]
  int32_t *counts;        // [E+1]
  int32_t *offsets;       // [E+2]
  int32_t *sorted_token;  // [R]
  int32_t *pos_of;        // [T*K]
  int32_t *tiles;         // [2*max_tiles + 2]: pairs, tile count, routed tile count
  int T, K, E, T_shared, nchunks, tile_rows, max_tiles;
  int sort_tiles;         // tile list largest groups first (else group order)
  int shared_last;        // the shared expert's tiles after every routed tile
};
hipError_t launch_permute(const PermArgs &a, hipStream_t stream);
// Metadata of the shared expert's own launches, which need no routing: a
// tile list [2*max_tiles + 2] holding only its tiles (group E, rows N + i
// tile_rows, then the tile count and a routed tile count of 0), offsets
// [E+2] (every routed group empty at row N, the shared rows [N, N + T)) and
// the identity map sorted_token[N + t] = t of a [N + T] row map.
hipError_t launch_shared_meta(int32_t *tiles, int32_t *offsets, int32_t *sorted_token, int T,
                              int N, int E, int tile_rows, int max_tiles, hipStream_t stream);

// Expert GEMMs ----------------------------------------------------------------
struct ExpertArgs {
  const void *act;        // gate-up: x [T][H]; down: h [R][ldh]
  const void *w0;         // gate-up: w_gate [E][I][H]; down: w_down [E][H][I]
  const void *w1;         // gate-up: w_up [E][I][H]; down: unused
  const void *ws0;        // shared: gate [Is][H] / down [H][Is]
  const void *ws1;        // shared: up [Is][H]
  void *out;              // gate-up: h [R][ldh]; down: y [R][H] (fp16 for bf16 layers)
  const int32_t *sorted_token;
  const int32_t *offsets;
  const int32_t *tiles;   // (group, first row) pairs, then the tile count and the
                          // routed tile count
  int E, H, I, I_shared, ldh, max_tiles;
  int n_rows;             // rows of sorted_token (T K routed + T shared)
  int n_tok;              // T (rows of x)
  // Groups this launch computes: GRP_ALL, GRP_ROUTED (the tiles before the
  // routed tile count) or GRP_SHARED (the tiles after it); the last two need
  // a tile list made with shared_last, or the shared expert's own list
  // (launch_shared_meta).
  int grp_sel;
  // FP8 E4M3 expert weights (w_fp8 = 1): w0/w1/ws0/ws1 hold bytes and the
  // weight is scale * value, with scales sc0[g] / sc1[g] for routed group g
  // and *ssc0 / *ssc1 for the shared expert (gate-up: gate, up; down: down).
  int w_fp8;
  const float *sc0, *sc1, *ssc0, *ssc1;
  // MXFP4 expert weights (w_fp4 = 1): w0/w1/ws0/ws1 hold E2M1 codes, two per
  // byte (rows of K/2 bytes), and mx0/mx1 (routed, [E][rows][K/32]) and
  // mxs0/mxs1 (shared, [rows][K/32]) one E8M0 scale per 32 weights of a row.
  int w_fp4;
  const uint8_t *mx0, *mx1, *mxs0, *mxs1;
  // Dynamic MXFP8 token rows (amx = 1, weight-streaming and large-tile
  // paths): act holds E4M3 codes (rows of H or ldh bytes) and act_sc their
  // E8M0 scales (rows of H / 32 or ldh / 32 bytes).  The tiled path reads the
  // exact bf16 values instead (amx = 0 there).  out_sc: when set, the
  // large-tile gate-up GEMM quantises h itself and writes codes to out and
  // their scales there (rows of ldh / 32 bytes).
  int amx;
  const uint8_t *act_sc;
  uint8_t *out_sc;
  // Static FP8 activations (a8 = 1, with w_fp8): act holds E4M3 codes on the
  // large-tile path and their exact bf16 values on the other two; *xs is the
  // scale of x and hs[g] that of group g's h (hs[E]: shared).  The gate-up
  // GEMMs store h quantised with hs[g] in the same form.
  int a8;
  const float *xs, *hs;
  // With a8: the token rows are E4M3 codes (FP8 MFMAs: the large-tile path,
  // and the weight-streaming path when H, I and I_shared are multiples of
  // 128), else the bf16 values of the codes (bf16 MFMAs).
  int a8_codes;
};
// The slice of the tile list a launch walks (ExpertArgs::grp_sel): first
// tile index and tile count.
__device__ __forceinline__ void tile_slice(const ExpertArgs &a, const int32_t *tiles, int &base,
                                           int &n) {
  const int total = tiles[2 * a.max_tiles], routed = tiles[2 * a.max_tiles + 1];
  base = a.grp_sel == GRP_SHARED ? routed : 0;
  n = a.grp_sel == GRP_ROUTED ? routed : (a.grp_sel == GRP_SHARED ? total - routed : total);
}

hipError_t launch_gate_up(const ExpertArgs &a, int dtype, int path, hipStream_t stream);
hipError_t launch_down(const ExpertArgs &a, int dtype, int path, hipStream_t stream);

// Static FP8 activation quantisation: q[i] = E4M3(x[i] / *scale) for n
// elements of x (dtype); carrier = 0 stores the code bytes, 1 their values as
// bf16.  n % 8 == 0 and 16-byte aligned buffers for the vector path; any n
// otherwise.
hipError_t launch_quant_e4m3(const void *x, int dtype, int64_t n, const float *scale, void *q,
                             int carrier, hipStream_t stream);

// Dynamic MXFP8 quantisation of n bf16 values (rows of a multiple of 32):
// carrier = 0 writes E4M3 codes (q, n bytes) and one E8M0 scale per 32
// (scales, n / 32 bytes); carrier = 1 writes the exact bf16 values (q, n
// bf16; may be `in` itself).  n % 32 == 0, 16-byte aligned buffers.
hipError_t launch_quant_mxfp8(const void *in, int64_t n, void *q, uint8_t *scales, int carrier,
                              hipStream_t stream);

// Combine ---------------------------------------------------------------------
hipError_t launch_combine(const void *y, const int32_t *pos_of, const float *weight,
                          const int32_t *offsets, int T, int K, int H, int E, int has_shared,
                          void *out, int dtype, hipStream_t stream);

}  // namespace hy3moe
