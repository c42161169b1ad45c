/*
 * hy3moe.h -- C ABI of the MI355X (gfx950) Hy3-style sparse MoE FFN layer.
 *
 * The layer (hy3 README "Model facts": 192 routed experts, top-8, one shared
 * expert that is always active, expert intermediate 1536, hidden 4096):
 *
 *   logits = x W_r^T                      bias-free router linear, fp32-accurate
 *   s      = sigmoid(logits)              (HYV3Config moe_router_use_sigmoid)
 *   pick   = top-K of s + expert_bias     bias steers the choice only
 *   w      = scale * s[pick] / sum s[pick]   unbiased, renormalised, x2.826
 *   out    = shared(x) + sum_j w_j * expert_{pick_j}(x)
 *   expert(a) = W_down ( silu(W_gate a) * (W_up a) )     SwiGLU
 *
 * and the HunyuanImage-3.0 softmax variant (HunyuanImage 3.0 MoE reading,
 * easy_topk): p = softmax(logits); pick = top-K of p;
 * w = p[pick] / max(sum p[pick], renorm_eps); no bias, no scale.
 *
 * Everything runs as hand-written HIP kernels on the caller's stream.
 *
 * Conventions for every entry point
 * ---------------------------------
 *  - All tensor pointers are DEVICE memory owned by the caller, row-major,
 *    dense, and 16-byte aligned.  The library allocates nothing and keeps no
 *    state between calls.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    asynchronously; the call returns after enqueueing.  Calls on different
 *    streams are safe when each has its own workspace; calls sharing one
 *    workspace must be ordered by the caller.
 *  - Validation happens before anything is enqueued: on a non-zero return
 *    nothing has been launched.  Faults during kernel execution surface at
 *    the caller's next synchronisation on the stream.
 *  - T == 0 is a successful no-op.  Non-finite inputs are undefined.
 *  - Element types: HY3MOE_BF16 means bfloat16 (1-8-7 bits) for x, out and
 *    all expert weights; HY3MOE_F32 means float32 for them.  The router
 *    weight, the expert bias and the combine weights are always float32.
 *    With w_format HY3MOE_WFMT_FP8_E4M3 the expert weights are instead one
 *    byte per element (see hy3moe_config.w_format).
 */
#ifndef HY3MOE_H
#define HY3MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---- */
#define HY3MOE_OK               0
#define HY3MOE_ERR_INVALID     -1  /* null pointer, T<0, K<1, K>E, E>256, K>64, bad enum */
#define HY3MOE_ERR_UNSUPPORTED -2  /* H, I or I_shared not a multiple of 64; T > 2^24;
                                      H, I or I_shared > 65536; T*H or H*max(I, I_shared)
                                      elements of 4 GiB or more; split router with fp32 x;
                                      FP8 expert weights with fp32 x                  */
#define HY3MOE_ERR_WORKSPACE   -3  /* workspace smaller than hy3moe_workspace_bytes()   */
#define HY3MOE_ERR_ALIGN       -4  /* a pointer is not 16-byte aligned                  */
#define HY3MOE_ERR_HIP         -5  /* a kernel launch failed (hipGetLastError)          */
#define HY3MOE_ERR_SCRATCH     -6  /* hy3moe_forward_static: the batch's workspace would
                                      exceed HY3MOE_STATIC_SCRATCH_BYTES               */

/* ---- enums ---- */
#define HY3MOE_F32  0
#define HY3MOE_BF16 1

#define HY3MOE_ROUTE_SIGMOID_BIAS 0  /* Hy3: sigmoid, biased top-K, unbiased renorm x scale */
#define HY3MOE_ROUTE_SOFTMAX      1  /* HunyuanImage-3.0 easy_topk: softmax, top-K, clamp  */

/* Router arithmetic.  FP32: logits exact to fp32 accumulation (the fp32 weight
 * is split on the fly into three bf16 terms whose sum is the weight exactly,
 * each term runs on bf16 MFMA with fp32 accumulation; fp32 activations use
 * fp32 MFMA).  SPLIT2_BF16: the two-term approximation W ~ W_hi + W_lo/256
 * with two accumulators and one fused multiply-add in the epilogue (Hy3
 * Preview inference case, section 2 "Router GEMM"); bf16 activations only. */
#define HY3MOE_ROUTER_FP32        0
#define HY3MOE_ROUTER_SPLIT2_BF16 1

/* Storage of the expert weights (w_gate, w_up, w_down and the shared
 * expert's).  DTYPE: elements of cfg.dtype.  FP8_E4M3: one byte per element
 * in the OCP FP8 E4M3 encoding (sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities; S.1111.111 is NaN) with one float32 scale per expert
 * matrix, the weight being scale * value (the FP8 W8A8 weights of the CANN
 * deployment article, section 8.2, with tensor-wise scales).  Activations
 * stay bfloat16 (x and out bf16, cfg.dtype must be HY3MOE_BF16); the expert
 * GEMMs decode the codes exactly to bfloat16 and apply the scale to the
 * float32 accumulators.  All three GEMM paths take FP8 weights: the
 * weight-streaming one (T <= 64), where the weight bytes set the time, and
 * the tile paths, which decode each chunk on its way into LDS. */
#define HY3MOE_WFMT_DTYPE    0
#define HY3MOE_WFMT_FP8_E4M3 1
/* MXFP4 (OCP microscaling; the CANN deployment article, section 8.2: routed
 * experts W4 = MXFP4): each expert tensor holds FP4 E2M1 codes (sign, 2
 * exponent bits with bias 1, 1 mantissa bit: 0, 0.5, 1, 1.5, 2, 3, 4, 6),
 * two per byte with the even element in the low nibble, rows of K/2 bytes;
 * every block of 32 consecutive weights of a row (along K) has one E8M0
 * scale 2^(s - 127) in the matching *_mx array.  Activations stay bfloat16
 * (cfg.dtype HY3MOE_BF16, act_format DTYPE); H, I and I_shared must be
 * multiples of 128.  The GEMMs decode the codes with their scale exactly to
 * bfloat16: in registers on the weight-streaming path (T <= 64), on the way
 * into LDS on the tile paths. */
#define HY3MOE_WFMT_MXFP4    2

/* Activations of the expert GEMMs.  DTYPE: x and h as cfg.dtype.
 * FP8_STATIC (W8A8; needs w_format FP8_E4M3): static per-tensor FP8
 * activations, the FP8 path of the CANN deployment article (section 六: an
 * FP8 Linear quantises its input with a static per-tensor input scale;
 * section 8.2: W8A8).  The experts' input x is quantised once with the
 * layer's scale x_scale and each group's h (the SwiGLU output rounded to
 * bf16, the layer's activation tensor) with its own scale h_scale[g]:
 * code = E4M3(v / scale), the quotient a correctly rounded float32 division,
 * clamped to +-448 (saturating), rounded to nearest even.  The GEMMs then
 * run on scale * value of both operands (FP8 MFMAs on the large-tile path,
 * the same values in bf16 on the other two).  The router reads the
 * unquantised x. */
#define HY3MOE_AFMT_DTYPE      0
#define HY3MOE_AFMT_FP8_STATIC 1
/* MXFP8 (W4A8 with w_format MXFP4; the CANN deployment article, section 8.2:
 * routed experts W4A8; section 六: dynamic MXFP8 values): x and every
 * group's h are quantised per block of 32 consecutive values of a row (along
 * H and I) by the OCP microscaling rule: E8M0 scale 2^(floor(log2 amax) - 8)
 * (floored at 2^-127), elements E4M3(v / scale), saturating, nearest even.
 * h is the SwiGLU output rounded to bf16, then quantised.  The
 * weight-streaming and large-tile paths multiply MXFP4 weights by the MXFP8
 * codes with block-scaled FP4 x FP8 MFMAs (the large-tile gate-up GEMM
 * quantises h in its epilogue); the tiled path multiplies the same values
 * in bf16. */
#define HY3MOE_AFMT_MXFP8      2

/* hy3moe_config.shared_w_format / shared_act_format: the shared expert uses
 * the routed experts' formats. */
#define HY3MOE_FMT_AS_ROUTED  -1

/* Shape and mode of one layer call. */
typedef struct hy3moe_config {
  int64_t T;          /* tokens (rows of x)                                   */
  int32_t H;          /* hidden size                                          */
  int32_t E;          /* routed experts, 1..256                               */
  int32_t K;          /* experts per token, 1..min(E,64)                      */
  int32_t I;          /* routed expert intermediate size                      */
  int32_t I_shared;   /* shared expert intermediate size; 0 = no shared expert */
  int32_t dtype;      /* HY3MOE_BF16 or HY3MOE_F32 (x, out, expert weights)   */
  int32_t route_mode; /* HY3MOE_ROUTE_*                                       */
  int32_t router_prec;/* HY3MOE_ROUTER_*                                      */
  float   scale;      /* routed-weight scale: 2.826 for Hy3, 1 for softmax    */
  float   renorm_eps; /* softmax mode: clamp of the top-K sum (1e-8); sigmoid mode: unused */
  int32_t w_format;   /* HY3MOE_WFMT_*: storage of the expert weights            */
  int32_t act_format; /* HY3MOE_AFMT_*: activations of the expert GEMMs          */
  /* Formats of the shared expert, or HY3MOE_FMT_AS_ROUTED (-1) for the routed
   * ones.  The CANN deployment article (section 8.2) runs the routed experts
   * at W4A8 (w_format MXFP4, act_format MXFP8) and the shared expert at W8A8
   * (shared_w_format FP8_E4M3, shared_act_format FP8_STATIC).  Formats of its
   * own follow the same rules as the routed ones (checked against I_shared)
   * and read the shared tensors in those formats: ws_scale for FP8 weights,
   * the ws_*_mx scales for MXFP4, x_scale and h_scale[E] for static FP8
   * activations.  The expert GEMMs then run as two launches each (routed
   * groups, then the shared group), sharing the permutation and the combine. */
  int32_t shared_w_format;
  int32_t shared_act_format;
} hy3moe_config;

/* Weights.  Layouts follow nn.Linear [out, in] (K-contiguous rows), stacked
 * over experts (HunyuanImage 3.0 MoE reading, stacked moe_weight/moe_weight_2):
 *   w_router  [E, H]     fp32
 *   expert_bias [E]      fp32, sigmoid mode only; NULL means all zero
 *   w_gate, w_up [E, I, H]      dtype
 *   w_down       [E, H, I]      dtype
 *   ws_gate, ws_up [I_shared, H], ws_down [H, I_shared]  dtype (NULL if I_shared==0)
 * With w_format FP8_E4M3 the six expert tensors hold E4M3 bytes and
 *   w_gate_scale, w_up_scale, w_down_scale [E]   fp32, one per routed matrix
 *   ws_scale [3]   fp32: shared gate, up, down (NULL if I_shared == 0)
 * are required (4-byte aligned); with FP8 weights the six expert pointers
 * need 16-byte alignment as always.  The scale pointers are ignored for
 * w_format DTYPE.  With act_format FP8_STATIC
 *   x_scale [1]      fp32: static scale of the experts' input x
 *   h_scale [E + 1]  fp32: static scale of each routed expert's h, then the
 *                    shared expert's (entry E read only if I_shared > 0)
 * are required (4-byte aligned); ignored otherwise.  With w_format MXFP4 the
 * six expert tensors hold packed E2M1 codes (gate/up [E, I, H/2], down
 * [E, H, I/2], shared [I_shared, H/2] / [H, I_shared/2]) and
 *   w_gate_mx, w_up_mx [E, I, H/32], w_down_mx [E, H, I/32]   E8M0 bytes
 *   ws_gate_mx, ws_up_mx [I_shared, H/32], ws_down_mx [H, I_shared/32]
 * are required (16-byte aligned; NULL only for the shared ones when
 * I_shared == 0); the float scale pointers are then ignored. */
typedef struct hy3moe_weights {
  const float *w_router;
  const float *expert_bias;
  const void  *w_gate;
  const void  *w_up;
  const void  *w_down;
  const void  *ws_gate;
  const void  *ws_up;
  const void  *ws_down;
  const float *w_gate_scale;
  const float *w_up_scale;
  const float *w_down_scale;
  const float *ws_scale;
  const float *x_scale;
  const float *h_scale;
  const uint8_t *w_gate_mx;
  const uint8_t *w_up_mx;
  const uint8_t *w_down_mx;
  const uint8_t *ws_gate_mx;
  const uint8_t *ws_up_mx;
  const uint8_t *ws_down_mx;
  /* Optional: the router weight split offline by hy3moe_router_split with
   * this layer's E, H and router_prec (NULL: split per call).  Used by bf16
   * batches of 1024 tokens or more, which run the router GEMM on bf16 planes;
   * smaller batches split w_router in registers and ignore it. */
  const void *w_router_planes;
} hy3moe_weights;

/* Byte offsets of the intermediate buffers inside a forward workspace (for
 * inspection by tests; all offsets are from the workspace base and 256-byte
 * aligned).  Groups 0..E-1 are the routed experts, group E the shared expert.
 * Rows are "expert-major": group g owns rows [offsets[g], offsets[g+1]).      */
typedef struct hy3moe_ws_layout {
  size_t total;          /* == hy3moe_workspace_bytes(cfg, 1)                  */
  size_t logits_part;    /* double [S][T][E] router K-slice partial sums (S = n_ksplit) */
  int32_t n_ksplit;
  size_t idx;            /* int32 [T][K]  (used when the caller passes no idx_out)    */
  size_t weight;         /* float [T][K]  (used when the caller passes no weight_out) */
  size_t counts;         /* int32 [E+1]   rows per group (counts[E] = T or 0)   */
  size_t offsets;        /* int32 [E+2]   exclusive prefix of counts            */
  size_t sorted_token;   /* int32 [R]     token of each expert-major row, R = T*K + T_shared */
  size_t pos_of;         /* int32 [T][K]  expert-major row of (token, pick)     */
  size_t hist;           /* int32 [n_chunks][E] per-chunk expert counts / prefixes */
  int32_t n_chunks;      /* (token, pick) chunks of the permutation             */
  size_t tiles;          /* int32 [2*max_tiles+2] (group, first row) per row tile, then the
                            tile count and the routed tile count (the shared expert's
                            tiles come last when it has formats of its own) */
  int32_t max_tiles;
  int32_t tile_rows;     /* rows per tile of the expert GEMMs for this T       */
  size_t h;              /* dtype [R][I_max]  SwiGLU activations, I_max = max(I, I_shared) */
  size_t y;              /* [R][H] expert outputs before the combine: IEEE fp16 for
                            bf16 layers (11 significant bits), float32 for fp32 layers */
  size_t w_planes;       /* router weight split into 3 bf16 terms (E padded to a
                            multiple of 16), stored in the order the router GEMM
                            reads its operand fragments; used for bf16 batches of
                            T >= 1024 (0 = not used)                              */
  size_t xq;             /* act_format FP8_STATIC: quantised x [T][H], E4M3 bytes
                            when a8_codes is set, else their bf16 values (0 = not
                            used); h then holds h quantised the same way.
                            MXFP8: x as E4M3 bytes (weight-streaming and large-tile
                            paths) or the bf16 values of the codes (tiled path) */
  size_t xs;             /* MXFP8: E8M0 scales of x [T][H/32] (0 = not used)   */
  size_t hq;             /* MXFP8: E4M3 codes of h [R][I_max] (weight-streaming and
                            large-tile paths; the tiled path rewrites h in place
                            with the bf16 values)                              */
  size_t hs;             /* MXFP8: E8M0 scales of h [R][I_max/32]              */
  size_t xq_shared;      /* the shared expert's quantised x when its activation
                            format differs from the routed one (as xq; 0 = not used) */
  size_t xs_shared;      /* its MXFP8 scales (0 = not used)                       */
  size_t shared_meta;    /* int32: the shared expert's own tile list [2*max_tiles+2],
                            offsets [E+2] and row map [R] for its launches on the
                            side stream (0: the shared expert, if any, runs in
                            the routed experts' launches on the caller's stream) */
  int32_t gemm_path;     /* expert GEMMs: 0 weight streaming (T <= 64, tiles of 16
                            rows), 1 tiles of 128 rows, 2 tiles of 256 rows    */
  int32_t a8_codes;      /* static FP8 activations (x and h) are stored as E4M3
                            codes for FP8 MFMAs (large tiles; weight streaming
                            when H, I and I_shared are multiples of 128), else
                            as the bf16 values of the codes                    */
} hy3moe_ws_layout;

/* Workspace size in bytes for hy3moe_forward (for_forward != 0) or for
 * hy3moe_route (for_forward == 0).  Returns 0 if cfg is invalid. */
size_t hy3moe_workspace_bytes(const hy3moe_config *cfg, int for_forward);

/* Fill *out with the forward workspace layout.  Returns HY3MOE_OK or an error. */
int hy3moe_workspace_layout(const hy3moe_config *cfg, hy3moe_ws_layout *out);

/* The gate: router GEMM, scoring and top-K selection.
 *   x        [T, H] dtype
 *   w_router [E, H] fp32;  expert_bias [E] fp32 (sigmoid mode; NULL = zero)
 *   idx      [T, K] int32 out: picked experts in descending selection score,
 *            equal scores ordered by ascending expert index
 *   weight   [T, K] fp32 out: combine weights (sum to `scale` per token in
 *            sigmoid mode, to 1 in softmax mode)
 *   workspace: hy3moe_workspace_bytes(cfg, 0) bytes.
 * Follows the hy3 README "Model facts" MoE routing row and the HunyuanImage
 * 3.0 MoE reading's HunyuanTopKGate (easy_topk). */
int hy3moe_route(const hy3moe_config *cfg, const void *x, const float *w_router,
                 const float *expert_bias, int32_t *idx, float *weight,
                 void *workspace, size_t ws_bytes, void *stream);

/* The offline split of the router weight (Hy3 Preview inference case,
 * section 2 "Router GEMM: dual BF16": the fp32 weight is split once, offline,
 * into bf16 planes, so that no call re-splits it or writes and re-reads a
 * split copy).  router_prec HY3MOE_ROUTER_FP32: the exact three-term split
 * (hi, mid, lo, summing to the weight exactly); HY3MOE_ROUTER_SPLIT2_BF16:
 * the page's two terms hi + lo/256.  The planes are stored in the order the
 * router GEMM reads its operand fragments (an internal layout: pass them
 * back unchanged as hy3moe_weights.w_router_planes or to
 * hy3moe_route_planes, with the same E, H and router_prec).
 *   w_router [E, H] fp32 device, 16-byte aligned; E 1..256, H % 64 == 0
 *   planes   device out, hy3moe_router_planes_bytes(E, H, router_prec) bytes,
 *            16-byte aligned
 * Errors: HY3MOE_ERR_INVALID (bad E, H, router_prec, null pointer),
 * HY3MOE_ERR_UNSUPPORTED (H % 64 or H > 65536), HY3MOE_ERR_WORKSPACE
 * (planes_bytes too small), HY3MOE_ERR_ALIGN; launched on `stream`. */
size_t hy3moe_router_planes_bytes(int32_t E, int32_t H, int32_t router_prec);
int hy3moe_router_split(const float *w_router, int32_t E, int32_t H, int32_t router_prec,
                        void *planes, size_t planes_bytes, void *stream);

/* hy3moe_route with the router weight's offline split (w_router_planes from
 * hy3moe_router_split, or NULL): identical results to hy3moe_route. */
int hy3moe_route_planes(const hy3moe_config *cfg, const void *x, const float *w_router,
                        const void *w_router_planes, const float *expert_bias, int32_t *idx,
                        float *weight, void *workspace, size_t ws_bytes, void *stream);

/* The whole layer: gate, token->expert permutation, grouped SwiGLU experts
 * (routed + shared), and the weighted top-K combine back to token order.
 *   x   [T, H] dtype;   out [T, H] dtype (may not alias x)
 *   idx_out [T, K] int32, weight_out [T, K] fp32: optional (NULL allowed)
 *       copies of the route this call used
 *   workspace: hy3moe_workspace_bytes(cfg, 1) bytes.
 * The steps follow the FusedMoE chain of the Hy3 Preview inference case
 * (section 3: routing/index preprocessing with a contiguous row range per
 * expert, gate-up GEMM reading x through the route index, down GEMM written
 * compactly per expert, top-K weighted aggregation at the end) and the
 * shared/routed sum of the HunyuanImage 3.0 MoE reading ("Shared MLP").
 * The shared expert depends on x only, so when it has GEMM launches of its
 * own (formats of its own, or the large-tile path of prefill batches:
 * hy3moe_ws_layout.shared_meta != 0) they run on a side stream that the
 * library creates on its first such call on each device (default
 * priority), beside the routing chain on `stream`: forked from
 * `stream` by an event after x is quantised and joined back into it by
 * another before the combine (the CANN deployment article, section 8.5, and
 * the hy3 README's performance notes run shared and routed experts on two
 * streams).  Everything the call enqueues is ordered before work later
 * enqueued on `stream`; under HIP graph capture of `stream` the fork and
 * join become graph edges.  A call made while `stream` is being captured
 * before the side stream exists keeps the shared expert on `stream`.
 * Results are identical either way.  Calls from several host threads on one
 * device enqueue their fork and join under a lock and share the side
 * stream. */
int hy3moe_forward(const hy3moe_config *cfg, const void *x, const hy3moe_weights *w,
                   void *out, int32_t *idx_out, float *weight_out,
                   void *workspace, size_t ws_bytes, void *stream);

/* Stages of hy3moe_forward on `stream`, in launch order: router GEMM (with
 * act_format FP8_STATIC or MXFP8 preceded by the quantisation of x),
 * score+select, permutation (histogram, scan + tile list, scatter),
 * gate-up + SwiGLU, down (with MXFP8 off the large-tile path preceded by
 * the quantisation of h), combine (preceded by the join of the side
 * stream).  When the shared expert runs on the side stream (shared_meta !=
 * 0) the gate-up and down stages are the routed experts' GEMMs alone. */
#define HY3MOE_N_STAGES 6

/* hy3moe_forward that also records HY3MOE_N_STAGES + 1 caller-created HIP
 * events (hipEvent_t handles, passed as void*) on `stream`: stage_events[0]
 * before the first kernel and stage_events[i + 1] after stage i, so that
 * hipEventElapsedTime between consecutive events gives each stage's duration
 * on the stream the kernels run on.  Used for per-kernel timing; results are
 * identical to hy3moe_forward.  Returns HY3MOE_ERR_INVALID if any event is
 * NULL; otherwise as hy3moe_forward. */
int hy3moe_forward_timed(const hy3moe_config *cfg, const void *x, const hy3moe_weights *w,
                         void *out, int32_t *idx_out, float *weight_out,
                         void *workspace, size_t ws_bytes, void *stream,
                         void *const *stage_events);

/* hy3moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Identical results to hy3moe_forward, with every kernel on `stream` (no
 * side stream); the workspace is a static device
 * array of HY3MOE_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on
 * each GPU it runs on until the process ends (its address is looked up on
 * the first call on a device), so the call itself allocates nothing.
 *   x, w, out, idx_out, weight_out, stream: as hy3moe_forward.
 * Batches whose forward workspace (hy3moe_workspace_bytes(cfg, 1)) exceeds
 * the array return HY3MOE_ERR_SCRATCH before anything is launched (the Hy3
 * layer fits up to about 350 tokens: decode batches).  Nothing in the array
 * needs clearing between calls: every kernel writes what a later one reads.
 * All calls on one GPU share its array: calls that overlap on a GPU (other
 * streams, other threads) race and give undefined results; the caller must
 * order them. */
#define HY3MOE_STATIC_SCRATCH_BYTES (64u << 20)
int hy3moe_forward_static(const hy3moe_config *cfg, const void *x, const hy3moe_weights *w,
                          void *out, int32_t *idx_out, float *weight_out, void *stream);
/* == HY3MOE_STATIC_SCRATCH_BYTES */
size_t hy3moe_static_scratch_bytes(void);

/* Static FP8 activation quantisation on its own: q[i] = E4M3(x[i] / *scale)
 * for i < n, as act_format FP8_STATIC quantises the experts' input (the CANN
 * deployment article, section 六, FP8 path: static per-tensor input scale).
 *   x      [n] dtype (HY3MOE_BF16 or HY3MOE_F32), device, 16-byte aligned
 *   scale  [1] fp32, device, 4-byte aligned (read on the device: no sync)
 *   q      [n] uint8 out, device, 16-byte aligned: OCP E4M3 codes
 * Quotient a correctly rounded float32 division, clamped to +-448, rounded to
 * nearest even.  Errors: HY3MOE_ERR_INVALID (n < 0, bad dtype, null pointer
 * with n > 0), HY3MOE_ERR_ALIGN.  n == 0 is a no-op. */
int hy3moe_quantize_e4m3(const void *x, int32_t dtype, int64_t n, const float *scale, uint8_t *q,
                         void *stream);

/* Human-readable text of a return code (static storage). */
const char *hy3moe_strerror(int code);

/* Library ABI version (increments on any change of the structs above). */
int hy3moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HY3MOE_H */
