// C ABI of the MoE layer: validation, workspace layout and the launch chain.
//
// The chain, all on the caller's stream with no host synchronisation and no
// device-to-host copy (routing counts stay on the device; the expert GEMM
// grids are sized by an upper bound and surplus workgroups exit at once):
//   router GEMM -> score/select -> permutation (hist, scan+tiles, scatter)
//   -> grouped gate-up + SwiGLU -> grouped down -> weighted combine.
#include <string.h>

#include <mutex>

#include "hy3moe.h"
#include "internal.h"

using namespace hy3moe;

namespace {

constexpr size_t ALIGN = 256;

size_t al(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

int elt_bytes(int dtype) { return dtype == HY3MOE_F32 ? 4 : 2; }

// Formats of one branch of the layer: the routed experts, or the shared
// expert (its own formats when shared_w_format / shared_act_format are set).
struct BranchFmt {
  int w, act;
  bool operator!=(const BranchFmt &o) const { return w != o.w || act != o.act; }
};
BranchFmt routed_fmt(const hy3moe_config *c) { return {c->w_format, c->act_format}; }
BranchFmt shared_fmt(const hy3moe_config *c) {
  return {c->shared_w_format == HY3MOE_FMT_AS_ROUTED ? c->w_format : c->shared_w_format,
          c->shared_act_format == HY3MOE_FMT_AS_ROUTED ? c->act_format : c->shared_act_format};
}
// Does the shared expert run in formats of its own (separate GEMM launches)?
bool mixed(const hy3moe_config *c) { return c->I_shared > 0 && shared_fmt(c) != routed_fmt(c); }

// The format rules of one branch whose expert intermediate size is Ib.
int validate_fmt(const hy3moe_config *c, BranchFmt f, int Ib) {
  if (f.w != HY3MOE_WFMT_DTYPE && f.w != HY3MOE_WFMT_FP8_E4M3 && f.w != HY3MOE_WFMT_MXFP4)
    return HY3MOE_ERR_INVALID;
  if (f.act != HY3MOE_AFMT_DTYPE && f.act != HY3MOE_AFMT_FP8_STATIC && f.act != HY3MOE_AFMT_MXFP8)
    return HY3MOE_ERR_INVALID;
  // FP8 and MXFP4 expert weights need bf16 activations.
  if (f.w != HY3MOE_WFMT_DTYPE && c->dtype != HY3MOE_BF16) return HY3MOE_ERR_UNSUPPORTED;
  // MXFP4: 128 K values per 64-byte step of a streamed weight row.
  if (f.w == HY3MOE_WFMT_MXFP4 && (c->H % 128 || Ib % 128)) return HY3MOE_ERR_UNSUPPORTED;
  // Dynamic MXFP8 activations go with MXFP4 weights, static FP8 with FP8.
  if (f.act == HY3MOE_AFMT_MXFP8 && f.w != HY3MOE_WFMT_MXFP4) return HY3MOE_ERR_UNSUPPORTED;
  if (f.act == HY3MOE_AFMT_FP8_STATIC && f.w != HY3MOE_WFMT_FP8_E4M3)
    return HY3MOE_ERR_UNSUPPORTED;
  return HY3MOE_OK;
}

int validate_cfg(const hy3moe_config *c) {
  if (!c) return HY3MOE_ERR_INVALID;
  if (c->T < 0 || c->E < 1 || c->E > 256 || c->K < 1 || c->K > c->E || c->K > 64)
    return HY3MOE_ERR_INVALID;
  if (c->H < 1 || c->I < 1 || c->I_shared < 0) return HY3MOE_ERR_INVALID;
  if (c->dtype != HY3MOE_F32 && c->dtype != HY3MOE_BF16) return HY3MOE_ERR_INVALID;
  if (c->route_mode != HY3MOE_ROUTE_SIGMOID_BIAS && c->route_mode != HY3MOE_ROUTE_SOFTMAX)
    return HY3MOE_ERR_INVALID;
  if (c->router_prec != HY3MOE_ROUTER_FP32 && c->router_prec != HY3MOE_ROUTER_SPLIT2_BF16)
    return HY3MOE_ERR_INVALID;
  if (c->H % 64 || c->I % 64 || c->I_shared % 64) return HY3MOE_ERR_UNSUPPORTED;
  if (c->H > 65536 || c->I > 65536 || c->I_shared > 65536) return HY3MOE_ERR_UNSUPPORTED;
  if (c->T > (int64_t(1) << 24)) return HY3MOE_ERR_UNSUPPORTED;
  if (c->router_prec == HY3MOE_ROUTER_SPLIT2_BF16 && c->dtype != HY3MOE_BF16)
    return HY3MOE_ERR_UNSUPPORTED;
  if ((c->shared_w_format < HY3MOE_FMT_AS_ROUTED) || (c->shared_act_format < HY3MOE_FMT_AS_ROUTED))
    return HY3MOE_ERR_INVALID;
  int rc = validate_fmt(c, routed_fmt(c), c->I);
  if (rc != HY3MOE_OK) return rc;
  if (c->I_shared > 0) {
    rc = validate_fmt(c, shared_fmt(c), c->I_shared);
    if (rc != HY3MOE_OK) return rc;
  }
  // The expert GEMMs address x and every expert matrix with 32-bit offsets.
  const uint64_t eb = c->dtype == HY3MOE_F32 ? 4 : 2, lim = uint64_t(1) << 32;
  const uint64_t Imax = c->I > c->I_shared ? c->I : c->I_shared;
  if ((uint64_t)c->T * c->H * eb >= lim || (uint64_t)c->H * Imax * eb >= lim)
    return HY3MOE_ERR_UNSUPPORTED;
  return HY3MOE_OK;
}

// GEMM path of a layer call: static FP8 activations run the large-tile
// path's FP8 MFMAs, whose 128-value K stages need H and the branch's
// intermediate size % 128 == 0.
int path_of(const hy3moe_config *c) {
  const bool r_ok = c->act_format != HY3MOE_AFMT_FP8_STATIC || (c->H % 128 == 0 && c->I % 128 == 0);
  const bool s_ok = c->I_shared == 0 || shared_fmt(c).act != HY3MOE_AFMT_FP8_STATIC ||
                    (c->H % 128 == 0 && c->I_shared % 128 == 0);
  return expert_path(c->T, c->K, c->E, r_ok && s_ok);
}

void compute_layout(const hy3moe_config *c, int for_forward, hy3moe_ws_layout *L) {
  memset(L, 0, sizeof(*L));
  const int64_t T = c->T;
  const int E = c->E, K = c->K, H = c->H;
  const int64_t N = T * K;
  size_t off = 0;
  L->n_ksplit = router_ksplit(T, H, E, c->dtype);
  L->logits_part = off; off += al((size_t)L->n_ksplit * T * E * 8);
  L->idx = off;         off += al((size_t)N * 4);
  L->weight = off;      off += al((size_t)N * 4);
  if (router_use_planes(T, c->dtype)) {
    L->w_planes = off;  off += al((size_t)3 * ((E + 15) / 16 * 16) * H * 2);
  }
  if (!for_forward) { L->total = off; return; }
  L->n_chunks = (int32_t)((N + PERM_CHUNK - 1) / PERM_CHUNK);
  L->hist = off;        off += al((size_t)L->n_chunks * E * 4);
  L->counts = off;      off += al((size_t)(E + 1) * 4);
  L->offsets = off;     off += al((size_t)(E + 2) * 4);
  const int64_t T_sh = c->I_shared > 0 ? T : 0;
  const int64_t R = N + T_sh;
  L->sorted_token = off; off += al((size_t)R * 4);
  L->pos_of = off;      off += al((size_t)N * 4);
  const int path = path_of(c);
  L->gemm_path = path;
  // static FP8 activations as E4M3 codes for FP8 MFMAs: the large-tile path,
  // and weight streaming when every K (H, I, I_shared) is a multiple of 128
  L->a8_codes = path == PATH_BIG ||
                (path == PATH_SKINNY && c->H % 128 == 0 && c->I % 128 == 0 &&
                 c->I_shared % 128 == 0);
  if (path == PATH_SKINNY) {
    L->tile_rows = SKINNY_ROWS;
  } else {
    L->tile_rows = path == PATH_BIG ? BIG_ROWS : TILED_ROWS;
  }
  L->max_tiles = (int32_t)((R + L->tile_rows - 1) / L->tile_rows + E + 1);
  L->tiles = off;       off += al((size_t)(2 * L->max_tiles + 2) * 4);
  const int Imax = c->I > c->I_shared ? c->I : c->I_shared;
  const int eb = elt_bytes(c->dtype);
  L->h = off;           off += al((size_t)R * Imax * eb);
  L->y = off;           off += al((size_t)R * H * eb);  // fp16 (bf16 layers) or float32
  // quantised x of the routed branch (xq, xs) and, with formats of its own,
  // of the shared branch (xq_shared, xs_shared); MXFP8 codes of h (hq, hs)
  const BranchFmt rf = routed_fmt(c), sf = shared_fmt(c);
  const bool mix = mixed(c);
  if (rf.act != HY3MOE_AFMT_DTYPE || (!mix && sf.act != HY3MOE_AFMT_DTYPE)) {
    L->xq = off;        off += al((size_t)T * H * 2);
  }
  if (rf.act == HY3MOE_AFMT_MXFP8) {
    L->xs = off;        off += al((size_t)T * H / 32);
  }
  if (mix && sf.act != HY3MOE_AFMT_DTYPE) {
    L->xq_shared = off; off += al((size_t)T * H * 2);
    if (sf.act == HY3MOE_AFMT_MXFP8) {
      L->xs_shared = off; off += al((size_t)T * H / 32);
    }
  }
  if (rf.act == HY3MOE_AFMT_MXFP8 || (c->I_shared > 0 && sf.act == HY3MOE_AFMT_MXFP8)) {
    L->hq = off;        off += al((size_t)R * Imax);
    L->hs = off;        off += al((size_t)R * Imax / 32);
  }
  // the shared expert's own tile list, offsets and row map, for launches
  // beside the routing chain: when it has launches of its own anyway
  // (formats of its own) and on the large-tile path.  A weight-streaming
  // launch of one group has too little parallelism to gain from it and
  // holds CUs the routing kernels need; there the shared expert stays a
  // group of the routed experts' launches.
  if (c->I_shared > 0 && (mix || path == PATH_BIG)) {
    L->shared_meta = off;
    off += al((size_t)(2 * L->max_tiles + 2 + E + 2 + R) * 4);
  }
  L->total = off;
}

bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool al4(const void *p) { return ((uintptr_t)p & 3) == 0; }

int check_launch(hipError_t e) { return e == hipSuccess ? HY3MOE_OK : HY3MOE_ERR_HIP; }

// The side stream of each device: the shared expert's branch runs on it,
// forked from and joined back into the caller's stream by two events.
// Created on the first hy3moe_forward on the device (not while the caller's
// stream is being captured: such a call stays on the caller's stream);
// default priority.  The lock is held while a call enqueues its fork and
// join, so calls from several host threads do not interleave them.
constexpr int kMaxSideDevices = 64;
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int state = 0;   // 0 not created, 1 ready, -1 creation failed
};
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// The current device's side stream with *lock holding g_side_mu, or null
// (then the shared expert runs on the caller's stream).
SideStream *side_stream(hipStream_t caller, std::unique_lock<std::mutex> *lock) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return nullptr;
  std::unique_lock<std::mutex> lk(g_side_mu);
  SideStream &sd = g_side[dev];
  if (sd.state == 0) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
      return nullptr;
    const bool ok = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking) == hipSuccess &&
                    hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming) == hipSuccess &&
                    hipEventCreateWithFlags(&sd.join, hipEventDisableTiming) == hipSuccess;
    sd.state = ok ? 1 : -1;
  }
  if (sd.state != 1) return nullptr;
  *lock = std::move(lk);
  return &sd;
}

}  // namespace

extern "C" {

int hy3moe_abi_version(void) { return 12; }

const char *hy3moe_strerror(int code) {
  switch (code) {
    case HY3MOE_OK: return "ok";
    case HY3MOE_ERR_INVALID: return "invalid argument";
    case HY3MOE_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
    case HY3MOE_ERR_WORKSPACE: return "workspace too small";
    case HY3MOE_ERR_ALIGN: return "pointer not aligned (16 bytes for tensors, 4 for idx/weight/bias)";
    case HY3MOE_ERR_HIP: return "HIP kernel launch failed";
    case HY3MOE_ERR_SCRATCH:
      return "batch needs more scratch than hy3moe_forward_static's static array holds "
             "(use hy3moe_forward with a workspace)";
    default: return "unknown error code";
  }
}

size_t hy3moe_workspace_bytes(const hy3moe_config *cfg, int for_forward) {
  if (validate_cfg(cfg) != HY3MOE_OK) return 0;
  hy3moe_ws_layout L;
  compute_layout(cfg, for_forward, &L);
  return L.total;
}

int hy3moe_workspace_layout(const hy3moe_config *cfg, hy3moe_ws_layout *out) {
  const int rc = validate_cfg(cfg);
  if (rc != HY3MOE_OK) return rc;
  if (!out) return HY3MOE_ERR_INVALID;
  compute_layout(cfg, 1, out);
  return HY3MOE_OK;
}

size_t hy3moe_router_planes_bytes(int32_t E, int32_t H, int32_t router_prec) {
  if (E < 1 || E > 256 || H < 64 || H % 64 || H > 65536 ||
      (router_prec != HY3MOE_ROUTER_FP32 && router_prec != HY3MOE_ROUTER_SPLIT2_BF16))
    return 0;
  return router_planes_bytes(E, H, router_prec);
}

int hy3moe_router_split(const float *w_router, int32_t E, int32_t H, int32_t router_prec,
                        void *planes, size_t planes_bytes, void *stream) {
  if (E < 1 || E > 256 || H < 1 || !w_router || !planes ||
      (router_prec != HY3MOE_ROUTER_FP32 && router_prec != HY3MOE_ROUTER_SPLIT2_BF16))
    return HY3MOE_ERR_INVALID;
  if (H % 64 || H > 65536) return HY3MOE_ERR_UNSUPPORTED;
  if (planes_bytes < router_planes_bytes(E, H, router_prec)) return HY3MOE_ERR_WORKSPACE;
  if (!al16(w_router) || !al16(planes)) return HY3MOE_ERR_ALIGN;
  return check_launch(launch_router_split(w_router, router_prec, static_cast<uint16_t *>(planes),
                                          E, H, static_cast<hipStream_t>(stream)));
}

int hy3moe_route(const hy3moe_config *cfg, const void *x, const float *w_router,
                 const float *expert_bias, int32_t *idx, float *weight, void *workspace,
                 size_t ws_bytes, void *stream) {
  return hy3moe_route_planes(cfg, x, w_router, nullptr, expert_bias, idx, weight, workspace,
                             ws_bytes, stream);
}

int hy3moe_route_planes(const hy3moe_config *cfg, const void *x, const float *w_router,
                        const void *w_router_planes, const float *expert_bias, int32_t *idx,
                        float *weight, void *workspace, size_t ws_bytes, void *stream) {
  int rc = validate_cfg(cfg);
  if (rc != HY3MOE_OK) return rc;
  if (cfg->T == 0) return HY3MOE_OK;
  if (!x || !w_router || !idx || !weight || !workspace) return HY3MOE_ERR_INVALID;
  if (!al16(x) || !al16(w_router) || !al16(workspace) || !al4(idx) || !al4(weight) ||
      (expert_bias && !al4(expert_bias)) || (w_router_planes && !al16(w_router_planes)))
    return HY3MOE_ERR_ALIGN;
  hy3moe_ws_layout L;
  compute_layout(cfg, 0, &L);
  if (ws_bytes < L.total) return HY3MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  const int T = (int)cfg->T;
  double *part = reinterpret_cast<double *>(ws + L.logits_part);
  uint16_t *planes = L.w_planes ? reinterpret_cast<uint16_t *>(ws + L.w_planes) : nullptr;
  rc = check_launch(launch_router(x, cfg->dtype, cfg->router_prec, w_router, planes,
                                  static_cast<const uint16_t *>(w_router_planes), part, T,
                                  cfg->H, cfg->E, L.n_ksplit, s));
  if (rc) return rc;
  const float *bias = cfg->route_mode == HY3MOE_ROUTE_SIGMOID_BIAS ? expert_bias : nullptr;
  return check_launch(launch_select(part, L.n_ksplit, T, cfg->E, cfg->K, bias, cfg->route_mode,
                                    cfg->scale, cfg->renorm_eps, idx, weight, s));
}

// Pointer and alignment checks of one branch's weights (routed: the stacked
// tensors; shared: the shared expert's).
static int check_branch_weights(const hy3moe_weights *w, BranchFmt f, bool shared) {
  if (f.w == HY3MOE_WFMT_FP8_E4M3) {
    if (shared) {
      if (!w->ws_scale) return HY3MOE_ERR_INVALID;
      if (!al4(w->ws_scale)) return HY3MOE_ERR_ALIGN;
    } else {
      if (!w->w_gate_scale || !w->w_up_scale || !w->w_down_scale) return HY3MOE_ERR_INVALID;
      if (!al4(w->w_gate_scale) || !al4(w->w_up_scale) || !al4(w->w_down_scale))
        return HY3MOE_ERR_ALIGN;
    }
  }
  if (f.w == HY3MOE_WFMT_MXFP4) {
    const uint8_t *g = shared ? w->ws_gate_mx : w->w_gate_mx, *u = shared ? w->ws_up_mx : w->w_up_mx,
                  *d = shared ? w->ws_down_mx : w->w_down_mx;
    if (!g || !u || !d) return HY3MOE_ERR_INVALID;
    if (!al16(g) || !al16(u) || !al16(d)) return HY3MOE_ERR_ALIGN;
  }
  if (f.act == HY3MOE_AFMT_FP8_STATIC) {
    if (!w->x_scale || !w->h_scale) return HY3MOE_ERR_INVALID;
    if (!al4(w->x_scale) || !al4(w->h_scale)) return HY3MOE_ERR_ALIGN;
  }
  return HY3MOE_OK;
}

// The format-dependent fields of one branch's expert GEMM (gate-up or down).
static void set_branch_weights(ExpertArgs &ea, const hy3moe_weights *w, BranchFmt f,
                               bool gate_up, bool has_shared) {
  const bool fp8 = f.w == HY3MOE_WFMT_FP8_E4M3, fp4 = f.w == HY3MOE_WFMT_MXFP4;
  const bool a8 = f.act == HY3MOE_AFMT_FP8_STATIC;
  ea.w0 = gate_up ? w->w_gate : w->w_down;
  ea.w1 = gate_up ? w->w_up : nullptr;
  ea.ws0 = gate_up ? w->ws_gate : w->ws_down;
  ea.ws1 = gate_up ? w->ws_up : nullptr;
  ea.w_fp8 = fp8 ? 1 : 0;
  ea.sc0 = fp8 ? (gate_up ? w->w_gate_scale : w->w_down_scale) : nullptr;
  ea.sc1 = fp8 && gate_up ? w->w_up_scale : nullptr;
  ea.ssc0 = fp8 && has_shared ? w->ws_scale + (gate_up ? 0 : 2) : nullptr;
  ea.ssc1 = fp8 && has_shared && gate_up ? w->ws_scale + 1 : nullptr;
  ea.a8 = a8 ? 1 : 0;
  ea.xs = a8 ? w->x_scale : nullptr;
  ea.hs = a8 ? w->h_scale : nullptr;
  ea.w_fp4 = fp4 ? 1 : 0;
  ea.mx0 = fp4 ? (gate_up ? w->w_gate_mx : w->w_down_mx) : nullptr;
  ea.mx1 = fp4 && gate_up ? w->w_up_mx : nullptr;
  ea.mxs0 = fp4 && has_shared ? (gate_up ? w->ws_gate_mx : w->ws_down_mx) : nullptr;
  ea.mxs1 = fp4 && has_shared && gate_up ? w->ws_up_mx : nullptr;
}

static int forward_impl(const hy3moe_config *cfg, const void *x, const hy3moe_weights *w,
                        void *out, int32_t *idx_out, float *weight_out, void *workspace,
                        size_t ws_bytes, void *stream, void *const *events, bool overlap) {
  int rc = validate_cfg(cfg);
  if (rc != HY3MOE_OK) return rc;
  if (cfg->T == 0) return HY3MOE_OK;
  if (!x || !w || !out || !workspace || !w->w_router || !w->w_gate || !w->w_up || !w->w_down)
    return HY3MOE_ERR_INVALID;
  const bool has_shared = cfg->I_shared > 0;
  if (has_shared && (!w->ws_gate || !w->ws_up || !w->ws_down)) return HY3MOE_ERR_INVALID;
  if (x == out) return HY3MOE_ERR_INVALID;
  if (!al16(x) || !al16(out) || !al16(workspace) || !al16(w->w_router) || !al16(w->w_gate) ||
      !al16(w->w_up) || !al16(w->w_down) || (w->expert_bias && !al4(w->expert_bias)) ||
      (idx_out && !al4(idx_out)) || (weight_out && !al4(weight_out)) ||
      (w->w_router_planes && !al16(w->w_router_planes)))
    return HY3MOE_ERR_ALIGN;
  if (has_shared && (!al16(w->ws_gate) || !al16(w->ws_up) || !al16(w->ws_down)))
    return HY3MOE_ERR_ALIGN;
  const BranchFmt rf = routed_fmt(cfg), sf = shared_fmt(cfg);
  const bool mix = mixed(cfg);
  rc = check_branch_weights(w, rf, false);
  if (rc == HY3MOE_OK && has_shared) rc = check_branch_weights(w, sf, true);
  if (rc != HY3MOE_OK) return rc;
  hy3moe_ws_layout L;
  compute_layout(cfg, 1, &L);
  if (ws_bytes < L.total) return HY3MOE_ERR_WORKSPACE;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  const int T = (int)cfg->T, H = cfg->H, E = cfg->E, K = cfg->K;
  double *part = reinterpret_cast<double *>(ws + L.logits_part);
  uint16_t *planes = L.w_planes ? reinterpret_cast<uint16_t *>(ws + L.w_planes) : nullptr;
  int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(ws + L.idx);
  float *weight = weight_out ? weight_out : reinterpret_cast<float *>(ws + L.weight);

  // The shared expert needs x only, not the route: with a side stream it
  // runs there, beside the routing chain (the CANN deployment article,
  // section 8.5, and the hy3 README's performance notes put the shared and
  // routed experts on two streams).
  std::unique_lock<std::mutex> side_lock;
  SideStream *side = (overlap && L.shared_meta) ? side_stream(s, &side_lock) : nullptr;

  int stage = 0;
  auto mark = [&]() {
    if (events) hipEventRecord(static_cast<hipEvent_t>(events[stage]), s);
    ++stage;
  };

  // A branch is the routed experts (group selection GRP_ROUTED), or the
  // shared expert (GRP_SHARED) when it runs on the side stream or has
  // formats of its own; otherwise one launch per GEMM covers both (GRP_ALL).
  const int path = path_of(cfg);
  const int Imax = cfg->I > cfg->I_shared ? cfg->I : cfg->I_shared;
  const int64_t N = (int64_t)T * K;
  const int64_t R = N + (has_shared ? T : 0);
  const bool split = has_shared && (mix || side);
  struct Branch {
    BranchFmt f;
    int grp_sel;
    int64_t r0, r1;            // its rows of h and y
    hipStream_t st;            // the stream it runs on
    const void *act;           // its x: as given, or quantised
    const uint8_t *act_sc;     // MXFP8 scales of its x
    char *xq;                  // where its quantised x goes
    uint8_t *xs;
    int32_t *tiles, *offsets, *sorted_token;   // its tile list and row maps
  };
  int32_t *meta = L.shared_meta ? reinterpret_cast<int32_t *>(ws + L.shared_meta) : nullptr;
  Branch br[2];
  const int nbr = split ? 2 : 1;
  br[0] = {rf, split ? GRP_ROUTED : GRP_ALL, 0, split ? N : R, s, x, nullptr, ws + L.xq,
           reinterpret_cast<uint8_t *>(ws + L.xs), reinterpret_cast<int32_t *>(ws + L.tiles),
           reinterpret_cast<int32_t *>(ws + L.offsets),
           reinterpret_cast<int32_t *>(ws + L.sorted_token)};
  if (split) {
    br[1] = {sf, GRP_SHARED, N, R, side ? side->s : s, x, nullptr,
             mix ? ws + L.xq_shared : ws + L.xq,
             reinterpret_cast<uint8_t *>(mix ? ws + L.xs_shared : ws + L.xs), br[0].tiles,
             br[0].offsets, br[0].sorted_token};
    if (side) {   // its own metadata, written on the side stream
      br[1].tiles = meta;
      br[1].offsets = meta + 2 * L.max_tiles + 2;
      br[1].sorted_token = br[1].offsets + E + 2;
    }
  }

  // Quantisation of x for a branch that quantises its activations: MXFP8
  // codes and scales for the block-scaled MFMAs of the weight-streaming and
  // large-tile paths (bf16 values for the tiled path); static FP8 code bytes
  // for the large-tile path's FP8 MFMAs, else their bf16 values.
  // The quantisation quantise_x launches, as the select launch can host it.
  auto hosted_quant = [&](const Branch &B) {
    HostedQuant h;
    if (B.f.act == HY3MOE_AFMT_MXFP8) {
      h.mode = QH_MXFP8;
      h.carrier = path != PATH_TILED ? 0 : 1;
      h.scales = B.xs;
    } else if (B.f.act == HY3MOE_AFMT_FP8_STATIC) {
      h.mode = QH_E4M3;
      h.carrier = L.a8_codes ? 0 : 1;
      h.scale = w->x_scale;
    }
    h.x = x;
    h.dtype = cfg->dtype;
    h.n = (int64_t)T * H;
    h.q = B.xq;
    return h;
  };
  auto quantise_x = [&](Branch &B) -> int {
    int e = HY3MOE_OK;
    if (B.f.act == HY3MOE_AFMT_MXFP8) {
      e = check_launch(launch_quant_mxfp8(x, (int64_t)T * H, B.xq, B.xs,
                                          path != PATH_TILED ? 0 : 1, B.st));
      B.act_sc = B.xs;
    } else if (B.f.act == HY3MOE_AFMT_FP8_STATIC) {
      e = check_launch(launch_quant_e4m3(x, cfg->dtype, (int64_t)T * H, w->x_scale, B.xq,
                                         L.a8_codes ? 0 : 1, B.st));
    }
    if (B.f.act != HY3MOE_AFMT_DTYPE) B.act = B.xq;
    return e;
  };

  // The expert GEMMs of one branch.  h of every branch shares one buffer by
  // rows; a branch that stores 1-byte codes there (static FP8 on the
  // large-tile path: row r at byte r * ldh) is shifted by r0 * ldh bytes,
  // past the 2-byte rows before it, when the formats differ.  On the
  // large-tile path MXFP8 h is quantised by the gate-up epilogue itself.
  ExpertArgs base;
  base.E = E; base.H = H; base.I = cfg->I; base.I_shared = cfg->I_shared; base.ldh = Imax;
  base.max_tiles = L.max_tiles;
  base.n_rows = (int)R;
  base.n_tok = T;
  base.a8_codes = L.a8_codes;
  auto branch_args = [&](const Branch &B, bool gate_up) {
    ExpertArgs ea = base;
    ea.sorted_token = B.sorted_token;
    ea.offsets = B.offsets;
    ea.tiles = B.tiles;
    set_branch_weights(ea, w, B.f, gate_up, has_shared);
    ea.grp_sel = B.grp_sel;
    return ea;
  };
  auto h_base = [&](const Branch &B) {
    return ws + L.h + (B.f.act == HY3MOE_AFMT_FP8_STATIC && L.a8_codes && mix
                           ? B.r0 * Imax : 0);
  };
  auto gate_up = [&](const Branch &B) -> int {
    const bool amx = B.f.act == HY3MOE_AFMT_MXFP8;
    const bool amx_codes = amx && path != PATH_TILED, fused = amx_codes && path == PATH_BIG;
    ExpertArgs ea = branch_args(B, true);
    ea.act = B.act;
    ea.amx = amx_codes ? 1 : 0;
    ea.act_sc = amx ? B.act_sc : nullptr;
    ea.out = fused ? ws + L.hq : h_base(B);
    ea.out_sc = fused ? reinterpret_cast<uint8_t *>(ws + L.hs) : nullptr;
    return check_launch(launch_gate_up(ea, cfg->dtype, path, B.st));
  };
  auto down = [&](const Branch &B) -> int {
    const bool amx = B.f.act == HY3MOE_AFMT_MXFP8;
    const bool amx_codes = amx && path != PATH_TILED, fused = amx_codes && path == PATH_BIG;
    ExpertArgs ea = branch_args(B, false);
    ea.act = h_base(B);
    ea.amx = amx_codes ? 1 : 0;
    ea.act_sc = nullptr;
    ea.out_sc = nullptr;
    if (amx) {
      // h, dynamic MXFP8 per 32 along I over the branch's rows: codes and
      // scales, or the bf16 values in place
      const int64_t h0 = B.r0 * Imax, nh = (B.r1 - B.r0) * Imax;
      int e = HY3MOE_OK;
      if (!fused && amx_codes)
        e = check_launch(launch_quant_mxfp8(ws + L.h + h0 * 2, nh, ws + L.hq + h0,
                                            reinterpret_cast<uint8_t *>(ws + L.hs) + h0 / 32, 0,
                                            B.st));
      else if (!fused)
        e = check_launch(launch_quant_mxfp8(ws + L.h + h0 * 2, nh, ws + L.h + h0 * 2, nullptr,
                                            1, B.st));
      if (e) return e;
      if (amx_codes) {
        ea.act = ws + L.hq;
        ea.act_sc = reinterpret_cast<const uint8_t *>(ws + L.hs);
      }
    }
    ea.out = ws + L.y;
    return check_launch(launch_down(ea, cfg->dtype, path, B.st));
  };

  mark();
  // 0. x quantised once for the routed experts (and for the shared expert
  // when it shares their format), before the fork.  A weight-streaming
  // batch with one branch has the select launch host it instead (one launch
  // fewer on the decode chain).
  HostedQuant hq;
  if (path == PATH_SKINNY && !split && br[0].f.act != HY3MOE_AFMT_DTYPE) {
    hq = hosted_quant(br[0]);
    br[0].act = br[0].xq;
    if (br[0].f.act == HY3MOE_AFMT_MXFP8) br[0].act_sc = br[0].xs;
  } else {
    rc = quantise_x(br[0]);
    if (rc) return rc;
  }
  if (split && !mix) {
    br[1].act = br[0].act;
    br[1].act_sc = br[0].act_sc;
  }
  bool joined = true;
  if (side) {
    // fork: the shared expert's metadata, x quantisation (formats of its
    // own) and GEMMs on the side stream; the caller's stream waits for the
    // join before the combine (or before returning an error)
    hipStream_t ss = side->s;
    rc = check_launch(hipEventRecord(side->fork, s));
    if (!rc) rc = check_launch(hipStreamWaitEvent(ss, side->fork, 0));
    if (rc) return rc;
    joined = false;
    rc = check_launch(launch_shared_meta(br[1].tiles, br[1].offsets, br[1].sorted_token, T,
                                         (int)N, E, L.tile_rows, L.max_tiles, ss));
    if (!rc && mix) rc = quantise_x(br[1]);
    if (!rc) rc = gate_up(br[1]);
    if (!rc) rc = down(br[1]);
    const int jr = check_launch(hipEventRecord(side->join, ss));
    if (!rc) rc = jr;
  }
  auto join = [&]() -> int {
    if (joined) return HY3MOE_OK;
    joined = true;
    return check_launch(hipStreamWaitEvent(s, side->join, 0));
  };
  auto fail = [&](int e) {
    join();
    return e;
  };
  if (rc) return fail(rc);

  // 1-2. gate
  rc = check_launch(launch_router(x, cfg->dtype, cfg->router_prec, w->w_router, planes,
                                  static_cast<const uint16_t *>(w->w_router_planes), part, T, H,
                                  E, L.n_ksplit, s));
  if (rc) return fail(rc);
  mark();
  const float *bias = cfg->route_mode == HY3MOE_ROUTE_SIGMOID_BIAS ? w->expert_bias : nullptr;
  rc = check_launch(launch_select(part, L.n_ksplit, T, E, K, bias, cfg->route_mode, cfg->scale,
                                  cfg->renorm_eps, idx, weight, s, hq));
  if (rc) return fail(rc);
  mark();

  // 3. the shared expert's x in formats of its own when it stays on this
  // stream, then the permutation (the shared expert's tiles last when it
  // has launches of its own)
  if (split && !side && mix) {
    rc = quantise_x(br[1]);
    if (rc) return fail(rc);
  }
  PermArgs pa;
  pa.idx = idx;
  pa.hist = reinterpret_cast<int32_t *>(ws + L.hist);
  pa.counts = reinterpret_cast<int32_t *>(ws + L.counts);
  pa.offsets = br[0].offsets;
  pa.sorted_token = br[0].sorted_token;
  pa.pos_of = reinterpret_cast<int32_t *>(ws + L.pos_of);
  pa.tiles = br[0].tiles;
  pa.T = T; pa.K = K; pa.E = E;
  pa.T_shared = has_shared ? T : 0;
  pa.nchunks = L.n_chunks;
  pa.tile_rows = L.tile_rows;
  pa.max_tiles = L.max_tiles;
  pa.sort_tiles = path != PATH_SKINNY;
  pa.shared_last = split ? 1 : 0;
  rc = check_launch(launch_permute(pa, s));
  if (rc) return fail(rc);
  mark();

  // 4-5. grouped experts of the branches on this stream
  const int nb_here = side ? 1 : nbr;
  for (int b = 0; b < nb_here; ++b) {
    rc = gate_up(br[b]);
    if (rc) return fail(rc);
  }
  mark();
  for (int b = 0; b < nb_here; ++b) {
    rc = down(br[b]);
    if (rc) return fail(rc);
  }
  mark();

  // 6. combine, after the join
  rc = join();
  if (rc) return rc;
  rc = check_launch(launch_combine(ws + L.y, pa.pos_of, weight, pa.offsets, T, K, H, E,
                                   has_shared ? 1 : 0, out, cfg->dtype, s));
  if (rc) return rc;
  mark();
  return HY3MOE_OK;
}

}  // extern "C"

// Scratch of hy3moe_forward_static: one array per GPU, resident until the
// process ends.  Its name is a host-side stand-in in host code; the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
static __device__ __align__(256) uint8_t scratch[HY3MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, or null

// The current device's scratch address (looked up on its first use), or null
// with *rc set.
void *static_scratch(int *rc) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *rc = HY3MOE_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *rc = HY3MOE_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" {

int hy3moe_forward_static(const hy3moe_config *cfg, const void *x, const hy3moe_weights *w,
                          void *out, int32_t *idx_out, float *weight_out, void *stream) {
  const int vrc = validate_cfg(cfg);
  if (vrc != HY3MOE_OK) return vrc;
  if (cfg->T == 0) return HY3MOE_OK;
  hy3moe_ws_layout L;
  compute_layout(cfg, 1, &L);
  if (L.total > (size_t)HY3MOE_STATIC_SCRATCH_BYTES) return HY3MOE_ERR_SCRATCH;
  int rc = HY3MOE_OK;
  void *ws = static_scratch(&rc);
  if (!ws) return rc;
  // the shared expert stays on the caller's stream: no side stream is created
  return forward_impl(cfg, x, w, out, idx_out, weight_out, ws, HY3MOE_STATIC_SCRATCH_BYTES,
                      stream, nullptr, false);
}

size_t hy3moe_static_scratch_bytes(void) { return HY3MOE_STATIC_SCRATCH_BYTES; }

int hy3moe_quantize_e4m3(const void *x, int32_t dtype, int64_t n, const float *scale, uint8_t *q,
                         void *stream) {
  if (n < 0 || (dtype != HY3MOE_F32 && dtype != HY3MOE_BF16)) return HY3MOE_ERR_INVALID;
  if (n == 0) return HY3MOE_OK;
  if (!x || !scale || !q) return HY3MOE_ERR_INVALID;
  if (!al16(x) || !al16(q) || !al4(scale)) return HY3MOE_ERR_ALIGN;
  return check_launch(
      launch_quant_e4m3(x, dtype, n, scale, q, 0, static_cast<hipStream_t>(stream)));
}

int hy3moe_forward(const hy3moe_config *cfg, const void *x, const hy3moe_weights *w, void *out,
                   int32_t *idx_out, float *weight_out, void *workspace, size_t ws_bytes,
                   void *stream) {
  return forward_impl(cfg, x, w, out, idx_out, weight_out, workspace, ws_bytes, stream, nullptr,
                      true);
}

int hy3moe_forward_timed(const hy3moe_config *cfg, const void *x, const hy3moe_weights *w,
                         void *out, int32_t *idx_out, float *weight_out, void *workspace,
                         size_t ws_bytes, void *stream, void *const *stage_events) {
  if (!stage_events) return HY3MOE_ERR_INVALID;
  for (int i = 0; i <= HY3MOE_N_STAGES; ++i)
    if (!stage_events[i]) return HY3MOE_ERR_INVALID;
  return forward_impl(cfg, x, w, out, idx_out, weight_out, workspace, ws_bytes, stream,
                      stage_events, true);
}

}  // extern "C"
