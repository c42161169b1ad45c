"""Thin ctypes binding of libhy3moe.so (argument marshalling only).

Every step of the layer runs in the library's HIP kernels.  PyTorch supplies
device memory (``tensor.data_ptr()``) and the current HIP stream; nothing
here computes any part of the layer, and there is no fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch  # noqa: F401  (loads the HIP runtime the library then shares)

from .build import LIB_PATH

HY3MOE_OK = 0
HY3MOE_F32 = 0
HY3MOE_BF16 = 1
HY3MOE_ROUTE_SIGMOID_BIAS = 0
HY3MOE_ROUTE_SOFTMAX = 1
HY3MOE_ROUTER_FP32 = 0
HY3MOE_ROUTER_SPLIT2_BF16 = 1
HY3MOE_WFMT_DTYPE = 0
HY3MOE_WFMT_FP8_E4M3 = 1
HY3MOE_WFMT_MXFP4 = 2
HY3MOE_AFMT_DTYPE = 0
HY3MOE_AFMT_FP8_STATIC = 1
HY3MOE_AFMT_MXFP8 = 2
HY3MOE_FMT_AS_ROUTED = -1

HY3MOE_N_STAGES = 6
ABI_VERSION = 12          # hy3moe_abi_version() of the library this binding matches
STAGE_NAMES = ("router", "select", "permute", "gate_up", "down", "combine")

EXPORTED_SYMBOLS = (
    "hy3moe_abi_version", "hy3moe_strerror", "hy3moe_workspace_bytes",
    "hy3moe_workspace_layout", "hy3moe_route", "hy3moe_forward", "hy3moe_forward_timed",
    "hy3moe_quantize_e4m3", "hy3moe_forward_static", "hy3moe_static_scratch_bytes",
    "hy3moe_router_planes_bytes", "hy3moe_router_split", "hy3moe_route_planes",
)
HY3MOE_ERR_SCRATCH = -6


class hy3moe_config(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
        ("K", ctypes.c_int32), ("I", ctypes.c_int32), ("I_shared", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("route_mode", ctypes.c_int32),
        ("router_prec", ctypes.c_int32), ("scale", ctypes.c_float),
        ("renorm_eps", ctypes.c_float), ("w_format", ctypes.c_int32),
        ("act_format", ctypes.c_int32), ("shared_w_format", ctypes.c_int32),
        ("shared_act_format", ctypes.c_int32),
    ]


WEIGHT_NAMES = ("w_router", "expert_bias", "w_gate", "w_up", "w_down", "ws_gate", "ws_up",
                "ws_down", "w_gate_scale", "w_up_scale", "w_down_scale", "ws_scale",
                "x_scale", "h_scale", "w_gate_mx", "w_up_mx", "w_down_mx", "ws_gate_mx",
                "ws_up_mx", "ws_down_mx", "w_router_planes")


class hy3moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_NAMES]


class hy3moe_ws_layout(ctypes.Structure):
    _fields_ = [
        ("total", ctypes.c_size_t), ("logits_part", ctypes.c_size_t),
        ("n_ksplit", ctypes.c_int32), ("idx", ctypes.c_size_t), ("weight", ctypes.c_size_t),
        ("counts", ctypes.c_size_t), ("offsets", ctypes.c_size_t),
        ("sorted_token", ctypes.c_size_t), ("pos_of", ctypes.c_size_t),
        ("hist", ctypes.c_size_t), ("n_chunks", ctypes.c_int32),
        ("tiles", ctypes.c_size_t), ("max_tiles", ctypes.c_int32),
        ("tile_rows", ctypes.c_int32), ("h", ctypes.c_size_t), ("y", ctypes.c_size_t),
        ("w_planes", ctypes.c_size_t), ("xq", ctypes.c_size_t), ("xs", ctypes.c_size_t),
        ("hq", ctypes.c_size_t), ("hs", ctypes.c_size_t),
        ("xq_shared", ctypes.c_size_t), ("xs_shared", ctypes.c_size_t),
        ("shared_meta", ctypes.c_size_t), ("gemm_path", ctypes.c_int32),
        ("a8_codes", ctypes.c_int32),
    ]


class Hy3MoEError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {code} ({strerror(code)})")
        self.code = code


_LIB: Optional[ctypes.CDLL] = None


def lib_path() -> str:
    return os.environ.get("HY3MOE_LIB", LIB_PATH)


def load() -> ctypes.CDLL:
    """Load libhy3moe.so (built in-tree); raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    p = lib_path()
    if not os.path.exists(p):
        raise RuntimeError(
            f"HIP MoE library not found at {p}; build it with `python -m sparse_moe_amd.build` "
            "(or __graft_entry__.build()).  There is no fallback path.")
    L = ctypes.CDLL(p)
    L.hy3moe_abi_version.restype = ctypes.c_int
    L.hy3moe_strerror.restype = ctypes.c_char_p
    L.hy3moe_strerror.argtypes = [ctypes.c_int]
    L.hy3moe_workspace_bytes.restype = ctypes.c_size_t
    L.hy3moe_workspace_bytes.argtypes = [ctypes.POINTER(hy3moe_config), ctypes.c_int]
    L.hy3moe_workspace_layout.restype = ctypes.c_int
    L.hy3moe_workspace_layout.argtypes = [ctypes.POINTER(hy3moe_config),
                                          ctypes.POINTER(hy3moe_ws_layout)]
    L.hy3moe_route.restype = ctypes.c_int
    L.hy3moe_route.argtypes = [ctypes.POINTER(hy3moe_config), ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.hy3moe_forward.restype = ctypes.c_int
    L.hy3moe_forward.argtypes = [ctypes.POINTER(hy3moe_config), ctypes.c_void_p,
                                 ctypes.POINTER(hy3moe_weights), ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_size_t, ctypes.c_void_p]
    L.hy3moe_forward_timed.restype = ctypes.c_int
    L.hy3moe_forward_timed.argtypes = [ctypes.POINTER(hy3moe_config), ctypes.c_void_p,
                                       ctypes.POINTER(hy3moe_weights), ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.POINTER(ctypes.c_void_p)]
    L.hy3moe_router_planes_bytes.restype = ctypes.c_size_t
    L.hy3moe_router_planes_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.hy3moe_router_split.restype = ctypes.c_int
    L.hy3moe_router_split.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p]
    L.hy3moe_route_planes.restype = ctypes.c_int
    L.hy3moe_route_planes.argtypes = [ctypes.POINTER(hy3moe_config), ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]
    L.hy3moe_forward_static.restype = ctypes.c_int
    L.hy3moe_forward_static.argtypes = [ctypes.POINTER(hy3moe_config), ctypes.c_void_p,
                                        ctypes.POINTER(hy3moe_weights), ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.hy3moe_static_scratch_bytes.restype = ctypes.c_size_t
    L.hy3moe_static_scratch_bytes.argtypes = []
    L.hy3moe_quantize_e4m3.restype = ctypes.c_int
    L.hy3moe_quantize_e4m3.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.hy3attn_max_tasks.restype = ctypes.c_int64
    L.hy3attn_max_tasks.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.hy3attn_workspace_bytes.restype = ctypes.c_size_t
    L.hy3attn_workspace_bytes.argtypes = [ctypes.c_int64]
    L.hy3attn_plan.restype = ctypes.c_int
    L.hy3attn_plan.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
    L.hy3attn_decode.restype = ctypes.c_int
    L.hy3attn_decode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                 ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    if L.hy3moe_abi_version() != ABI_VERSION:
        raise RuntimeError("libhy3moe ABI version mismatch")
    _LIB = L
    return L


def strerror(code: int) -> str:
    return load().hy3moe_strerror(int(code)).decode()


_WFMT = {"dtype": HY3MOE_WFMT_DTYPE, "fp8_e4m3": HY3MOE_WFMT_FP8_E4M3, "mxfp4": HY3MOE_WFMT_MXFP4}
_AFMT = {"dtype": HY3MOE_AFMT_DTYPE, "fp8_static": HY3MOE_AFMT_FP8_STATIC,
         "mxfp8": HY3MOE_AFMT_MXFP8}


def make_config(T: int, H: int, E: int, K: int, I: int, I_shared: int, dtype: str = "bf16",
                route_mode: int = HY3MOE_ROUTE_SIGMOID_BIAS,
                router_prec: int = HY3MOE_ROUTER_FP32, scale: float = 2.826,
                renorm_eps: float = 1e-8, w_format: str = "dtype",
                act_format: str = "dtype", shared_w_format: Optional[str] = None,
                shared_act_format: Optional[str] = None) -> hy3moe_config:
    """shared_w_format / shared_act_format: None for the routed formats."""
    return hy3moe_config(T=int(T), H=int(H), E=int(E), K=int(K), I=int(I),
                         I_shared=int(I_shared),
                         dtype=HY3MOE_BF16 if dtype == "bf16" else HY3MOE_F32,
                         route_mode=int(route_mode), router_prec=int(router_prec),
                         scale=float(scale), renorm_eps=float(renorm_eps),
                         w_format=_WFMT[w_format], act_format=_AFMT[act_format],
                         shared_w_format=(HY3MOE_FMT_AS_ROUTED if shared_w_format is None
                                          else _WFMT[shared_w_format]),
                         shared_act_format=(HY3MOE_FMT_AS_ROUTED if shared_act_format is None
                                            else _AFMT[shared_act_format]))


def hy3moe_workspace_bytes(cfg: hy3moe_config, for_forward: bool = True) -> int:
    return int(load().hy3moe_workspace_bytes(ctypes.byref(cfg), 1 if for_forward else 0))


def hy3moe_workspace_layout(cfg: hy3moe_config) -> hy3moe_ws_layout:
    out = hy3moe_ws_layout()
    rc = load().hy3moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(out))
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_workspace_layout")
    return out


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def alloc_workspace(cfg: hy3moe_config, for_forward: bool, device) -> torch.Tensor:
    n = hy3moe_workspace_bytes(cfg, for_forward)
    if n == 0:
        raise Hy3MoEError(-1, "hy3moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def hy3moe_route(cfg: hy3moe_config, x: torch.Tensor, w_router: torch.Tensor,
                 expert_bias: Optional[torch.Tensor], idx: torch.Tensor, weight: torch.Tensor,
                 workspace: torch.Tensor, stream=None) -> None:
    """C ABI hy3moe_route on torch device tensors (results in idx/weight)."""
    _check_dev(x, w_router, expert_bias, idx, weight, workspace)
    rc = load().hy3moe_route(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(expert_bias),
                             _ptr(idx), _ptr(weight), _ptr(workspace), workspace.numel(),
                             _stream(stream))
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_route")


def hy3moe_quantize_e4m3(x: torch.Tensor, scale: torch.Tensor, q: torch.Tensor,
                         stream=None) -> None:
    """C ABI hy3moe_quantize_e4m3: q = E4M3 codes of x / scale (uint8, x.numel())."""
    _check_dev(x, scale, q)
    if x.dtype not in (torch.bfloat16, torch.float32) or q.dtype != torch.uint8:
        raise ValueError("x must be bf16 or float32 and q uint8")
    if q.numel() != x.numel() or scale.dtype != torch.float32 or scale.numel() < 1:
        raise ValueError("q needs x.numel() bytes and scale one float32")
    dt = HY3MOE_BF16 if x.dtype == torch.bfloat16 else HY3MOE_F32
    rc = load().hy3moe_quantize_e4m3(_ptr(x), dt, x.numel(), _ptr(scale), _ptr(q),
                                     _stream(stream))
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_quantize_e4m3")


def hy3moe_forward(cfg: hy3moe_config, x: torch.Tensor, weights: Dict[str, torch.Tensor],
                   out: torch.Tensor, workspace: torch.Tensor,
                   idx_out: Optional[torch.Tensor] = None,
                   weight_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """C ABI hy3moe_forward on torch device tensors (result in out)."""
    ts = [weights.get(n) for n in WEIGHT_NAMES]
    _check_dev(x, out, workspace, idx_out, weight_out, *ts)
    w = hy3moe_weights(*[_ptr(t) for t in ts])
    rc = load().hy3moe_forward(ctypes.byref(cfg), _ptr(x), ctypes.byref(w), _ptr(out),
                               _ptr(idx_out), _ptr(weight_out), _ptr(workspace),
                               workspace.numel(), _stream(stream))
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_forward")


def router_split(w_router: torch.Tensor, router_prec: int = HY3MOE_ROUTER_FP32,
                 stream=None) -> torch.Tensor:
    """C ABI hy3moe_router_split: the offline bf16 split of the fp32 router
    weight [E, H], returned as a uint8 device tensor of planes."""
    _check_dev(w_router)
    if w_router.dtype != torch.float32 or w_router.dim() != 2:
        raise ValueError("w_router must be a float32 [E, H] tensor")
    E, H = (int(v) for v in w_router.shape)
    n = load().hy3moe_router_planes_bytes(E, H, router_prec)
    if n == 0:
        raise Hy3MoEError(-1, "hy3moe_router_planes_bytes")
    planes = torch.empty(n, dtype=torch.uint8, device=w_router.device)
    rc = load().hy3moe_router_split(_ptr(w_router), E, H, router_prec, _ptr(planes), n,
                                    _stream(stream))
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_router_split")
    return planes


def hy3moe_route_planes(cfg: hy3moe_config, x: torch.Tensor, w_router: torch.Tensor,
                        w_router_planes: Optional[torch.Tensor],
                        expert_bias: Optional[torch.Tensor], idx: torch.Tensor,
                        weight: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    """C ABI hy3moe_route_planes (results in idx/weight)."""
    _check_dev(x, w_router, w_router_planes, expert_bias, idx, weight, workspace)
    rc = load().hy3moe_route_planes(ctypes.byref(cfg), _ptr(x), _ptr(w_router),
                                    _ptr(w_router_planes), _ptr(expert_bias), _ptr(idx),
                                    _ptr(weight), _ptr(workspace), workspace.numel(),
                                    _stream(stream))
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_route_planes")


def hy3moe_forward_static(cfg: hy3moe_config, x: torch.Tensor, weights: Dict[str, torch.Tensor],
                          out: torch.Tensor, idx_out: Optional[torch.Tensor] = None,
                          weight_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """C ABI hy3moe_forward_static: hy3moe_forward with the library's static
    per-GPU scratch instead of a caller workspace (allocates nothing)."""
    ts = [weights.get(n) for n in WEIGHT_NAMES]
    _check_dev(x, out, idx_out, weight_out, *ts)
    w = hy3moe_weights(*[_ptr(t) for t in ts])
    rc = load().hy3moe_forward_static(ctypes.byref(cfg), _ptr(x), ctypes.byref(w), _ptr(out),
                                      _ptr(idx_out), _ptr(weight_out), _stream(stream))
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_forward_static")


def hy3moe_forward_timed(cfg: hy3moe_config, x: torch.Tensor, weights: Dict[str, torch.Tensor],
                         out: torch.Tensor, workspace: torch.Tensor, events,
                         idx_out: Optional[torch.Tensor] = None,
                         weight_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """C ABI hy3moe_forward_timed; ``events`` are HY3MOE_N_STAGES + 1 torch.cuda.Event
    objects created with enable_timing=True (already recorded once, so that their
    HIP handles exist)."""
    ts = [weights.get(n) for n in WEIGHT_NAMES]
    _check_dev(x, out, workspace, idx_out, weight_out, *ts)
    if len(events) != HY3MOE_N_STAGES + 1:
        raise ValueError("need HY3MOE_N_STAGES + 1 events")
    w = hy3moe_weights(*[_ptr(t) for t in ts])
    evs = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    rc = load().hy3moe_forward_timed(ctypes.byref(cfg), _ptr(x), ctypes.byref(w), _ptr(out),
                                     _ptr(idx_out), _ptr(weight_out), _ptr(workspace),
                                     workspace.numel(), _stream(stream), evs)
    if rc != HY3MOE_OK:
        raise Hy3MoEError(rc, "hy3moe_forward_timed")


# Convenience wrappers that allocate outputs (tests and benchmark).
def route(cfg: hy3moe_config, x, w_router, expert_bias=None, workspace=None,
          stream=None, w_router_planes=None) -> Tuple[torch.Tensor, torch.Tensor]:
    T, K = int(cfg.T), int(cfg.K)
    idx = torch.empty((T, K), dtype=torch.int32, device=x.device)
    weight = torch.empty((T, K), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(cfg, False, x.device)
    if w_router_planes is None:
        hy3moe_route(cfg, x, w_router, expert_bias, idx, weight, workspace, stream)
    else:
        hy3moe_route_planes(cfg, x, w_router, w_router_planes, expert_bias, idx, weight,
                            workspace, stream)
    return idx, weight


def forward(cfg: hy3moe_config, x, weights, workspace=None, return_route=False, stream=None):
    out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(cfg, True, x.device)
    idx = weight = None
    if return_route:
        idx = torch.empty((int(cfg.T), int(cfg.K)), dtype=torch.int32, device=x.device)
        weight = torch.empty((int(cfg.T), int(cfg.K)), dtype=torch.float32, device=x.device)
    hy3moe_forward(cfg, x, weights, out, workspace, idx, weight, stream)
    return (out, idx, weight) if return_route else out


# ---------------------------------------------------------------------------
# Split-KV decode attention (include/hy3attn.h): argument marshalling only.
# ---------------------------------------------------------------------------
ATTN_EXPORTED_SYMBOLS = ("hy3attn_max_tasks", "hy3attn_workspace_bytes", "hy3attn_plan",
                         "hy3attn_decode")
ATTN_TILE = 256


class AttnPlan:
    """Task map from hy3attn_plan (host numpy arrays)."""

    def __init__(self, tasks, worker_begin, row_begin, n_workers, tile, B=None, n_kv_heads=None):
        self.tasks, self.worker_begin, self.row_begin = tasks, worker_begin, row_begin
        self.n_workers, self.tile = n_workers, tile
        self.B, self.n_kv_heads = B, n_kv_heads


def attn_plan(kv_len, n_kv_heads: int, tile: int = ATTN_TILE, n_workers: int = 512) -> AttnPlan:
    import numpy as np
    L = load()
    kv = np.ascontiguousarray(np.asarray(kv_len, dtype=np.int32))
    B = int(kv.size)
    cap = int(L.hy3attn_max_tasks(B, n_kv_heads, n_workers))
    tasks = np.zeros((max(cap, 1), 4), dtype=np.int32)
    wb = np.zeros(n_workers + 1, dtype=np.int32)
    rb = np.zeros(B * n_kv_heads + 1, dtype=np.int32)
    nt = ctypes.c_int64(0)
    rc = L.hy3attn_plan(kv.ctypes.data if B else None, B, n_kv_heads, tile, n_workers,
                        tasks.ctypes.data, cap, wb.ctypes.data, rb.ctypes.data,
                        ctypes.byref(nt))
    if rc != 0:
        raise RuntimeError(f"hy3attn_plan failed ({rc})")
    return AttnPlan(tasks[:nt.value].copy(), wb, rb, n_workers, tile, B, n_kv_heads)


def attn_decode(q, k, v, kv_len, plan: AttnPlan, out=None, workspace=None):
    """q [B][Hq][128], k, v [Hkv][sum L][128] bf16 torch tensors on one GPU;
    returns out [B][Hq][128] bf16.  The plan's arrays are copied to the
    device (the caller may build and copy them once per inference)."""
    import numpy as np
    import torch
    L = load()
    dev = q.device
    B, Hq, _ = q.shape
    Hkv = k.shape[0]
    if Hq != 8 * Hkv or q.shape[2] != 128 or k.shape != v.shape or k.shape[2] != 128:
        raise ValueError("q must be [B][8*Hkv][128] and k, v [Hkv][tokens][128]")
    if len(kv_len) != B or plan.row_begin.size != B * Hkv + 1:
        raise ValueError("the plan was made for another batch or KV head count")
    if plan.tasks.size and (int(plan.tasks[:, 0].max()) >= B or int(plan.tasks[:, 1].max()) >= Hkv
                            or int(plan.tasks.min()) < 0):
        raise ValueError("the plan holds tasks outside this batch")
    if plan.worker_begin.size != plan.n_workers + 1:
        raise ValueError("worker_begin must hold n_workers + 1 entries")
    starts = np.zeros(B + 1, dtype=np.int32)
    starts[1:] = np.cumsum(np.asarray(kv_len, dtype=np.int64))
    kv_start = torch.from_numpy(starts).to(dev)
    tasks = torch.from_numpy(plan.tasks.reshape(-1)).to(dev) if plan.tasks.size else \
        torch.zeros(4, dtype=torch.int32, device=dev)
    wb = torch.from_numpy(plan.worker_begin).to(dev)
    rb = torch.from_numpy(plan.row_begin).to(dev)
    n_tasks = int(plan.tasks.shape[0])
    need = int(L.hy3attn_workspace_bytes(n_tasks))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev).cuda_stream
    rc = L.hy3attn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), kv_start.data_ptr(), B, Hkv,
                          plan.tile, tasks.data_ptr(), n_tasks, wb.data_ptr(), plan.n_workers,
                          rb.data_ptr(), plan.row_begin.size - 1, workspace.data_ptr(),
                          workspace.numel(), out.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError(f"hy3attn_decode failed ({rc})")
    return out
