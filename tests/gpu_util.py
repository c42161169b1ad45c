"""Helpers shared by the GPU parity tests: device upload of seeded inputs,
oracle evaluation, and the comparison rules.

Comparison rules
----------------
* Route indices: for every token whose oracle selection margin (K-th minus
  (K+1)-th selection score, float64) exceeds 1e-6, the set of picked experts
  must equal the oracle's exactly, and the weight of each picked expert must
  agree to 2e-6 relative.  Tokens at or below the margin have several correct
  answers; their outputs are checked against the oracle run on the GPU's own
  route (oracle.forward_given_route).
* Outputs: bf16 activations/weights at the Hy3 / HunyuanImage workload shapes:
  max-abs error <= 2e-2 and rel-L2 <= 5e-3 against the float64 oracle.  Other
  synthetic shapes can have larger outputs, where one bf16 rounding of the
  output alone exceeds 2e-2 (|out| >= 4 has a half-ulp of 1/64), so there the
  absolute bound is max(2e-2, 2^-6 * max|ref|), two bf16 ulps at the largest
  output; rel-L2 stays 5e-3.  fp32: max-abs <= 1e-4 and rel-L2 <= 1e-5.
"""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

import oracle
import sparse_moe_amd as sm
from synth import MoEInputs

MARGIN = 1e-6
TOL = {"bf16": (2e-2, 5e-3), "f32": (1e-4, 1e-5)}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


from synth.device import (to_torch, upload_weights, with_act_scales,  # noqa: E402,F401
                          with_bias_of)


def config_of(inp: MoEInputs, **kw) -> sm.hy3moe_config:
    c = inp.cfg
    d = dict(T=c.T, H=c.H, E=c.E, K=c.K, I=c.I, I_shared=c.I_shared, dtype=c.dtype,
             route_mode=c.route_mode, scale=c.scale, renorm_eps=c.renorm_eps,
             w_format=c.w_format, act_format=c.act_format)
    d.update(kw)
    return sm.make_config(**d)


def oracle_route(inp: MoEInputs, x64: Optional[np.ndarray] = None) -> oracle.Route:
    c = inp.cfg
    if x64 is None:
        x64 = inp.x_f64()
    b = inp.bias()
    return oracle.route(x64, inp.w_router().astype(np.float64), c.K, c.route_mode,
                        None if b is None else b.astype(np.float64), c.scale, c.renorm_eps)


def check_route(gpu_idx: np.ndarray, gpu_w: np.ndarray, r: oracle.Route,
                wtol: float = 2e-6) -> dict:
    ok = r.margin > MARGIN
    gs, os_ = np.sort(gpu_idx, 1), np.sort(r.idx, 1)
    bad = np.nonzero(ok & (gs != os_).any(1))[0]
    assert bad.size == 0, f"route indices differ on {bad.size} tokens, first {bad[:5]}"
    assert ((gpu_idx >= 0) & (gpu_idx < r.select_score.shape[1])).all()
    # every token's picks are distinct
    assert (np.diff(gs, axis=1) != 0).all()
    # weights per picked expert (align by expert id)
    go, oo = np.argsort(gpu_idx, 1), np.argsort(r.idx, 1)
    gw = np.take_along_axis(gpu_w.astype(np.float64), go, 1)
    ow = np.take_along_axis(r.weight, oo, 1)
    rel = np.abs(gw[ok] - ow[ok]) / np.maximum(np.abs(ow[ok]), 1e-30)
    assert rel.size == 0 or rel.max() <= wtol, f"weights rel err {rel.max():.3e}"
    # GPU picks are in descending selection score (checked on the oracle's scores)
    sc = np.take_along_axis(r.select_score, gpu_idx.astype(np.int64), 1)
    assert (np.diff(sc, axis=1) <= 1e-6).all()
    return {"near_ties": int((~ok).sum()), "weight_rel_err": float(rel.max()) if rel.size else 0.0}


def output_errors(got: np.ndarray, ref: np.ndarray) -> tuple:
    d = got.astype(np.float64) - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def check_output(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "",
                 workload_shape: bool = False) -> tuple:
    """workload_shape=True: one of the named workloads, strict bf16 bound."""
    mx, rel = output_errors(got, ref)
    tmax, trel = TOL[dtype]
    if dtype == "bf16" and not workload_shape and ref.size:
        tmax = max(tmax, 2.0 ** -6 * float(np.abs(ref).max()))
    top = float(np.abs(ref).max()) if ref.size else 0.0
    log(f"  {what} max_abs={mx:.3e} rel_l2={rel:.3e} (tol {tmax:g}/{trel:g}; max|ref| {top:.3g})")
    assert mx <= tmax and rel <= trel, f"{what}: max_abs {mx:.3e} rel_l2 {rel:.3e}"
    return mx, rel


def expert_cache(inp: MoEInputs):
    """expert(e) -> float64 (gate, up, down); FP8 weights dequantised by the oracle."""
    cache = {}
    fp8 = inp.cfg.w_format == "fp8_e4m3"
    fp4 = inp.cfg.w_format == "mxfp4"

    def f(e):
        if e not in cache:
            if fp4:
                codes, sc = inp.expert_mxfp4(e)
                cache[e] = tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(codes, sc))
            elif fp8:
                codes, sc = inp.expert_fp8(e)
                cache[e] = tuple(oracle.dequant_fp8(q, s) for q, s in zip(codes, sc))
            else:
                cache[e] = inp.expert_f64(e)
        return cache[e]
    return f


def shared_f64(inp: MoEInputs):
    """float64 (gate, up, down) of the shared expert, or None."""
    if inp.cfg.w_format == "mxfp4":
        sh = inp.shared_mxfp4()
        return None if sh is None else tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(*sh))
    if inp.cfg.w_format != "fp8_e4m3":
        return inp.shared_f64()
    sh = inp.shared_fp8()
    if sh is None:
        return None
    return tuple(oracle.dequant_fp8(q, s) for q, s in zip(*sh))


def amx_of(inp: MoEInputs) -> bool:
    """True for dynamic MXFP8 activations (W4A8)."""
    return inp.cfg.act_format == "mxfp8"


def a8_of(inp: MoEInputs):
    """(a1, a2) static FP8 activation scales for the oracle, or None."""
    if inp.cfg.act_format != "fp8_static":
        return None
    a1, a2 = inp.act_scales()
    return float(a1), a2.astype(np.float64)


def out_to_np(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)
