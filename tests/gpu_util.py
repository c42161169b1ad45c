"""Helpers shared by the GPU parity tests: device upload of seeded inputs,
oracle evaluation, and the comparison rules.

Comparison rules
----------------
* Route indices: for every token whose oracle selection margin (K-th minus
  (K+1)-th selection score, float64) exceeds 1e-6, the set of picked experts
  must equal the oracle's exactly.  A token at or below the margin has
  several correct answers; the GPU's picks must then be one of them: a
  top-K of the float64 selection scores up to the margin (every picked score
  at least every unpicked score minus 1e-6).
* Weights: on every token, the GPU weight of each picked expert equals the
  oracle's weight formula evaluated on the GPU's own picks, to 2e-6
  relative, and the K weights sum to the scale (sigmoid mode) or 1 (softmax
  mode) within K/2 float32 ulps of that sum.
* Outputs: near-tie tokens are checked against the oracle run on the GPU's
  picks with the oracle's weights for them (``route_for_reference``), never
  the GPU's weights.  bf16 activations/weights at the Hy3 / HunyuanImage
  workload shapes: max-abs error <= 2e-2 and rel-L2 <= 5e-3 against the
  float64 oracle.  Elsewhere (small synthetic shapes, quantised weights) the
  bound is derived from the two roundings that remain in the bf16 path: h
  rounded to bf16 and carried through the down projection, an error that
  scales with the layer's output scale, and the output's own bf16 rounding,
  at most 2^-8 |ref| at each element.  The 2e-2 is stated for the Hy3 layer,
  whose float64 output has RMS 0.844 (Hy3 decode batch), so each element
  must satisfy |got - ref| <= 2e-2 max(1, rms(ref) / 0.844) + 2^-8 |ref|;
  rel-L2 stays 5e-3.  fp32: max-abs <= 1e-4 and rel-L2 <= 1e-5.
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
HY3_OUT_RMS = 0.844     # RMS of the Hy3 layer's float64 output (decode batch)


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


from synth.device import (to_torch, upload_weights, with_act_scales,  # noqa: E402,F401
                          with_bias_of)


def config_of(inp: MoEInputs, **kw) -> sm.hy3moe_config:
    c = inp.cfg
    d = dict(T=c.T, H=c.H, E=c.E, K=c.K, I=c.I, I_shared=c.I_shared, dtype=c.dtype,
             route_mode=c.route_mode, scale=c.scale, renorm_eps=c.renorm_eps,
             w_format=c.w_format, act_format=c.act_format,
             shared_w_format=c.shared_w_format, shared_act_format=c.shared_act_format)
    d.update(kw)
    return sm.make_config(**d)


def oracle_route(inp: MoEInputs, x64: Optional[np.ndarray] = None) -> oracle.Route:
    c = inp.cfg
    if x64 is None:
        x64 = inp.x_f64()
    b = inp.bias()
    r = oracle.route(x64, inp.w_router().astype(np.float64), c.K, c.route_mode,
                     None if b is None else b.astype(np.float64), c.scale, c.renorm_eps)
    # the weight formula's parameters, for weights on the GPU's own picks
    r.mode, r.scale, r.renorm_eps = c.route_mode, c.scale, c.renorm_eps
    return r


def oracle_weights_on(r: oracle.Route, picks: np.ndarray) -> np.ndarray:
    """The oracle's combine weights (float64) for the given picks."""
    return oracle.combine_weights(r.prob, picks.astype(np.int64), getattr(r, "mode", 0),
                                  getattr(r, "scale", 2.826), getattr(r, "renorm_eps", 1e-8))


def check_route(gpu_idx: np.ndarray, gpu_w: np.ndarray, r: oracle.Route,
                wtol: float = 2e-6) -> dict:
    T, E = r.select_score.shape
    K = gpu_idx.shape[1] if gpu_idx.ndim == 2 else 0
    ok = r.margin > MARGIN
    gi = gpu_idx.astype(np.int64)
    assert ((gi >= 0) & (gi < E)).all(), "route index out of range"
    gs, os_ = np.sort(gi, 1), np.sort(r.idx, 1)
    # every token's picks are distinct
    assert (np.diff(gs, axis=1) != 0).all(), "repeated expert in a token's picks"
    bad = np.nonzero(ok & (gs != os_).any(1))[0]
    assert bad.size == 0, f"route indices differ on {bad.size} tokens, first {bad[:5]}"
    # near-tie tokens: the picks are a top-K of the float64 selection scores
    # up to the margin (a valid answer where several are correct)
    sel = r.select_score
    picked = np.take_along_axis(sel, gi, 1)
    mask = np.ones((T, E), dtype=bool)
    np.put_along_axis(mask, gi, False, 1)
    unpicked_max = np.where(mask, sel, -np.inf).max(1) if K < E else np.full(T, -np.inf)
    slack = picked.min(1) - unpicked_max if T else np.zeros(0)
    assert (slack >= -MARGIN).all(), \
        f"not a top-K on tokens {np.nonzero(slack < -MARGIN)[0][:5]} (slack {slack.min():.3e})"
    # weights: the formula on the GPU's own picks, on every token
    want = oracle_weights_on(r, gi)
    rel = np.abs(gpu_w.astype(np.float64) - want) / np.maximum(np.abs(want), 1e-30)
    assert rel.size == 0 or rel.max() <= wtol, f"weights rel err {rel.max():.3e}"
    # sums: the scale in sigmoid mode; 1 in softmax mode unless the clamp
    # binds (picked mass below renorm_eps), where the formula's own sum holds
    if getattr(r, "mode", 0) == 0:
        target = np.full(T, getattr(r, "scale", 2.826))
    else:
        mass = np.take_along_axis(r.prob, gi, 1).sum(1)
        target = np.where(mass >= r.renorm_eps, 1.0, want.sum(1))
    sums = gpu_w.astype(np.float64).sum(1)
    tol_sum = 0.5 * K * np.spacing(np.float32(target.max() if T else 1.0))
    assert (np.abs(sums - target) <= tol_sum).all(), \
        f"weight sums off by {np.abs(sums - target).max():.3e} (tol {tol_sum:.3e})"
    # GPU picks are in descending selection score (checked on the oracle's scores)
    assert (np.diff(picked, axis=1) <= MARGIN).all(), "picks not in descending score"
    return {"near_ties": int((~ok).sum()), "weight_rel_err": float(rel.max()) if rel.size else 0.0,
            "near_tie_min_slack": float(slack[~ok].min()) if (~ok).any() else None}


def route_for_reference(r: oracle.Route, gpu_idx: np.ndarray):
    """(idx, weight) to evaluate the oracle's layer on: the oracle's route
    where the margin exceeds 1e-6; elsewhere the GPU's picks (a valid top-K,
    by check_route) with the oracle's float64 weights for them."""
    idx, w = r.idx.copy(), r.weight.copy()
    tie = r.margin <= MARGIN
    if tie.any():
        idx[tie] = gpu_idx[tie]
        w[tie] = oracle_weights_on(r, gpu_idx)[tie]
    return idx, w


def output_errors(got: np.ndarray, ref: np.ndarray) -> tuple:
    d = got.astype(np.float64) - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))


def check_output(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "",
                 workload_shape: bool = False) -> tuple:
    """workload_shape=True: one of the named workloads, the stated bf16 bound.
    Otherwise (bf16) each element is held to 2e-2 max(1, rms(ref)/0.844) +
    2^-8 |ref| (module docstring)."""
    mx, rel = output_errors(got, ref)
    tmax, trel = TOL[dtype]
    top = float(np.abs(ref).max()) if ref.size else 0.0
    if dtype == "bf16" and not workload_shape and ref.size:
        rms = float(np.sqrt(np.mean(ref ** 2)))
        absb = tmax * max(1.0, rms / HY3_OUT_RMS)
        excess = np.abs(got.astype(np.float64) - ref) - (absb + 2.0 ** -8 * np.abs(ref))
        worst = float(excess.max())
        log(f"  {what} max_abs={mx:.3e} rel_l2={rel:.3e} (per element {absb:.3g} + "
            f"2^-8|ref|: worst margin {-worst:.3e}; rel tol {trel:g}; rms {rms:.3g}, "
            f"max|ref| {top:.3g})")
        assert worst <= 0 and rel <= trel, f"{what}: max_abs {mx:.3e} rel_l2 {rel:.3e}"
        return mx, rel
    log(f"  {what} max_abs={mx:.3e} rel_l2={rel:.3e} (tol {tmax:g}/{trel:g}; max|ref| {top:.3g})")
    assert mx <= tmax and rel <= trel, f"{what}: max_abs {mx:.3e} rel_l2 {rel:.3e}"
    return mx, rel


def h_error_bound(a, wg, wu, gemm):
    """h = SiLU(a wg^T) (a wu^T) in float64, and how far the GPU's float32 h
    can be from it: the GEMM's error, at most `gemm` times the sum of
    |products| (1024 ulps (2^-23) for the FP8 and FP4 x FP8 MFMAs, measured
    in test_gpu_mfma_fp8.py; the bf16 MFMAs are far closer), propagated
    through SiLU(g) u, plus a few ulps of h for the epilogue's arithmetic."""
    u32 = 2.0 ** -24
    gg, uu = a @ wg.T, a @ wu.T
    h64 = oracle.silu(gg) * uu
    dg = gemm * (np.abs(a) @ np.abs(wg).T) + 4 * u32 * np.abs(gg)
    du = gemm * (np.abs(a) @ np.abs(wu).T) + 4 * u32 * np.abs(uu)
    sg = oracle.sigmoid(gg)
    dsilu = np.abs(sg * (1 + gg * (1 - sg)))
    dh = dsilu * np.abs(uu) * dg + np.abs(gg * sg) * du + 8 * u32 * np.abs(h64)
    return h64, dh


def grid_step(v):
    """Spacing of the E4M3 grid at |v| (2^(e-3) in [2^e, 2^(e+1)), 2^-9 below 2^-6)."""
    a = np.abs(v)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    return np.exp2(np.maximum(ex - 1, -6) - 3.0)


class WorkspaceActivations:
    """The quantised h a forward left in its workspace, as an ``h_hook`` for
    ``oracle.forward_by_expert``.

    For each group it reads the GPU's h rows (E4M3 codes, MXFP8 codes and
    block scales, or the bf16 values of the codes, depending on the path),
    checks them against the oracle's and returns what the oracle's down
    projection continues with:

    * the GPU's float32 h lies within dh of the float64 h (dh: the GEMM and
      epilogue error bound, ``h_error_bound``).  W8A8: bf16 rounding and the
      quantisation are monotone, so the GPU's code must lie between the
      codes of h - dh and h + dh, and equal the oracle's where those agree.
      W4A8: per block of 32 (whose shared scale every element can move), the
      GPU's values must equal the oracle's where no element's bf16 value is
      in doubt (no bf16 rounding boundary within dh of h);
    * elsewhere several codes are valid.  W4A8: the block's values must lie within dh, one bf16
      rounding and one grid step (or saturation) of the float64 h.  The GPU's
      values are then taken, as the GPU's picks are for near-tie tokens.
    """

    def __init__(self, inp: MoEInputs, ws: torch.Tensor, L, codes_path=None):
        """codes_path: None for where the forward's GEMM path leaves h, or
        (routed, shared) booleans that say so (checks of fake workspaces)."""
        c = inp.cfg
        self.E, self.K = c.E, c.K
        self.ldh = max(c.I, c.I_shared)
        R = c.T * c.K + (c.T if c.I_shared else 0)
        self.N = c.T * c.K
        i32 = lambda off, n: ws[off:off + 4 * n].cpu().numpy().view(np.int32)
        self.offsets = i32(L.offsets, c.E + 2)
        self.sorted_token = i32(L.sorted_token, R)
        # per branch (routed, shared): format, and where the forward left h.
        # MXFP8: codes and block scales in hq / hs on the weight-streaming
        # and large-tile paths; static FP8: codes in h (row r at byte r *
        # ldh, past the earlier rows' 2-byte h when the shared expert has
        # formats of its own) where the layout says the token rows are codes
        # (a8_codes).  Elsewhere h holds the bf16 values of the codes.
        mixed = c.I_shared > 0 and (c.sw_format, c.sa_format) != (c.w_format, c.act_format)
        self.fmt = {}
        for i, (br, act) in enumerate((("routed", c.act_format), ("shared", c.sa_format))):
            a8 = _a8(inp, act)
            codes = bool(L.a8_codes) if a8 is not None else L.gemm_path != 1
            if codes_path is not None:
                codes = bool(codes_path[i])
            self.fmt[br] = (a8, act == "mxfp8", codes)
        self.R = R
        self.ws, self.L = ws, L
        self.h8_base = {"routed": 0, "shared": self.N * self.ldh if mixed else 0}
        self._arr = {}
        self.n = self.n_amb = 0

    def _get(self, key):
        if key not in self._arr:
            ws, L, R, ldh = self.ws, self.L, self.R, self.ldh
            if key == "hq":
                a = ws[L.hq:L.hq + R * ldh].cpu().numpy().reshape(R, ldh)
            elif key == "hs":
                a = ws[L.hs:L.hs + R * ldh // 32].cpu().numpy().reshape(R, ldh // 32)
            elif key == "hv":
                bits = ws[L.h:L.h + 2 * R * ldh].cpu().numpy().view(np.uint16)
                a = (bits.astype(np.uint32) << 16).view(np.float32).reshape(R, ldh)
            else:        # ("h8", byte offset of row 0)
                o = L.h + key[1]
                a = ws[o:o + R * ldh].cpu().numpy().reshape(R, ldh)
            self._arr[key] = a
        return self._arr[key]

    def gpu_values(self, br, e, r0, r1, Ig):
        """The GPU's h_in of group e: the MXFP8 values, or the static scale
        times the E4M3 values (stored as codes or as their bf16 values)."""
        a8, amx, codes = self.fmt[br]
        if amx:        # codes and block scales, or their values in bf16 (exact)
            if not codes:
                return self._get("hv")[r0:r1, :Ig].astype(np.float64)
            return oracle.dequant_mxfp8(self._get("hq")[r0:r1, :Ig],
                                        self._get("hs")[r0:r1, :Ig // 32])
        v = (oracle.fp8_e4m3_value(self._get(("h8", self.h8_base[br]))[r0:r1, :Ig]) if codes
             else self._get("hv")[r0:r1, :Ig].astype(np.float64))
        return np.float64(np.float32(a8[1][e])) * v

    def __call__(self, e, tok, a, wg, wu, h, h_in):
        r0, r1 = self.offsets[e], self.offsets[e + 1]
        assert r1 - r0 == len(tok) and (self.sorted_token[r0:r1] == tok).all(), \
            f"group {e}: the GPU's rows are not the oracle's tokens"
        br = "shared" if e == self.E else "routed"
        a8, amx, codes = self.fmt[br]
        if a8 is None and not amx:
            return h_in          # this branch keeps its activations unquantised
        Ig = wg.shape[0]
        got = self.gpu_values(br, e, r0, r1, Ig)
        # the FP8 and FP4 x FP8 MFMAs' accumulation error; bf16 MFMAs far closer
        gemm = (1024 * 2.0 ** -23) if codes else 64 * 2.0 ** -24
        _, dh = h_error_bound(a, wg, wu, gemm)
        if amx:
            amb = oracle.round_bf16(h - dh) != oracle.round_bf16(h + dh)
            amb = np.repeat(amb.reshape(len(tok), -1, 32).any(axis=2), 32, axis=1)
            # the GPU's block scales (its largest code is in [256, 448]: the
            # scale is 2^(floor(log2 max|value|) - 8)); a value may be a grid
            # step off, or saturated
            bmax = np.abs(got).reshape(len(tok), -1, 32).max(axis=2)
            _, ex = np.frexp(np.where(bmax > 0, bmax, 1.0))
            sc = np.repeat(np.where(bmax > 0, np.exp2(ex - 1.0 - 8.0), 2.0 ** -127), 32, axis=1)
            step = grid_step(np.abs(got) / sc) * sc
            sat = np.maximum(np.abs(h) + dh - 448.0 * sc, 0.0)
            allowed = dh + 2.0 ** -8 * np.abs(h) + step + sat
            ok_amb = np.abs(got - h) <= allowed * (1 + 1e-12)
        else:
            a2 = float(a8[1][e])
            # bf16 rounding and the quantisation are monotone: the valid
            # values are the grid values between those of the interval's
            # ends, and the code is ambiguous only where those differ
            lo = oracle.quant_dequant_e4m3(oracle.round_bf16(h - dh), a2)
            hi = oracle.quant_dequant_e4m3(oracle.round_bf16(h + dh), a2)
            amb = lo != hi
            ok_amb = (got >= lo) & (got <= hi)
        bad = np.argwhere(np.where(amb, ~ok_amb, got != h_in))
        if bad.size:
            i, j = bad[0]
            log(f"  group {e} row {i} col {j}: h={h[i, j]:.9g} dh={dh[i, j]:.3g} "
                f"gpu={got[i, j]:.9g} oracle={h_in[i, j]:.9g} ambiguous={bool(amb[i, j])}")
        assert bad.size == 0, f"group {e}: {bad.shape[0]} activation codes off"
        self.n += h.size
        self.n_amb += int(amb.sum())
        return np.where(amb, got, h_in)


def expert_fn(inp: MoEInputs):
    """expert(e) -> float64 (gate, up, down), regenerated on every call (no
    cache: the layer-sized checks request each expert once)."""
    fmt = inp.cfg.w_format

    def f(e):
        if fmt == "mxfp4":
            codes, sc = inp.expert_mxfp4(e)
            return tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(codes, sc))
        if fmt == "fp8_e4m3":
            codes, sc = inp.expert_fp8(e)
            return tuple(oracle.dequant_fp8(q, s) for q, s in zip(codes, sc))
        return inp.expert_f64(e)
    return f


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
    """float64 (gate, up, down) of the shared expert (in its own weight format), or None."""
    fmt = inp.cfg.sw_format
    if inp.cfg.I_shared == 0:
        return None
    if fmt == "mxfp4":
        return tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(*inp.shared_mxfp4()))
    if fmt == "fp8_e4m3":
        return tuple(oracle.dequant_fp8(q, s) for q, s in zip(*inp.shared_fp8()))
    return inp.shared_f64()


def _a8(inp: MoEInputs, fmt: str):
    if fmt != "fp8_static":
        return None
    a1, a2 = inp.act_scales()
    return float(a1), a2.astype(np.float64)


def amx_of(inp: MoEInputs) -> bool:
    """True for dynamic MXFP8 activations (W4A8) of the routed experts."""
    return inp.cfg.act_format == "mxfp8"


def a8_of(inp: MoEInputs):
    """(a1, a2) static FP8 activation scales of the routed experts for the oracle, or None."""
    return _a8(inp, inp.cfg.act_format)


def quant_act(inp: MoEInputs) -> bool:
    """Does either branch quantise its activations?"""
    c = inp.cfg
    return c.act_format != "dtype" or (c.I_shared > 0 and c.sa_format != "dtype")


def act_kw(inp: MoEInputs) -> dict:
    """The oracle's activation-format arguments of this workload (both branches)."""
    c = inp.cfg
    return dict(a8=a8_of(inp), amx=amx_of(inp), shared_a8=_a8(inp, c.sa_format),
                shared_amx=c.sa_format == "mxfp8")


def out_to_np(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)
