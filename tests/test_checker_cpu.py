"""CPU checks of the GPU tests' own checkers (no GPU): the workspace
activation hook accepts the oracle's own quantised activations laid out as
the forward lays them out, and rejects a code moved off a decision that is
not ambiguous."""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_amd as sm
from gpu_util import (WorkspaceActivations, a8_of, act_kw, config_of, expert_cache, oracle_route,
                      shared_f64)
from synth import random_small


def _fake_workspace(inp, codes_path):
    """A workspace with the permutation and the oracle's h written where the
    forward writes them, per branch (routed, shared) as ``codes_path`` says:
    W8A8 E4M3 bytes (the large-tile path; past the routed rows' 2-byte h when
    the shared expert has formats of its own) or the bf16 values of the
    codes; MXFP8 codes and scales in hq / hs, or the bf16 values."""
    c = inp.cfg
    cfg = config_of(inp)
    L = sm.hy3moe_workspace_layout(cfg)
    ws = np.zeros(L.total, dtype=np.uint8)
    r = oracle_route(inp)
    flat = r.idx.reshape(-1)
    counts = np.bincount(flat, minlength=c.E)
    offsets = np.concatenate([[0], np.cumsum(counts), [counts.sum() + c.T]]).astype(np.int32)
    order = np.argsort(flat, kind="stable")
    sorted_token = np.concatenate([order // c.K, np.arange(c.T)]).astype(np.int32)
    ws[L.offsets:L.offsets + offsets.nbytes] = offsets.view(np.uint8)
    ws[L.sorted_token:L.sorted_token + sorted_token.nbytes] = sorted_token.view(np.uint8)
    mixed = (c.sw_format, c.sa_format) != (c.w_format, c.act_format)
    ex, sh = expert_cache(inp), shared_f64(inp)
    ldh = max(c.I, c.I_shared)
    N = c.T * c.K
    for g in range(c.E + 1):
        r0, r1 = offsets[g], offsets[g + 1]
        if r1 == r0:
            continue
        shared = g == c.E
        act = c.sa_format if shared else c.act_format
        codes = codes_path[1 if shared else 0]
        amx = act == "mxfp8"
        if amx:
            a2 = None
            xq = oracle.quant_dequant_mxfp8(inp.x_f64())
        else:
            a1, a2s = inp.act_scales()
            a2 = float(a2s[g])
            xq = oracle.quant_dequant_e4m3(inp.x_f64(), float(a1))
        wg, wu, _ = sh if shared else ex(g)
        h, h_in = oracle.expert_h(xq[sorted_token[r0:r1]], wg, wu, a2=a2, amx=amx)
        h8 = L.h + (N * ldh if shared and mixed else 0)
        for i, row in enumerate(range(r0, r1)):
            if amx and codes:
                q, sc = oracle.quant_mxfp8(oracle.round_bf16(h[i:i + 1]))
                ws[L.hq + row * ldh:L.hq + row * ldh + q.shape[1]] = q[0]
                ws[L.hs + row * ldh // 32:L.hs + row * ldh // 32 + sc.shape[1]] = sc[0]
            elif codes:
                q = oracle.quant_e4m3(h_in[i], np.float32(a2))   # exact: h_in is on the grid
                ws[h8 + row * ldh:h8 + row * ldh + q.size] = q
            else:
                v = h_in[i] if amx else h_in[i] / np.float64(np.float32(a2))
                b = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact
                ws[L.h + 2 * row * ldh:L.h + 2 * row * ldh + 2 * b.size] = b.view(np.uint8)
    return torch.from_numpy(ws), L, r, offsets


@pytest.mark.parametrize("codes_path", [True, False])
def test_workspace_hook_accepts_the_oracle_and_rejects_a_moved_code(codes_path):
    inp = random_small(61, T=40, H=128, E=6, K=2, I=64, I_shared=64, dtype="bf16",
                       w_format="fp8_e4m3", act_format="fp8_static")
    c = inp.cfg
    ws, L, r, offsets = _fake_workspace(inp, (codes_path, codes_path))
    hook = WorkspaceActivations(inp, ws, L, (codes_path, codes_path))
    args = (inp.x_f64(), r.idx, r.weight, expert_cache(inp), c.E, shared_f64(inp))
    want = oracle.forward_by_expert(*args, a8=a8_of(inp))
    got = oracle.forward_by_expert(*args, a8=a8_of(inp), h_hook=hook)
    np.testing.assert_array_equal(got, want)
    assert hook.n > 0
    # move one code of the shared expert's first row by a grid step
    row = int(offsets[c.E])
    if codes_path:
        ws[L.h + row * max(c.I, c.I_shared)] ^= 1
    else:
        off = L.h + 2 * row * max(c.I, c.I_shared)
        ws[off + 1] ^= 1        # the low bit of the bf16 exponent/mantissa byte
    hook = WorkspaceActivations(inp, ws, L, (codes_path, codes_path))
    with pytest.raises(AssertionError):
        oracle.forward_by_expert(*args, a8=a8_of(inp), h_hook=hook)


def test_workspace_hook_mxfp8_accepts_the_oracle_and_rejects_a_moved_code():
    inp = random_small(62, T=24, H=128, E=6, K=2, I=128, I_shared=128, dtype="bf16",
                       w_format="mxfp4", act_format="mxfp8")
    c = inp.cfg
    ws, L, r, offsets = _fake_workspace(inp, (True, True))
    hook = WorkspaceActivations(inp, ws, L, (True, True))
    args = (inp.x_f64(), r.idx, r.weight, expert_cache(inp), c.E, shared_f64(inp))
    want = oracle.forward_by_expert(*args, amx=True)
    got = oracle.forward_by_expert(*args, amx=True, h_hook=hook)
    np.testing.assert_array_equal(got, want)
    row = int(offsets[c.E])
    ws[L.hq + row * max(c.I, c.I_shared) + 3] ^= 0x10     # an exponent bit of one code
    hook = WorkspaceActivations(inp, ws, L, (True, True))
    with pytest.raises(AssertionError):
        oracle.forward_by_expert(*args, amx=True, h_hook=hook)


@pytest.mark.parametrize("codes_path", [(True, True), (True, False), (False, False)])
def test_workspace_hook_mixed_branches(codes_path):
    """Routed W4A8 and shared W8A8 in one layer, h laid out as on the
    large-tile (codes, codes), weight-streaming (codes, values) and tiled
    (values, values) paths; a moved code of either branch is caught."""
    inp = random_small(63, T=24, H=128, E=6, K=2, I=128, I_shared=128, dtype="bf16",
                       w_format="mxfp4", act_format="mxfp8", shared_w_format="fp8_e4m3",
                       shared_act_format="fp8_static")
    c = inp.cfg
    kw = act_kw(inp)
    assert kw["amx"] and kw["shared_a8"] is not None and kw["a8"] is None
    ws, L, r, offsets = _fake_workspace(inp, codes_path)
    args = (inp.x_f64(), r.idx, r.weight, expert_cache(inp), c.E, shared_f64(inp))
    want = oracle.forward_by_expert(*args, **kw)
    hook = WorkspaceActivations(inp, ws, L, codes_path)
    got = oracle.forward_by_expert(*args, **kw, h_hook=hook)
    np.testing.assert_array_equal(got, want)
    assert hook.n == (c.T * c.K + c.T) * c.I
    ldh = max(c.I, c.I_shared)
    for g in (0, c.E):          # a routed group, then the shared one
        bad = ws.clone()
        row = int(offsets[g])
        if g == c.E and codes_path[1]:
            bad[L.h + c.T * c.K * ldh + row * ldh] ^= 1
        elif g < c.E and codes_path[0]:
            bad[L.hq + row * ldh + 3] ^= 0x10
        else:
            bad[L.h + 2 * row * ldh + 1] ^= 1
        hook = WorkspaceActivations(inp, bad, L, codes_path)
        with pytest.raises(AssertionError):
            oracle.forward_by_expert(*args, **kw, h_hook=hook)
