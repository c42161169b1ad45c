"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Small and medium cases run the oracle on every token; they span the
weight-streaming path (T <= 64; groups of one and of several 16-row
tiles) and the tiled path
(several row tiles per expert with ragged tails), fp32 and bf16, both routing
modes, with/without the shared expert, K = E, E = 256, forced routing and the
empty batch.  The full-size workloads check every route index and a seeded
sample of output rows (plus every near-tie token) in the launch
configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_amd as sm
from gpu_util import (MARGIN, WorkspaceActivations, act_kw, check_output, check_route,
                      config_of, expert_cache, log, oracle_route, out_to_np, quant_act,
                      route_for_reference, shared_f64, to_torch, upload_weights)
from synth import CONFIGS, MoEInputs, random_small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sm.load()
    return torch.device("cuda:0")


def reference(inp, r, gidx, gw, tokens=None):
    """Oracle output on the oracle's route, except near-tie tokens, which use
    the GPU's picks (a valid top-K) with the oracle's weights for them."""
    c = inp.cfg
    x64 = inp.x_f64()
    idx, w = route_for_reference(r, gidx)
    if tokens is not None:
        x64, idx, w = x64[tokens], idx[tokens], w[tokens]
    return oracle.forward_given_route(x64, idx, w, expert_cache(inp), c.E, shared_f64(inp),
                                      **act_kw(inp))


def run_gpu(inp, dev, weights=None, workspace=None):
    c = inp.cfg
    if weights is None:
        weights = upload_weights(inp, dev)
    cfg = config_of(inp)
    x = to_torch(inp.x(), c.dtype, dev)
    out, idx, w = sm.forward(cfg, x, weights, workspace=workspace, return_route=True)
    torch.cuda.synchronize()
    return out, idx.cpu().numpy(), w.cpu().numpy()


def full_check(inp, dev, **kw):
    c = inp.cfg
    log(f"case {c.name}: T={c.T} H={c.H} E={c.E} K={c.K} I={c.I} Is={c.I_shared} "
        f"{c.dtype} mode={c.route_mode}")
    quantised = quant_act(inp)
    if quantised and kw.get("workspace") is None:
        kw["workspace"] = sm.alloc_workspace(config_of(inp), True, dev)
    out, gidx, gw = run_gpu(inp, dev, **kw)
    r = oracle_route(inp)
    info = check_route(gidx, gw, r)
    if quantised:
        # activation codes with two valid answers: the GPU's, checked
        L = sm.hy3moe_workspace_layout(config_of(inp))
        hook = WorkspaceActivations(inp, kw["workspace"], L)
        ridx, rw = route_for_reference(r, gidx)
        ref = oracle.forward_by_expert(inp.x_f64(), ridx, rw, expert_cache(inp), c.E,
                                       shared_f64(inp), **act_kw(inp), h_hook=hook)
        log(f"  activation codes {hook.n}, {hook.n_amb} at an ambiguous decision")
    else:
        ref = reference(inp, r, gidx, gw)
    check_output(out_to_np(out), ref, c.dtype, c.name)
    return out, gidx, gw, r, info


SMALL = {
    "skinny_T1": dict(seed=1, T=1, H=512, E=32, K=8, I=256, I_shared=256, dtype="bf16"),
    "skinny_T32_rows256": dict(seed=7, T=32, H=256, E=12, K=4, I=128, I_shared=128,
                               dtype="bf16"),
    "skinny_T16": dict(seed=2, T=16, H=512, E=32, K=8, I=256, I_shared=256, dtype="bf16"),
    "skinny_T20": dict(seed=3, T=20, H=512, E=24, K=6, I=192, I_shared=128, dtype="bf16"),
    "skinny_T40": dict(seed=4, T=40, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16"),
    "skinny_T64_f32": dict(seed=5, T=64, H=256, E=16, K=4, I=128, I_shared=128, dtype="f32"),
    "tiled_T65": dict(seed=6, T=65, H=512, E=16, K=4, I=256, I_shared=256, dtype="bf16"),
    "tiled_T300_ragged": dict(seed=7, T=300, H=512, E=24, K=4, I=256, I_shared=128,
                              dtype="bf16"),
    "tiled_T200_f32": dict(seed=8, T=200, H=256, E=8, K=2, I=128, I_shared=192, dtype="f32"),
    "tiled_T700_H320": dict(seed=9, T=700, H=320, E=12, K=3, I=320, I_shared=64,
                            dtype="bf16"),
    "softmax_T150": dict(seed=10, T=150, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16",
                         route_mode=1, scale=1.0, renorm_eps=1e-8, bias_kind="none"),
    "softmax_T12": dict(seed=11, T=12, H=256, E=64, K=8, I=128, I_shared=128, dtype="bf16",
                        route_mode=1, scale=1.0, renorm_eps=1e-8, bias_kind="none"),
    "no_shared_T100": dict(seed=12, T=100, H=256, E=16, K=4, I=128, I_shared=0, dtype="bf16"),
    "no_shared_T8": dict(seed=13, T=8, H=256, E=16, K=4, I=128, I_shared=0, dtype="f32"),
    "k_equals_E": dict(seed=14, T=90, H=256, E=8, K=8, I=128, I_shared=128, dtype="bf16"),
    "E256_K16": dict(seed=15, T=80, H=256, E=256, K=16, I=64, I_shared=64, dtype="bf16"),
    "E1_K1": dict(seed=16, T=33, H=128, E=1, K=1, I=64, I_shared=64, dtype="bf16"),
    # large-tile path (mean routed rows per expert >= 192): ragged row tails,
    # an I % 128 == 64 gate-up column tail and an H % 256 == 64 down column tail
    "big_T400_E8": dict(seed=17, T=400, H=512, E=8, K=4, I=256, I_shared=128, dtype="bf16"),
    "big_T513_tails": dict(seed=18, T=513, H=320, E=4, K=2, I=192, I_shared=64, dtype="bf16"),
    "big_T300_f32": dict(seed=19, T=300, H=256, E=2, K=2, I=128, I_shared=192, dtype="f32"),
    "big_softmax_T600": dict(seed=20, T=600, H=256, E=8, K=3, I=128, I_shared=128, dtype="bf16",
                             route_mode=1, scale=1.0, renorm_eps=1e-8, bias_kind="none"),
    # FP8 E4M3 expert weights (weight-streaming path at 1 to 64 tokens;
    # ragged K blocks; no shared expert; softmax routing)
    "fp8_T1": dict(seed=30, T=1, H=512, E=32, K=8, I=256, I_shared=256, dtype="bf16",
                   w_format="fp8_e4m3"),
    "fp8_T16": dict(seed=31, T=16, H=512, E=32, K=8, I=256, I_shared=256, dtype="bf16",
                    w_format="fp8_e4m3"),
    "fp8_T20_noshared": dict(seed=32, T=20, H=512, E=24, K=6, I=192, I_shared=0,
                             dtype="bf16", w_format="fp8_e4m3"),
    "fp8_T40_H320": dict(seed=33, T=40, H=320, E=12, K=3, I=320, I_shared=64, dtype="bf16",
                         w_format="fp8_e4m3"),
    "fp8_T64_softmax": dict(seed=34, T=64, H=256, E=16, K=4, I=128, I_shared=128,
                            dtype="bf16", route_mode=1, scale=1.0, renorm_eps=1e-8,
                            bias_kind="none", w_format="fp8_e4m3"),
    # ... and on the 128-row tiled path and the large-tile path (ragged row
    # tails, I % 128 == 64 and H % 256 == 64 column tails)
    "fp8_tiled_T300": dict(seed=35, T=300, H=512, E=24, K=4, I=256, I_shared=128,
                           dtype="bf16", w_format="fp8_e4m3"),
    "fp8_tiled_T700_H320": dict(seed=36, T=700, H=320, E=12, K=3, I=320, I_shared=64,
                                dtype="bf16", w_format="fp8_e4m3"),
    "fp8_big_T513_tails": dict(seed=37, T=513, H=320, E=4, K=2, I=192, I_shared=64,
                               dtype="bf16", w_format="fp8_e4m3"),
    "fp8_big_T400_softmax": dict(seed=38, T=400, H=512, E=8, K=4, I=256, I_shared=128,
                                 dtype="bf16", route_mode=1, scale=1.0, renorm_eps=1e-8,
                                 bias_kind="none", w_format="fp8_e4m3"),
    # Static FP8 activations (W8A8) on every path: weight streaming (16 and 64
    # tokens), tiled, large-tile FP8 MFMAs (with an H % 256 == 128
    # column tail and softmax routing), and an H % 128 != 0 batch that the
    # large-tile path hands to the tiled one
    "w8a8_T16": dict(seed=40, T=16, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16",
                     w_format="fp8_e4m3", act_format="fp8_static"),
    "w8a8_T64_noshared": dict(seed=41, T=64, H=512, E=8, K=2, I=256, I_shared=0,
                              dtype="bf16", w_format="fp8_e4m3", act_format="fp8_static"),
    # weight-streaming W8A8 at 32 tokens (FP8 x FP8 MFMAs), and
    # with a K that is not a multiple of 128 (bf16 values of the codes)
    "w8a8_T32_codes": dict(seed=43, T=32, H=384, E=12, K=4, I=256, I_shared=128, dtype="bf16",
                           w_format="fp8_e4m3", act_format="fp8_static"),
    "w8a8_T16_values": dict(seed=44, T=16, H=320, E=10, K=4, I=192, I_shared=64, dtype="bf16",
                            w_format="fp8_e4m3", act_format="fp8_static"),
    # every weight row a multiple of 256 bytes: the
    # four-row weight loads (W8A8, W4A8 and bf16)
    "w8a8_T8_rows256": dict(seed=45, T=8, H=512, E=8, K=2, I=256, I_shared=256, dtype="bf16",
                            w_format="fp8_e4m3", act_format="fp8_static"),
    "w8a8_T24_rows256": dict(seed=46, T=24, H=512, E=8, K=2, I=256, I_shared=256, dtype="bf16",
                             w_format="fp8_e4m3", act_format="fp8_static"),
    "w8a8_tiled_T300": dict(seed=42, T=300, H=512, E=24, K=4, I=256, I_shared=128,
                            dtype="bf16", w_format="fp8_e4m3", act_format="fp8_static"),
    "w8a8_big_T513_H384": dict(seed=43, T=513, H=384, E=4, K=2, I=256, I_shared=128,
                               dtype="bf16", w_format="fp8_e4m3", act_format="fp8_static"),
    "w8a8_big_T400_softmax": dict(seed=44, T=400, H=512, E=8, K=4, I=256, I_shared=128,
                                  dtype="bf16", route_mode=1, scale=1.0, renorm_eps=1e-8,
                                  bias_kind="none", w_format="fp8_e4m3",
                                  act_format="fp8_static"),
    "w8a8_T700_H320_to_tiled": dict(seed=45, T=700, H=320, E=4, K=3, I=192, I_shared=64,
                                    dtype="bf16", w_format="fp8_e4m3",
                                    act_format="fp8_static"),
    # MXFP4 weights (E2M1 codes, E8M0 scale per 32) on the weight-streaming
    # path: 1 to 64 tokens, softmax routing, no shared expert, a
    # shared expert wider than the routed ones
    "mxfp4_T1": dict(seed=70, T=1, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16",
                     w_format="mxfp4"),
    "mxfp4_T16": dict(seed=71, T=16, H=512, E=32, K=4, I=256, I_shared=128, dtype="bf16",
                      w_format="mxfp4"),
    # x in LDS: rows of 192 bytes (no grouped loads, three
    # steps per set) and of 384 bytes (two groups of two per set, a partial
    # last set)
    "mxfp4_T8_H384": dict(seed=78, T=8, H=384, E=8, K=2, I=128, I_shared=128, dtype="bf16",
                          w_format="mxfp4"),
    "mxfp4_T12_H768": dict(seed=79, T=12, H=768, E=12, K=3, I=256, I_shared=128,
                           dtype="bf16", w_format="mxfp4"),
    "mxfp4_T20_noshared": dict(seed=72, T=20, H=256, E=8, K=2, I=128, I_shared=0,
                               dtype="bf16", w_format="mxfp4"),
    "mxfp4_T64_softmax": dict(seed=73, T=64, H=384, E=16, K=4, I=128, I_shared=256,
                              dtype="bf16", route_mode=1, scale=1.0, renorm_eps=1e-8,
                              bias_kind="none", w_format="mxfp4"),
    # ... and on the tiled and large-tile paths (ragged row tails; I % 256 ==
    # 128 and H % 256 == 128 column tails)
    "mxfp4_tiled_T300": dict(seed=74, T=300, H=512, E=24, K=4, I=256, I_shared=128,
                             dtype="bf16", w_format="mxfp4"),
    "mxfp4_tiled_T700_H384": dict(seed=75, T=700, H=384, E=12, K=3, I=384, I_shared=128,
                                  dtype="bf16", w_format="mxfp4"),
    "mxfp4_big_T513_H384": dict(seed=76, T=513, H=384, E=4, K=2, I=384, I_shared=128,
                                dtype="bf16", w_format="mxfp4"),
    "mxfp4_big_T400_softmax": dict(seed=77, T=400, H=512, E=8, K=4, I=256, I_shared=128,
                                   dtype="bf16", route_mode=1, scale=1.0, renorm_eps=1e-8,
                                   bias_kind="none", w_format="mxfp4"),
    # W4A8: MXFP4 weights with dynamic MXFP8 activations; block-scaled FP4 x
    # FP8 MFMAs on the weight-streaming path (1 to 64 tokens), the
    # same values in bf16 on the tile paths
    "w4a8_T1": dict(seed=80, T=1, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16",
                    w_format="mxfp4", act_format="mxfp8"),
    "w4a8_T16": dict(seed=81, T=16, H=512, E=32, K=4, I=256, I_shared=128, dtype="bf16",
                     w_format="mxfp4", act_format="mxfp8"),
    "w4a8_T12_rows256": dict(seed=84, T=12, H=512, E=8, K=3, I=512, I_shared=512, dtype="bf16",
                             w_format="mxfp4", act_format="mxfp8"),
    "w4a8_T24_rows128": dict(seed=85, T=24, H=512, E=8, K=2, I=256, I_shared=256, dtype="bf16",
                             w_format="mxfp4", act_format="mxfp8"),
    "w4a8_T20_noshared": dict(seed=82, T=20, H=256, E=8, K=2, I=128, I_shared=0,
                              dtype="bf16", w_format="mxfp4", act_format="mxfp8"),
    "w4a8_T64_softmax": dict(seed=83, T=64, H=384, E=16, K=4, I=128, I_shared=256,
                             dtype="bf16", route_mode=1, scale=1.0, renorm_eps=1e-8,
                             bias_kind="none", w_format="mxfp4", act_format="mxfp8"),
    "w4a8_tiled_T300": dict(seed=84, T=300, H=512, E=24, K=4, I=256, I_shared=128,
                            dtype="bf16", w_format="mxfp4", act_format="mxfp8"),
    "w4a8_big_T513_H384": dict(seed=85, T=513, H=384, E=4, K=2, I=384, I_shared=128,
                               dtype="bf16", w_format="mxfp4", act_format="mxfp8"),
    # The shared expert in formats of its own (separate launches over the
    # shared tiles, which the permutation places last): routed W4A8 with a
    # W8A8 shared expert on each path (a shared expert wider than the routed
    # ones; ragged tails), routed bf16 with an MXFP4 shared expert, routed
    # FP8 weights with a bf16 shared expert, and W8A8 routed experts with a
    # W4A8 shared one
    "mixed_T1": dict(seed=90, T=1, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16",
                     w_format="mxfp4", act_format="mxfp8", shared_w_format="fp8_e4m3",
                     shared_act_format="fp8_static"),
    "mixed_T16": dict(seed=91, T=16, H=512, E=32, K=4, I=256, I_shared=384, dtype="bf16",
                      w_format="mxfp4", act_format="mxfp8", shared_w_format="fp8_e4m3",
                      shared_act_format="fp8_static"),
    "mixed_tiled_T300": dict(seed=92, T=300, H=512, E=24, K=4, I=256, I_shared=128,
                             dtype="bf16", w_format="mxfp4", act_format="mxfp8",
                             shared_w_format="fp8_e4m3", shared_act_format="fp8_static"),
    "mixed_big_T513_H384": dict(seed=93, T=513, H=384, E=4, K=2, I=384, I_shared=256,
                                dtype="bf16", w_format="mxfp4", act_format="mxfp8",
                                shared_w_format="fp8_e4m3", shared_act_format="fp8_static"),
    "mixed_big_T400_softmax": dict(seed=94, T=400, H=512, E=8, K=4, I=256, I_shared=128,
                                   dtype="bf16", route_mode=1, scale=1.0, renorm_eps=1e-8,
                                   bias_kind="none", w_format="mxfp4", act_format="mxfp8",
                                   shared_w_format="fp8_e4m3", shared_act_format="fp8_static"),
    "mixed_bf16_shared_mxfp4_T40": dict(seed=95, T=40, H=256, E=16, K=4, I=128, I_shared=256,
                                        dtype="bf16", shared_w_format="mxfp4"),
    "mixed_fp8_shared_bf16_big_T400": dict(seed=96, T=400, H=512, E=8, K=4, I=256,
                                           I_shared=128, dtype="bf16", w_format="fp8_e4m3",
                                           shared_w_format="dtype"),
    "mixed_w8a8_shared_w4a8_T300": dict(seed=97, T=300, H=512, E=24, K=4, I=256, I_shared=128,
                                        dtype="bf16", w_format="fp8_e4m3",
                                        act_format="fp8_static", shared_w_format="mxfp4",
                                        shared_act_format="mxfp8"),
    "mixed_w8a8_shared_w4a8_big_T513": dict(seed=98, T=513, H=384, E=4, K=2, I=256,
                                            I_shared=384, dtype="bf16", w_format="fp8_e4m3",
                                            act_format="fp8_static", shared_w_format="mxfp4",
                                            shared_act_format="mxfp8"),
}


def test_cfg0_tiny_fp32(dev):
    inp = MoEInputs(CONFIGS["tiny_fp32"])
    out, gidx, gw, r, info = full_check(inp, dev)
    # the route itself: sums of weights are the scale
    np.testing.assert_allclose(gw.sum(1), 2.826, rtol=0, atol=4 * np.spacing(np.float32(2.826)))
    # brute-force dense evaluation of every expert agrees too
    dense = oracle.dense_masked(inp.x_f64(), r.idx, r.weight, inp.expert_f64, inp.cfg.E,
                                inp.shared_f64())
    check_output(out_to_np(out), dense, "f32", "cfg0 vs dense")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_small_cases(dev, name):
    full_check(random_small(**SMALL[name]), dev)


def test_forced_routing_single_expert_set(dev):
    """A +10 bias forces every token onto the same K experts: each of those
    groups holds all T rows (several row tiles)."""
    inp = random_small(21, T=333, H=256, E=16, K=3, I=128, I_shared=128, dtype="bf16")
    b = np.zeros(16, dtype=np.float32)
    b[[2, 9, 13]] = 10.0
    inp._cache[("bias",)] = b
    out, gidx, gw, r, info = full_check(inp, dev)
    assert (np.sort(gidx, 1) == np.array([2, 9, 13])).all()


# T=40: weight-streaming GEMMs (tiles in group order); 500: one-workgroup
# permutation; 3000: the three-kernel permutation (both largest groups first).
@pytest.mark.parametrize("T", [40, 500, 3000])
def test_permutation_is_exact_and_stable(dev, T):
    inp = random_small(22, T=T, H=256, E=24, K=4, I=128, I_shared=128, dtype="bf16")
    c = inp.cfg
    cfg = config_of(inp)
    L = sm.hy3moe_workspace_layout(cfg)
    ws = sm.alloc_workspace(cfg, True, dev)
    out, gidx, gw = run_gpu(inp, dev, workspace=ws)
    wsh = ws.cpu().numpy()

    def arr(off, n):
        return wsh[off:off + 4 * n].view(np.int32)

    counts = arr(L.counts, c.E + 1)
    offsets = arr(L.offsets, c.E + 2)
    N = c.T * c.K
    sorted_token = arr(L.sorted_token, N + c.T)
    pos_of = arr(L.pos_of, N)
    flat = gidx.reshape(-1)
    np.testing.assert_array_equal(counts[:c.E], np.bincount(flat, minlength=c.E))
    assert counts[c.E] == c.T
    np.testing.assert_array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    # stable order: rows of expert e are its (t, j) entries in ascending flat index
    order = np.argsort(flat, kind="stable")
    np.testing.assert_array_equal(pos_of[order], np.arange(N))
    np.testing.assert_array_equal(sorted_token[:N], order // c.K)
    np.testing.assert_array_equal(sorted_token[N:], np.arange(c.T))
    # tiles cover every row exactly once.  When the shared expert runs on
    # the side stream (the large-tile path) its tiles come last, after the
    # routed tile count; the groups before are ranked largest first on the
    # tile-grid paths and kept in group order on the weight-streaming path
    tiles = arr(L.tiles, 2 * L.max_tiles + 2)
    nt, n_routed = tiles[-2], tiles[-1]
    pairs = tiles[:2 * nt].reshape(-1, 2)
    covered = np.zeros(N + c.T, dtype=int)
    for g, r0 in pairs:
        covered[r0:min(r0 + L.tile_rows, offsets[g + 1])] += 1
    assert (covered == 1).all()
    side = L.shared_meta > 0
    assert side == (L.gemm_path == 2)
    G = c.E if side else c.E + 1
    if side:
        assert (pairs[:n_routed, 0] < c.E).all() and (pairs[n_routed:, 0] == c.E).all()
    else:
        assert n_routed == nt
    ranked = pairs[:n_routed]
    if T <= 64:
        assert (np.diff(ranked[:, 0]) >= 0).all()
    else:
        per_group = np.array([np.sum(ranked[:, 0] == g) for g in range(G)])
        firsts = [np.argmax(ranked[:, 0] == g) for g in range(G) if per_group[g]]
        assert all(per_group[ranked[i, 0]] >= per_group[ranked[j, 0]]
                   for i, j in zip(sorted(firsts)[:-1], sorted(firsts)[1:]))
    if not side:
        return
    # the side stream's own metadata: the shared tiles, empty routed groups
    # at row N, and the identity row map of the shared rows
    nm = 2 * L.max_tiles + 2
    meta = arr(L.shared_meta, nm + c.E + 2 + N + c.T)
    n_sh = -(-c.T // L.tile_rows)
    assert meta[nm - 2] == n_sh and meta[nm - 1] == 0
    np.testing.assert_array_equal(meta[:2 * n_sh].reshape(-1, 2),
                                  [[c.E, N + i * L.tile_rows] for i in range(n_sh)])
    np.testing.assert_array_equal(meta[nm:nm + c.E + 2], [N] * (c.E + 1) + [N + c.T])
    np.testing.assert_array_equal(meta[nm + c.E + 2 + N:], np.arange(c.T))


@pytest.mark.parametrize("name", ["skinny_T16", "tiled_T300_ragged", "big_T513_tails",
                                  "w8a8_big_T400_softmax", "w4a8_T16", "mixed_big_T513_H384",
                                  "mixed_tiled_T300", "skinny_T64_f32"])
def test_side_stream_matches_the_serial_chain(dev, name):
    """hy3moe_forward runs the shared expert on its side stream beside the
    routing chain on the large-tile path and with formats of its own;
    hy3moe_forward_static keeps every kernel on the caller's stream.  Same
    kernels on the same rows: the outputs and routes agree bit for bit, on
    every GEMM path."""
    inp = random_small(**SMALL[name])
    c = inp.cfg
    cfg = config_of(inp)
    assert sm.hy3moe_workspace_bytes(cfg, True) <= sm.load().hy3moe_static_scratch_bytes()
    w = upload_weights(inp, dev)
    x = to_torch(inp.x(), c.dtype, dev)
    log(f"side stream vs serial: {name}")
    out, idx, wt = sm.forward(cfg, x, w, return_route=True)
    ref = torch.empty_like(x)
    ridx = torch.empty_like(idx)
    rwt = torch.empty_like(wt)
    sm.hy3moe_forward_static(cfg, x, w, ref, ridx, rwt)
    torch.cuda.synchronize()
    bits = torch.int16 if c.dtype == "bf16" else torch.int32
    assert torch.equal(out.view(bits), ref.view(bits))
    assert torch.equal(idx, ridx) and torch.equal(wt.view(torch.int32), rwt.view(torch.int32))


def test_deterministic_bitwise(dev):
    inp = random_small(23, T=257, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16")
    w = upload_weights(inp, dev)
    a, _, _ = run_gpu(inp, dev, weights=w)
    b, _, _ = run_gpu(inp, dev, weights=w)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_batch(dev):
    inp = random_small(24, T=0, H=256, E=16, K=4, I=128, I_shared=128, dtype="bf16")
    w = upload_weights(inp, dev)
    cfg = config_of(inp)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(x)
    sm.hy3moe_forward(cfg, x, w, out, torch.empty(0, dtype=torch.uint8, device=dev))
    torch.cuda.synchronize()


def test_route_entry_matches_forward_route(dev):
    inp = random_small(25, T=77, H=512, E=32, K=8, I=128, I_shared=128, dtype="bf16")
    w = upload_weights(inp, dev)
    cfg = config_of(inp)
    x = to_torch(inp.x(), "bf16", dev)
    idx, wt = sm.route(cfg, x, w["w_router"], w["expert_bias"])
    _, fidx, fw = run_gpu(inp, dev, weights=w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), fidx)
    np.testing.assert_array_equal(wt.cpu().numpy(), fw)
    check_route(fidx, fw, oracle_route(inp))


@pytest.mark.parametrize("route_mode", [0, 1])
def test_route_indices_valid_with_nan_scores(dev, route_mode):
    """Rows of x holding NaN give NaN logits.  The routing still returns K
    distinct experts in [0, E) for every token (NaN scores never compare
    equal, so the selection falls back to the lowest remaining experts),
    and the rows without NaN match the oracle's routing.  hy3moe_route only:
    no kernel here indexes memory with the picks."""
    inp = random_small(26, T=70, H=256, E=24, K=6, I=128, I_shared=128, dtype="bf16",
                       route_mode=route_mode)
    w = upload_weights(inp, dev)
    cfg = config_of(inp)
    xb = np.array(inp.x(), copy=True)            # bf16 bits [T][H]
    nan_rows = np.arange(0, 70, 7)
    xb[nan_rows, 5] = 0x7FC0                      # bf16 quiet NaN
    xb[nan_rows[::2], :] = 0x7FC0                 # some rows all NaN
    idx, wt = sm.route(cfg, to_torch(xb, "bf16", dev), w["w_router"], w["expert_bias"])
    torch.cuda.synchronize()
    idx = idx.cpu().numpy().reshape(70, 6)
    assert ((idx >= 0) & (idx < 24)).all()
    assert all(len(set(r)) == 6 for r in idx)
    r = oracle_route(inp)
    ok = np.setdiff1d(np.arange(70), nan_rows)
    ok = ok[r.margin[ok] > MARGIN]
    assert ok.size > 40
    np.testing.assert_array_equal(np.sort(idx[ok], 1), np.sort(r.idx[ok], 1))


@pytest.mark.parametrize("route_mode", [0, 1])
@pytest.mark.parametrize("T", [16, 300, 1100])
def test_exact_ties_go_to_the_lower_expert_index(dev, T, route_mode):
    """Experts e and e + 8 get identical router rows (and, in sigmoid mode,
    identical biases), so their scores are equal on every token.  With K = 3
    the top three are the best pair and one expert of the second-best pair:
    every token has an exact tie at the K-th place.  The documented rule
    (equal scores ordered by ascending expert index) fixes the answer: the
    GPU's picks must equal the oracle's, order included.  T = 16, 300 and
    1100 run the small, tiled and plane-split router kernels."""
    kw = dict(route_mode=1, scale=1.0, renorm_eps=1e-8, bias_kind="none") if route_mode else {}
    inp = random_small(27, T=T, H=256, E=16, K=3, I=64, I_shared=64, dtype="bf16", **kw)
    wr = np.array(inp.w_router(), copy=True)
    wr[8:] = wr[:8]
    inp._cache[("wr",)] = wr
    if route_mode == 0:
        b = np.array(inp.bias(), copy=True)
        b[8:] = b[:8]
        inp._cache[("bias",)] = b
    w = upload_weights(inp, dev)
    cfg = config_of(inp)
    idx, wt = sm.route(cfg, to_torch(inp.x(), "bf16", dev), w["w_router"], w.get("expert_bias"))
    torch.cuda.synchronize()
    gidx, gw = idx.cpu().numpy(), wt.cpu().numpy()
    r = oracle_route(inp)
    # pair-level separation: best pair, second pair and third pair apart by
    # more than the margin, so the only ties are the constructed ones
    ps = -np.sort(-r.select_score[:, :8], axis=1)
    clear = (ps[:, 0] - ps[:, 1] > MARGIN) & (ps[:, 1] - ps[:, 2] > MARGIN)
    assert clear.sum() >= 0.9 * T
    np.testing.assert_array_equal(r.margin, 0.0)
    np.testing.assert_array_equal(gidx[clear], r.idx[clear])
    # the picks hold one full pair and the lower index of the next pair
    assert ((gidx[clear][:, 1] - gidx[clear][:, 0]) == 8).all()
    assert (gidx[clear][:, 2] < 8).all()
    check_route(gidx, gw, r)
