"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin is chosen so that a plausible mistake in the oracle fails it:

* hand-worked fixtures in tests/golden (closed forms; the pages print no
  numeric worked example of the layer);
* brute force over every K-subset for the selection;
* a loop-only, scalar re-derivation of the whole layer on tiny inputs;
* the eager masked dispatch against dense evaluation of every expert;
* invariants the pages' definitions imply (weight sums, bias-only-selects,
  relabelling/permutation symmetry, special cases).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import CONFIGS, MoEInputs, random_small

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def expert_fn_from_list(lst):
    return lambda e: (np.array(lst[e][0]), np.array(lst[e][1]), np.array(lst[e][2]))


# ---------------------------------------------------------------- golden ----
def test_golden_sigmoid_bias_route():
    c = load("route_sigmoid_bias_hand.json")
    r = oracle.route_from_logits(np.array(c["logits"]), c["K"], oracle.ROUTE_SIGMOID_BIAS,
                                 np.array(c["bias"]), c["scale"])
    assert r.idx.tolist() == c["idx"]
    np.testing.assert_allclose(r.weight, c["weight"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r.margin, c["margin"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("K", ["2", "3"])
def test_golden_sigmoid_ties(K):
    c = load("route_sigmoid_ties_hand.json")
    e = c["by_K"][K]
    r = oracle.route_from_logits(np.array(c["logits"]), int(K), oracle.ROUTE_SIGMOID_BIAS,
                                 np.array(c["bias"]), c["scale"])
    assert r.idx.tolist() == e["idx"]
    np.testing.assert_allclose(r.weight, e["weight"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r.margin, e["margin"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("K", ["2", "3"])
def test_golden_softmax_route(K):
    c = load("route_softmax_hand.json")
    e = c["by_K"][K]
    r = oracle.route_from_logits(np.array(c["logits"]), int(K), oracle.ROUTE_SOFTMAX,
                                 None, 1.0, 1e-8)
    assert r.idx.tolist() == e["idx"]
    np.testing.assert_allclose(r.weight, e["weight"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(r.margin, e["margin"], rtol=0, atol=1e-14)


def test_golden_router_identity_weight_gives_logits():
    c = load("route_sigmoid_bias_hand.json")
    L = np.array(c["logits"])
    np.testing.assert_array_equal(oracle.router_logits(L, np.eye(L.shape[1])), L)


def test_golden_swiglu():
    c = load("swiglu_hand.json")
    out = oracle.swiglu_expert(np.array(c["a"]), np.array(c["w_gate"]),
                               np.array(c["w_up"]), np.array(c["w_down"]))
    np.testing.assert_allclose(out, c["out"], rtol=0, atol=1e-13)


def test_golden_layer():
    c = load("layer_hand.json")
    ex = [(d["gate"], d["up"], d["down"]) for d in c["experts"]]
    sh = tuple(np.array(c["shared"][k]) for k in ("gate", "up", "down"))
    out, r = oracle.forward(np.array(c["x"]), np.array(c["w_router"]),
                            expert_fn_from_list(ex), E=3, K=c["K"], shared=sh,
                            mode=oracle.ROUTE_SIGMOID_BIAS, bias=np.array(c["bias"]),
                            scale=c["scale"])
    assert r.idx.tolist() == c["idx"]
    np.testing.assert_allclose(r.weight, c["weight"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out, c["out"], rtol=0, atol=1e-13)


# ------------------------------------------------------------ selection ----
@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force_all_subsets(seed):
    """The picked set maximises the sum of selection scores over all K-subsets."""
    rng = np.random.default_rng(seed)
    T, E, K = 5, 7, 3
    L = rng.normal(0, 1.5, (T, E))
    bias = rng.uniform(-0.3, 0.3, E)
    r = oracle.route_from_logits(L, K, oracle.ROUTE_SIGMOID_BIAS, bias, 2.826)
    for t in range(T):
        b = [1.0 / (1.0 + math.exp(-L[t, e])) + bias[e] for e in range(E)]
        best = max(itertools.combinations(range(E), K), key=lambda S: sum(b[e] for e in S))
        assert sorted(r.idx[t].tolist()) == sorted(best)
        picked = [b[e] for e in r.idx[t]]
        assert all(picked[i] >= picked[i + 1] for i in range(K - 1))
        rest = sorted((b[e] for e in range(E) if e not in best), reverse=True)
        assert abs(r.margin[t] - (min(picked) - rest[0])) < 1e-15


def test_zero_bias_selects_top_logits():
    """sigmoid is increasing, so with zero bias the picks are the top-K logits."""
    rng = np.random.default_rng(1)
    L = rng.normal(size=(50, 33))
    r = oracle.route_from_logits(L, 6, oracle.ROUTE_SIGMOID_BIAS, np.zeros(33), 2.826)
    expect = np.argsort(-L, axis=1)[:, :6]
    np.testing.assert_array_equal(r.idx, expect)


def test_large_bias_forces_selection():
    rng = np.random.default_rng(2)
    E, K = 24, 5
    forced = [3, 7, 11, 19, 20]
    bias = np.zeros(E)
    bias[forced] = 10.0
    r = oracle.route_from_logits(rng.normal(size=(40, E)), K, oracle.ROUTE_SIGMOID_BIAS,
                                 bias, 2.826)
    for t in range(40):
        assert sorted(r.idx[t].tolist()) == forced


def test_bias_selects_but_weights_are_unbiased():
    rng = np.random.default_rng(3)
    L = rng.normal(size=(64, 16))
    bias = rng.uniform(-0.3, 0.3, 16)
    r = oracle.route_from_logits(L, 4, oracle.ROUTE_SIGMOID_BIAS, bias, 2.826)
    s = np.array([[1.0 / (1.0 + math.exp(-v)) for v in row] for row in L])
    r0 = oracle.route_from_logits(L, 4, oracle.ROUTE_SIGMOID_BIAS, None, 2.826)
    assert (np.sort(r.idx, 1) != np.sort(r0.idx, 1)).any(), "bias must change some picks"
    for t in range(64):
        sel = s[t, r.idx[t]]
        np.testing.assert_allclose(r.weight[t], 2.826 * sel / sel.sum(), rtol=1e-14)
    np.testing.assert_allclose(r.weight.sum(1), 2.826, rtol=0, atol=1e-12)


def test_softmax_weights_sum_to_one_and_shift_invariant():
    rng = np.random.default_rng(4)
    L = rng.normal(size=(32, 64))
    r = oracle.route_from_logits(L, 8, oracle.ROUTE_SOFTMAX, None, 1.0, 1e-8)
    np.testing.assert_allclose(r.weight.sum(1), 1.0, rtol=0, atol=1e-14)
    r2 = oracle.route_from_logits(L + rng.normal(size=(32, 1)) * 5, 8, oracle.ROUTE_SOFTMAX,
                                  None, 1.0, 1e-8)
    np.testing.assert_array_equal(r.idx, r2.idx)
    np.testing.assert_allclose(r.weight, r2.weight, rtol=1e-12)
    np.testing.assert_allclose(r.prob.sum(1), 1.0, atol=1e-14)


def test_softmax_and_sigmoid_against_math():
    z = np.array([-800.0, -30.0, -1.0, 0.0, 0.5, 30.0, 800.0])
    expect = [0.0 if v < -700 else 1.0 / (1.0 + math.exp(-v)) for v in z]
    np.testing.assert_allclose(oracle.sigmoid(z), expect, rtol=1e-15, atol=1e-300)
    row = np.array([[1.0, 2.0, 3.0]])
    den = math.exp(1) + math.exp(2) + math.exp(3)
    np.testing.assert_allclose(oracle.softmax_rows(row),
                               [[math.exp(1) / den, math.exp(2) / den, math.exp(3) / den]],
                               rtol=1e-15)


def test_logits_against_fsum():
    inp = MoEInputs(CONFIGS["tiny_fp32"])
    x, w = inp.x_f64(), inp.w_router().astype(np.float64)
    L = oracle.router_logits(x, w)
    rng = np.random.default_rng(5)
    for _ in range(40):
        t, e = int(rng.integers(x.shape[0])), int(rng.integers(w.shape[0]))
        ref = math.fsum(float(x[t, h]) * float(w[e, h]) for h in range(x.shape[1]))
        assert abs(L[t, e] - ref) <= 1e-14 * max(1.0, abs(ref))


# ---------------------------------------------------------- whole layer ----
def _scalar_layer(x, wr, bias, experts, shared, K, scale):
    """Loop-only statement of the layer, token by token, no numpy arithmetic."""
    T, H = len(x), len(x[0])
    E = len(wr)
    outs = []
    for t in range(T):
        logit = [sum(x[t][h] * wr[e][h] for h in range(H)) for e in range(E)]
        s = [1.0 / (1.0 + math.exp(-v)) for v in logit]
        b = [s[e] + bias[e] for e in range(E)]
        picks = sorted(range(E), key=lambda e: (-b[e], e))[:K]
        tot = sum(s[e] for e in picks)
        out = [0.0] * H
        terms = [(e, scale * s[e] / tot) for e in picks] + [(None, 1.0)]
        for e, w in terms:
            wg, wu, wd = shared if e is None else experts[e]
            I = len(wg)
            g = [sum(wg[i][h] * x[t][h] for h in range(H)) for i in range(I)]
            u = [sum(wu[i][h] * x[t][h] for h in range(H)) for i in range(I)]
            hh = [g[i] / (1.0 + math.exp(-g[i])) * u[i] for i in range(I)]
            for o in range(H):
                out[o] += w * sum(wd[o][i] * hh[i] for i in range(I))
        outs.append(out)
    return outs


@pytest.mark.parametrize("seed", range(3))
def test_layer_matches_scalar_loops(seed):
    inp = random_small(seed, T=4, H=6, E=5, K=2, I=3, I_shared=2)
    c = inp.cfg
    x = inp.x_f64()
    wr = inp.w_router().astype(np.float64)
    bias = inp.bias().astype(np.float64)
    ex = [inp.expert_f64(e) for e in range(c.E)]
    sh = inp.shared_f64()
    out, _ = oracle.forward(x, wr, lambda e: ex[e], c.E, c.K, sh,
                            oracle.ROUTE_SIGMOID_BIAS, bias, c.scale)
    ref = _scalar_layer(x.tolist(), wr.tolist(), bias.tolist(),
                        [tuple(a.tolist() for a in t) for t in ex],
                        tuple(a.tolist() for a in sh), c.K, c.scale)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def _cfg0():
    inp = MoEInputs(CONFIGS["tiny_fp32"])
    c = inp.cfg
    ex = [inp.expert_f64(e) for e in range(c.E)]
    return inp, c, inp.x_f64(), inp.w_router().astype(np.float64), \
        inp.bias().astype(np.float64), ex, inp.shared_f64()


def test_eager_equals_dense_masked_cfg0():
    inp, c, x, wr, bias, ex, sh = _cfg0()
    out, r = oracle.forward(x, wr, lambda e: ex[e], c.E, c.K, sh,
                            oracle.ROUTE_SIGMOID_BIAS, bias, c.scale)
    dense = oracle.dense_masked(x, r.idx, r.weight, lambda e: ex[e], c.E, sh)
    np.testing.assert_allclose(out, dense, rtol=0, atol=1e-12)
    assert np.abs(out).max() > 0.1


@pytest.mark.parametrize("seed", range(4))
def test_eager_equals_dense_masked_random(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(2, 9))
    K = int(rng.integers(1, E + 1))
    inp = random_small(seed, T=int(rng.integers(1, 12)), H=8, E=E, K=K, I=5, I_shared=4)
    c = inp.cfg
    ex = [inp.expert_f64(e) for e in range(E)]
    x = inp.x_f64()
    out, r = oracle.forward(x, inp.w_router().astype(np.float64), lambda e: ex[e], E, K,
                            inp.shared_f64(), oracle.ROUTE_SIGMOID_BIAS,
                            inp.bias().astype(np.float64), c.scale)
    dense = oracle.dense_masked(x, r.idx, r.weight, lambda e: ex[e], E, inp.shared_f64())
    np.testing.assert_allclose(out, dense, rtol=0, atol=1e-12)


def test_softmax_layer_eager_equals_dense():
    inp = random_small(7, T=9, H=8, E=6, K=3, I=5, I_shared=4, route_mode=1, scale=1.0,
                       renorm_eps=1e-8, bias_kind="none")
    c = inp.cfg
    ex = [inp.expert_f64(e) for e in range(c.E)]
    x = inp.x_f64()
    out, r = oracle.forward(x, inp.w_router().astype(np.float64), lambda e: ex[e], c.E, c.K,
                            inp.shared_f64(), oracle.ROUTE_SOFTMAX, None, 1.0, 1e-8)
    dense = oracle.dense_masked(x, r.idx, r.weight, lambda e: ex[e], c.E, inp.shared_f64())
    np.testing.assert_allclose(out, dense, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r.weight.sum(1), 1.0, atol=1e-14)


def test_token_permutation_equivariance_and_duplicates():
    inp, c, x, wr, bias, ex, sh = _cfg0()
    perm = np.random.default_rng(6).permutation(c.T)
    f = lambda e: ex[e]
    out, _ = oracle.forward(x, wr, f, c.E, c.K, sh, 0, bias, c.scale)
    out_p, _ = oracle.forward(x[perm], wr, f, c.E, c.K, sh, 0, bias, c.scale)
    np.testing.assert_allclose(out_p, out[perm], rtol=0, atol=1e-13)
    xd = np.concatenate([x, x[:3]])
    out_d, _ = oracle.forward(xd, wr, f, c.E, c.K, sh, 0, bias, c.scale)
    np.testing.assert_allclose(out_d[c.T:], out[:3], rtol=0, atol=1e-13)


def test_expert_relabelling_invariance():
    inp, c, x, wr, bias, ex, sh = _cfg0()
    perm = np.random.default_rng(7).permutation(c.E)       # new expert i is old perm[i]
    f = lambda e: ex[e]
    out, r = oracle.forward(x, wr, f, c.E, c.K, sh, 0, bias, c.scale)
    out2, r2 = oracle.forward(x, wr[perm], lambda e: ex[perm[e]], c.E, c.K, sh, 0,
                              bias[perm], c.scale)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.sort(perm[r2.idx], 1), np.sort(r.idx, 1))


def test_k_equals_E_makes_bias_irrelevant():
    inp = random_small(11, T=6, H=8, E=5, K=5, I=4, I_shared=3)
    c = inp.cfg
    ex = [inp.expert_f64(e) for e in range(c.E)]
    x, wr = inp.x_f64(), inp.w_router().astype(np.float64)
    o1, r1 = oracle.forward(x, wr, lambda e: ex[e], c.E, c.K, inp.shared_f64(), 0,
                            inp.bias().astype(np.float64), c.scale)
    o2, _ = oracle.forward(x, wr, lambda e: ex[e], c.E, c.K, inp.shared_f64(), 0,
                           np.linspace(-1, 1, c.E), c.scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    assert np.isinf(r1.margin).all()


def test_zero_down_weights_leave_only_shared():
    inp, c, x, wr, bias, ex, sh = _cfg0()
    zero = [(g, u, np.zeros_like(d)) for g, u, d in ex]
    out, _ = oracle.forward(x, wr, lambda e: zero[e], c.E, c.K, sh, 0, bias, c.scale)
    np.testing.assert_allclose(out, oracle.swiglu_expert(x, *sh), rtol=0, atol=0)


def test_no_shared_expert():
    inp, c, x, wr, bias, ex, sh = _cfg0()
    f = lambda e: ex[e]
    with_sh, r = oracle.forward(x, wr, f, c.E, c.K, sh, 0, bias, c.scale)
    without, _ = oracle.forward(x, wr, f, c.E, c.K, None, 0, bias, c.scale)
    np.testing.assert_allclose(with_sh - without, oracle.swiglu_expert(x, *sh), atol=1e-13)


def test_empty_token_batch():
    inp, c, x, wr, bias, ex, sh = _cfg0()
    out, r = oracle.forward(x[:0], wr, lambda e: ex[e], c.E, c.K, sh, 0, bias, c.scale)
    assert out.shape == (0, c.H) and r.idx.shape == (0, c.K)


def test_flop_count():
    f = oracle.layer_flops(T=8192, H=4096, E=192, K=8, I=1536, I_shared=1536)
    assert abs(f["experts"] - 2.783e12) / 2.783e12 < 1e-3


# ------------------------------------------------------ FP8 expert weights ----
# OCP FP8 E4M3 (the encoding the FP8 weights are read in): code -> value,
# worked by hand from the layout (sign, exponent bias 7, 3 mantissa bits,
# subnormals at exponent field 0, S.1111.111 = NaN, no infinities).
E4M3_HAND = {
    0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
    0x0F: 1.875 * 2.0 ** -6, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0,
    0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x81: -(2.0 ** -9),
}


def test_fp8_e4m3_hand_values():
    codes = np.array(list(E4M3_HAND), dtype=np.uint8)
    got = oracle.fp8_e4m3_value(codes)
    np.testing.assert_array_equal(got, np.array(list(E4M3_HAND.values())))
    v = oracle.fp8_e4m3_value(np.array([0x7F, 0xFF, 0x80], dtype=np.uint8))
    assert np.isnan(v[0]) and np.isnan(v[1]) and v[2] == 0.0 and np.signbit(v[2])


def test_fp8_e4m3_matches_torch_for_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.fp8_e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_fp8_e4m3_structure():
    v = oracle.fp8_e4m3_value(np.arange(256, dtype=np.uint8))
    pos = v[:0x7F]                       # codes 0x00..0x7E
    assert (np.diff(pos) > 0).all()      # strictly increasing magnitudes
    np.testing.assert_array_equal(v[0x80:0xFF], -pos)
    assert np.isnan(v).sum() == 2
    assert len(np.unique(v[~np.isnan(v)])) == 253        # +0 and -0 compare equal
    # spacing: 2^-9 through the subnormals and the first binade, then doubling
    np.testing.assert_array_equal(np.diff(pos[:16]), np.full(15, 2.0 ** -9))
    assert pos[-1] - pos[-2] == 32.0


def test_fp8_dequant_is_scale_times_value():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, size=(7, 9)).astype(np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x10
    s = np.float32(0.0123)
    d = oracle.dequant_fp8(codes, s)
    np.testing.assert_array_equal(d, np.float64(s) * oracle.fp8_e4m3_value(codes))
    # exact: the product of a 4-bit significand and a 24-bit one fits float64
    assert (d / np.float64(s) == oracle.fp8_e4m3_value(codes)).all()


def test_fp8_layer_equals_layer_on_dequantised_weights():
    """The FP8 layer is the float64 layer on scale * value weights: a scale of
    2^k on a down matrix scales that expert's routed output by exactly 2^k."""
    inp = MoEInputs(CONFIGS["hy3_decode_T16_fp8"].with_T(6).with_(H=64, E=4, K=2, I=32, I_shared=32))
    c = inp.cfg
    x = inp.x_f64()
    wr = inp.w_router().astype(np.float64)
    experts = {}
    for e in range(c.E):
        codes, sc = inp.expert_fp8(e)
        experts[e] = tuple(oracle.dequant_fp8(q, s) for q, s in zip(codes, sc))
    out, r = oracle.forward(x, wr, lambda e: experts[e], c.E, c.K, None, 0,
                            inp.bias().astype(np.float64), c.scale)
    doubled = {e: (g, u, 2.0 * d) for e, (g, u, d) in experts.items()}
    out2 = oracle.forward_given_route(x, r.idx, r.weight, lambda e: doubled[e], c.E)
    np.testing.assert_allclose(out2, 2.0 * out, rtol=0, atol=0)


# --------------------------------------------------------------------------
# Static FP8 activations (W8A8): E4M3 quantiser and the layer that uses it
# --------------------------------------------------------------------------
_FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_e4m3_quant_round_trips_every_finite_code():
    """Every finite E4M3 value quantises (scale 1) back to its own code."""
    v = oracle.fp8_e4m3_value(_FINITE)
    np.testing.assert_array_equal(oracle.quant_e4m3(v, 1.0), _FINITE)


def test_e4m3_quant_ties_go_to_even_mantissa():
    """Midpoints of neighbouring codes go to the even code; a float32 ulp
    above or below decides for the upper or lower one."""
    for sign in (0, 0x80):
        lo = np.arange(0, 0x7E, dtype=np.int64) | sign
        hi = lo + 1
        vl = oracle.fp8_e4m3_value(lo.astype(np.uint8))
        vh = oracle.fp8_e4m3_value(hi.astype(np.uint8))
        mid = ((vl + vh) / 2).astype(np.float32)
        assert (mid.astype(np.float64) == (vl + vh) / 2).all()   # exact in float32
        even = np.where(lo % 2 == 0, lo, hi).astype(np.uint8)
        np.testing.assert_array_equal(oracle.quant_e4m3(mid, 1.0), even)
        away = np.nextafter(mid, np.float32(np.copysign(np.inf, mid[1])))
        toward = np.nextafter(mid, np.float32(0))
        np.testing.assert_array_equal(oracle.quant_e4m3(away, 1.0), hi.astype(np.uint8))
        np.testing.assert_array_equal(oracle.quant_e4m3(toward, 1.0), lo.astype(np.uint8))


def test_e4m3_quant_decides_in_float32():
    """A float64 value just above a tie that rounds onto the tie in float32 is
    a tie (the decision is taken on the float32 value)."""
    tie = np.float64(1.0625)                       # between 1.0 (0x38) and 1.125 (0x39)
    v = tie + 2.0 ** -40                           # above the tie in float64 only
    assert np.float32(v) == np.float32(tie)
    assert oracle.quant_e4m3(np.array([v]), 1.0)[0] == 0x38
    assert oracle.quant_e4m3(np.array([tie + 2.0 ** -20]), 1.0)[0] == 0x39


def test_e4m3_quant_matches_torch_cast_after_clamp():
    """Against torch's float32 -> float8_e4m3fn cast (round to nearest even,
    no saturation) of the clamped float32 quotient."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    n = 200_000
    mag = np.exp2(rng.uniform(-16, 11, n))
    v = (np.where(rng.random(n) < 0.5, -1.0, 1.0) * mag).astype(np.float32)
    for s in (1.0, 0.0101, 4.5 / 448, 1.7):
        got = oracle.quant_e4m3(v, s)
        q = torch.from_numpy(v) / torch.tensor(s, dtype=torch.float32)
        ref = q.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(got, ref)


def test_e4m3_quant_saturates_and_keeps_the_sign_of_zero():
    v = np.array([448.0, 464.0, 465.0, 1e30, -1e30, 0.0, -0.0, 2.0 ** -11, -2.0 ** -11])
    np.testing.assert_array_equal(oracle.quant_e4m3(v, 1.0),
                                  [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x00, 0x80])


def test_e4m3_quant_dequant_is_invariant_under_power_of_two_scales():
    """In the normal range, scaling the static scale by 2^k shifts the grid by
    whole binades: the dequantised values do not change."""
    rng = np.random.default_rng(8)
    s = 0.03
    # |v / s| in [2^-3, 2^7.5]: normal at every scale 2^k s below (k = 3 .. -1)
    v = s * np.exp2(rng.uniform(-3.0, 7.5, 10_000)) * np.where(rng.random(10_000) < 0.5, -1, 1)
    a = oracle.quant_dequant_e4m3(v, s)
    for k in (-1, 1, 3):
        np.testing.assert_array_equal(oracle.quant_dequant_e4m3(v, s * 2.0 ** k), a)
    # ... and the dequantised value is within half a grid step (2^-4 relative)
    assert (np.abs(a - v) <= np.abs(v) * 2.0 ** -4 + 1e-300).all()


def _w8a8_small(seed, T=12, H=64, E=5, K=2, I=32, I_shared=32, xmax=1.5, hmax=0.5):
    """A small FP8 layer with static activation scales a1 = xmax / 448 and
    a2[e] = hmax (1 + e / 4) / 448 (small maxima saturate many values)."""
    inp = random_small(seed, T, H, E, K, I, I_shared, dtype="bf16", w_format="fp8_e4m3")
    c = inp.cfg
    experts = {}
    for e in range(c.E):
        codes, sc = inp.expert_fp8(e)
        experts[e] = tuple(oracle.dequant_fp8(q, s) for q, s in zip(codes, sc))
    codes, sc = inp.shared_fp8()
    shared = tuple(oracle.dequant_fp8(q, s) for q, s in zip(codes, sc))
    r = oracle.route(inp.x_f64(), inp.w_router().astype(np.float64), c.K, 0,
                     inp.bias().astype(np.float64), c.scale)
    a1 = xmax / 448
    a2 = np.float32(hmax / 448) * (1.0 + np.arange(c.E + 1, dtype=np.float64) / 4)
    return inp, experts, shared, r, (a1, a2)


@pytest.mark.parametrize("seed", [1, 2])
def test_w8a8_layer_eager_equals_dense_masked(seed):
    inp, experts, shared, r, a8 = _w8a8_small(seed)
    c = inp.cfg
    x = inp.x_f64()
    got = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared, a8=a8)
    ref = oracle.dense_masked(x, r.idx, r.weight, lambda e: experts[e], c.E, shared, a8=a8)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_w8a8_layer_scalar_loops():
    """One token through a loop-only evaluation: quantise x with a1, run every
    picked expert with element loops, round each h value to bfloat16 (by
    torch) and quantise it with that expert's a2, and sum with the route
    weights."""
    torch = pytest.importorskip("torch")
    inp, experts, shared, r, (a1, a2) = _w8a8_small(3, T=2, H=16, E=4, K=2, I=8, I_shared=8)
    c = inp.cfg
    x = inp.x_f64()
    got = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared,
                                     a8=(a1, a2))
    for t in range(c.T):
        xq = [float(oracle.quant_dequant_e4m3(np.array([x[t, k]]), a1)[0]) for k in range(c.H)]
        ref = [0.0] * c.H
        picks = [(int(r.idx[t, j]), float(r.weight[t, j])) for j in range(c.K)] + [(c.E, 1.0)]
        for e, w in picks:
            wg, wu, wd = experts[e] if e < c.E else shared
            hq = []
            for i in range(wg.shape[0]):
                g = math.fsum(xq[k] * wg[i, k] for k in range(c.H))
                u = math.fsum(xq[k] * wu[i, k] for k in range(c.H))
                h = g / (1.0 + math.exp(-g)) * u
                hb = float(torch.tensor([h], dtype=torch.float32).to(torch.bfloat16).double())
                hq.append(float(oracle.quant_dequant_e4m3(np.array([hb]), a2[e])[0]))
            for n in range(c.H):
                ref[n] += w * math.fsum(hq[i] * wd[n, i] for i in range(len(hq)))
        np.testing.assert_allclose(got[t], ref, rtol=1e-12, atol=1e-13)


def test_w8a8_layer_is_within_the_quantisation_error_of_w8a16():
    """Quantising x and h (3 mantissa bits, round to nearest: at most 2^-4
    relative each) moves the output by a few percent, never by a factor; the
    difference is not zero (the activations really are quantised)."""
    inp, experts, shared, r, a8 = _w8a8_small(4, T=64, H=128, E=6, K=2, I=64, I_shared=64,
                                              xmax=5.0, hmax=12.0)
    c = inp.cfg
    x = inp.x_f64()
    ref = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared)
    got = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared, a8=a8)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 0.005 < rel < 0.08, rel


# --------------------------------------------------------------------------
# MXFP4 expert weights: E2M1 codes with E8M0 block scales
# --------------------------------------------------------------------------
# OCP Microscaling Formats v1.0, FP4 E2M1 table: codes 0..7 and their values
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    v = oracle.fp4_e2m1_value(np.arange(16))
    np.testing.assert_array_equal(v[:8], E2M1_TABLE)
    np.testing.assert_array_equal(v[8:], [-x for x in E2M1_TABLE])
    assert np.signbit(v[8])                        # code 8 is -0


def test_e8m0_matches_torch_for_every_code():
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    with np.errstate(invalid="ignore"):                   # code 255 is NaN
        ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).float().numpy()
        ref = ref.astype(np.float64)
    got = oracle.e8m0_value(codes)
    np.testing.assert_array_equal(got[:255], ref[:255])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert got[127] == 1.0 and got[128] == 2.0 and got[120] == 2.0 ** -7


def test_mxfp4_dequant_packing_and_blocks():
    """Even element in the low nibble; one scale per 32 consecutive elements."""
    packed = np.zeros((2, 32), dtype=np.uint8)          # 2 rows, K = 64
    packed[0, 0] = 0x7A                                  # el 0 = code 0xA (-1), el 1 = 7 (6)
    packed[0, 15] = 0x30                                 # el 31 = code 3 (1.5)
    packed[0, 16] = 0x05                                 # el 32 = code 5 (3)
    packed[1, 31] = 0xF0                                 # el 63 = code 0xF (-6)
    scales = np.array([[127, 129], [120, 121]], dtype=np.uint8)
    d = oracle.dequant_mxfp4(packed, scales)
    assert d.shape == (2, 64)
    assert d[0, 0] == -1.0 and d[0, 1] == 6.0 and d[0, 31] == 1.5
    assert d[0, 32] == 3.0 * 4.0                          # second block: scale 2^2
    assert d[1, 63] == -6.0 * 2.0 ** -6
    assert (d[0, 2:31] == 0).all() and (d[1, :63] == 0).all()


def test_mxfp4_layer_equals_layer_on_dequantised_weights():
    """An E8M0 scale code one higher on every block of a down matrix doubles
    that expert's routed output exactly (the layer runs on scale * value)."""
    inp = random_small(61, 6, 64, 4, 2, 32, 32, dtype="bf16", w_format="mxfp4")
    c = inp.cfg
    x = inp.x_f64()
    deq = {}
    for e in range(c.E):
        codes, sc = inp.expert_mxfp4(e)
        deq[e] = tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(codes, sc))
    r = oracle.route(x, inp.w_router().astype(np.float64), c.K, 0,
                     inp.bias().astype(np.float64), c.scale)
    out = oracle.forward_given_route(x, r.idx, r.weight, lambda e: deq[e], c.E)
    up1 = {}
    for e in range(c.E):
        codes, sc = inp.expert_mxfp4(e)
        up1[e] = (deq[e][0], deq[e][1], oracle.dequant_mxfp4(codes[2], sc[2] + 1))
    out2 = oracle.forward_given_route(x, r.idx, r.weight, lambda e: up1[e], c.E)
    np.testing.assert_array_equal(out2, 2.0 * out)


# --------------------------------------------------------------------------
# Dynamic MXFP8 activations (W4A8)
# --------------------------------------------------------------------------
def _nearest_e4m3_brute(q: float) -> int:
    """E4M3 code nearest to q (saturating at 448), ties to the even code, by
    search over every finite code."""
    best, bestd = None, None
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        v = float(oracle.fp8_e4m3_value(np.array([c], dtype=np.uint8))[0])
        if math.copysign(1.0, v) != math.copysign(1.0, q) and v != 0.0:
            continue
        d = abs(min(abs(q), 448.0) * math.copysign(1.0, q) - v)
        if bestd is None or d < bestd or (d == bestd and (c & 1) == 0 and (best & 1) == 1):
            best, bestd = c, d
    if best is not None and float(oracle.fp8_e4m3_value(np.array([best], np.uint8))[0]) == 0.0:
        best = 0x80 if math.copysign(1.0, q) < 0 else 0x00
    return best


def test_mxfp8_quant_against_brute_force():
    """Per block: scale 2^(floor(log2 amax) - 8) from the float's exponent;
    per element: the nearest E4M3 value of v / scale by exhaustive search."""
    rng = np.random.default_rng(21)
    rows = rng.standard_normal((3, 96)) * np.exp2(rng.integers(-20, 12, (3, 1)))
    rows[1, 32:64] *= 1e-6                       # a block far smaller than its row
    rows[2, 64:96] = 0.0                         # an all-zero block
    v32 = rows.astype(np.float32)
    codes, sc = oracle.quant_mxfp8(v32)
    for r in range(3):
        for b in range(3):
            blk = [float(x) for x in v32[r, 32 * b:32 * b + 32]]
            amax = max(abs(x) for x in blk)
            if amax == 0:
                assert sc[r, b] == 0 and (codes[r, 32 * b:32 * b + 32] & 0x7F == 0).all()
                continue
            e = math.frexp(amax)[1] - 1 - 8
            assert sc[r, b] == e + 127
            for k, x in enumerate(blk):
                assert codes[r, 32 * b + k] == _nearest_e4m3_brute(x / 2.0 ** e), (r, b, k)


def test_mxfp8_round_trip_and_saturation():
    rng = np.random.default_rng(22)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    codes = rng.choice(finite, size=(4, 64))
    codes[:, 0] = 0x78                           # 256: the largest element sets the scale
    codes[:, 32] = 0xFD                          # -416
    codes[:, 1:32] &= 0xBF                       # the rest below 256 in magnitude
    codes[:, 33:64] &= 0xBF
    s = rng.integers(100, 140, (4, 2)).astype(np.uint8)
    v = oracle.dequant_mxfp8(codes, s)
    c2, s2 = oracle.quant_mxfp8(v)
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(oracle.dequant_mxfp8(c2, s2), v)
    # a block maximum in (448, 512) x scale saturates to 448 x scale
    w = np.zeros((1, 32))
    w[0, 0], w[0, 1] = 500.0, 100.0
    c3, s3 = oracle.quant_mxfp8(w)
    assert s3[0, 0] == 127 and oracle.dequant_mxfp8(c3, s3)[0, 0] == 448.0


def _w4a8_small(seed, T=12, H=128, E=5, K=2, I=64, I_shared=64):
    inp = random_small(seed, T, H, E, K, I, I_shared, dtype="bf16", w_format="mxfp4")
    c = inp.cfg
    experts = {}
    for e in range(c.E):
        codes, sc = inp.expert_mxfp4(e)
        experts[e] = tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(codes, sc))
    codes, sc = inp.shared_mxfp4()
    shared = tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(codes, sc))
    r = oracle.route(inp.x_f64(), inp.w_router().astype(np.float64), c.K, 0,
                     inp.bias().astype(np.float64), c.scale)
    return inp, experts, shared, r


@pytest.mark.parametrize("seed", [5, 6])
def test_w4a8_layer_eager_equals_dense_masked(seed):
    inp, experts, shared, r = _w4a8_small(seed)
    c = inp.cfg
    x = inp.x_f64()
    got = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared, amx=True)
    ref = oracle.dense_masked(x, r.idx, r.weight, lambda e: experts[e], c.E, shared, amx=True)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(23)
    v = (rng.standard_normal(100_000) * np.exp2(rng.uniform(-30, 30, 100_000))).astype(np.float32)
    v[:4] = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0]   # ties
    ref = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(oracle.round_bf16(v), ref)


def test_w4a8_layer_scalar_loops():
    """One token at a time with element loops: x quantised per 32-block, each
    picked expert's h (rounded to bfloat16 by torch) quantised per 32-block,
    weighted sum."""
    torch = pytest.importorskip("torch")
    inp, experts, shared, r = _w4a8_small(7, T=2, H=64, E=4, K=2, I=64, I_shared=64)
    c = inp.cfg
    x = inp.x_f64()
    got = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared,
                                     amx=True)
    for t in range(c.T):
        xq = list(oracle.quant_dequant_mxfp8(x[t:t + 1])[0])
        ref = [0.0] * c.H
        picks = [(int(r.idx[t, j]), float(r.weight[t, j])) for j in range(c.K)] + [(c.E, 1.0)]
        for e, w in picks:
            wg, wu, wd = experts[e] if e < c.E else shared
            h = []
            for i in range(wg.shape[0]):
                g = math.fsum(xq[k] * wg[i, k] for k in range(c.H))
                u = math.fsum(xq[k] * wu[i, k] for k in range(c.H))
                h.append(g / (1.0 + math.exp(-g)) * u)
            hb = torch.tensor(h, dtype=torch.float32).to(torch.bfloat16).double().numpy()
            hq = list(oracle.quant_dequant_mxfp8(hb[None, :])[0])
            for n in range(c.H):
                ref[n] += w * math.fsum(hq[i] * wd[n, i] for i in range(len(hq)))
        np.testing.assert_allclose(got[t], ref, rtol=1e-12, atol=1e-13)


def test_w4a8_layer_is_within_the_quantisation_error_of_w4a16():
    inp, experts, shared, r = _w4a8_small(8, T=64, H=128, E=6, K=2, I=64, I_shared=64)
    c = inp.cfg
    x = inp.x_f64()
    ref = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared)
    got = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared,
                                     amx=True)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert 0.005 < rel < 0.08, rel


# ------------------------------- per-branch formats (routed W4A8, shared W8A8) ----
def _mixed_small(seed, T=12, H=128, E=5, K=2, I=64, I_shared=64):
    inp = random_small(seed, T, H, E, K, I, I_shared, dtype="bf16", w_format="mxfp4",
                       act_format="mxfp8", shared_w_format="fp8_e4m3",
                       shared_act_format="fp8_static")
    c = inp.cfg
    experts = {}
    for e in range(c.E):
        codes, sc = inp.expert_mxfp4(e)
        experts[e] = tuple(oracle.dequant_mxfp4(q, s) for q, s in zip(codes, sc))
    codes, sc = inp.shared_fp8()
    shared = tuple(oracle.dequant_fp8(q, s) for q, s in zip(codes, sc))
    a1, a2 = inp.act_scales()
    r = oracle.route(inp.x_f64(), inp.w_router().astype(np.float64), c.K, 0,
                     inp.bias().astype(np.float64), c.scale)
    return inp, experts, shared, r, (float(a1), a2.astype(np.float64))


def test_mixed_layer_scalar_loops():
    """One token at a time with element loops: the routed experts read x
    quantised per 32-block and quantise their h (rounded to bfloat16 by
    torch) per 32-block; the shared expert reads x quantised with a1 and
    quantises its h with a2[E]."""
    torch = pytest.importorskip("torch")
    inp, experts, shared, r, (a1, a2) = _mixed_small(9, T=2, H=64, E=4, K=2, I=64,
                                                     I_shared=64)
    c = inp.cfg
    x = inp.x_f64()
    got = oracle.forward_given_route(x, r.idx, r.weight, lambda e: experts[e], c.E, shared,
                                     amx=True, shared_a8=(a1, a2), shared_amx=False)
    for t in range(c.T):
        x_mx = list(oracle.quant_dequant_mxfp8(x[t:t + 1])[0])
        x_8 = [float(oracle.quant_dequant_e4m3(np.array([x[t, k]]), a1)[0]) for k in range(c.H)]
        ref = [0.0] * c.H
        picks = [(int(r.idx[t, j]), float(r.weight[t, j])) for j in range(c.K)] + [(c.E, 1.0)]
        for e, w in picks:
            wg, wu, wd = experts[e] if e < c.E else shared
            xq = x_8 if e == c.E else x_mx
            h = []
            for i in range(wg.shape[0]):
                g = math.fsum(xq[k] * wg[i, k] for k in range(c.H))
                u = math.fsum(xq[k] * wu[i, k] for k in range(c.H))
                h.append(g / (1.0 + math.exp(-g)) * u)
            hb = torch.tensor(h, dtype=torch.float32).to(torch.bfloat16).double().numpy()
            if e == c.E:
                hq = [float(oracle.quant_dequant_e4m3(np.array([v]), a2[e])[0]) for v in hb]
            else:
                hq = list(oracle.quant_dequant_mxfp8(hb[None, :])[0])
            for n in range(c.H):
                ref[n] += w * math.fsum(hq[i] * wd[n, i] for i in range(len(hq)))
        np.testing.assert_allclose(got[t], ref, rtol=1e-12, atol=1e-13)


def test_mixed_layer_is_the_sum_of_its_branches():
    """The routed part in the routed formats plus the shared expert alone in
    its own (no routed picks); and the shared formats given as the routed
    ones reproduce the single-format layer."""
    inp, experts, shared, r, a8 = _mixed_small(10, T=20)
    c = inp.cfg
    x = inp.x_f64()
    ex = lambda e: experts[e]
    got = oracle.forward_given_route(x, r.idx, r.weight, ex, c.E, shared, amx=True,
                                     shared_a8=a8, shared_amx=False)
    routed = oracle.forward_given_route(x, r.idx, r.weight, ex, c.E, None, amx=True)
    alone = oracle.forward_given_route(x, r.idx[:, :0], r.weight[:, :0], ex, c.E, shared, a8=a8)
    np.testing.assert_allclose(got, routed + alone, rtol=1e-12, atol=1e-12)
    # the branches differ: quantising the shared expert as the routed ones moves the output
    as_routed = oracle.forward_given_route(x, r.idx, r.weight, ex, c.E, shared, amx=True)
    assert np.abs(as_routed - got).max() > 1e-3
    same = oracle.forward_given_route(x, r.idx, r.weight, ex, c.E, shared, amx=True,
                                      shared_a8=None, shared_amx=True)
    np.testing.assert_array_equal(same, as_routed)


# ------------------------------------------------- weights on given picks ----
def test_combine_weights_closed_form():
    """Weights of hand-chosen picks: sigmoid mode renormalises the picked
    unbiased scores and scales them; softmax mode divides by the clamped sum."""
    prob = np.array([[0.5, 0.25, 0.75, 0.125]])
    w = oracle.combine_weights(prob, np.array([[2, 0]]), oracle.ROUTE_SIGMOID_BIAS, 2.826)
    np.testing.assert_allclose(w, [[2.826 * 0.6, 2.826 * 0.4]], rtol=0, atol=1e-15)
    w = oracle.combine_weights(prob, np.array([[1, 3]]), oracle.ROUTE_SOFTMAX, 1.0, 1e-8)
    np.testing.assert_allclose(w, [[2 / 3, 1 / 3]], rtol=0, atol=1e-15)
    # the clamp binds when the picked mass is below it
    w = oracle.combine_weights(np.array([[1e-10, 3e-10]]), np.array([[0, 1]]),
                               oracle.ROUTE_SOFTMAX, 1.0, 1e-8)
    np.testing.assert_allclose(w, [[1e-2, 3e-2]], rtol=1e-12)


# ------------------------------------- the expert-by-expert evaluation ----
@pytest.mark.parametrize("seed, mode, fmt", [(0, 0, None), (1, 1, None), (2, 0, "a8"),
                                              (3, 0, "amx"), (4, 0, "noshared"),
                                              (5, 0, "mixed")])
def test_forward_by_expert_equals_dense_masked(seed, mode, fmt):
    """The streamed form against brute-force dense evaluation of every expert
    (the same sum, every expert on every token, masked)."""
    kw = dict(route_mode=1, scale=1.0, renorm_eps=1e-8, bias_kind="none") if mode else {}
    if fmt in ("amx", "mixed"):
        inp = random_small(200 + seed, T=11, H=64, E=6, K=3, I=32, I_shared=32, **kw)
    else:
        inp = random_small(200 + seed, T=13, H=8, E=7, K=3, I=5,
                           I_shared=0 if fmt == "noshared" else 4, **kw)
    c = inp.cfg
    ex = [inp.expert_f64(e) for e in range(c.E)]
    x = inp.x_f64()
    b = inp.bias()
    r = oracle.route(x, inp.w_router().astype(np.float64), c.K, mode,
                     None if b is None else b.astype(np.float64), c.scale, c.renorm_eps)
    sh = None if fmt == "noshared" else inp.shared_f64()
    a8 = (0.01, np.linspace(0.002, 0.004, c.E + 1)) if fmt == "a8" else None
    amx = fmt in ("amx", "mixed")
    # mixed: routed MXFP8, the shared expert static FP8
    fk = dict(shared_a8=(0.01, np.linspace(0.002, 0.004, c.E + 1)),
              shared_amx=False) if fmt == "mixed" else {}
    got = oracle.forward_by_expert(x, r.idx, r.weight, lambda e: ex[e], c.E, sh, a8=a8, amx=amx,
                                   **fk)
    ref = oracle.dense_masked(x, r.idx, r.weight, lambda e: ex[e], c.E, sh, a8=a8, amx=amx, **fk)
    eager = oracle.forward_given_route(x, r.idx, r.weight, lambda e: ex[e], c.E, sh, a8=a8,
                                       amx=amx, **fk)
    np.testing.assert_allclose(eager, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.abs(ref).max() > 0.05


def test_forward_by_expert_requests_each_expert_once():
    inp = random_small(210, T=40, H=8, E=9, K=4, I=5, I_shared=4)
    c = inp.cfg
    ex = [inp.expert_f64(e) for e in range(c.E)]
    r = oracle.route(inp.x_f64(), inp.w_router().astype(np.float64), c.K, 0,
                     inp.bias().astype(np.float64), c.scale)
    asked = []
    oracle.forward_by_expert(inp.x_f64(), r.idx, r.weight,
                             lambda e: asked.append(e) or ex[e], c.E, inp.shared_f64())
    assert sorted(asked) == sorted(set(asked)) == sorted(set(r.idx.reshape(-1).tolist()))
