"""Planted mistakes in copies of the oracle's steps must be caught by the pins.

Each mutant below is a plausible error (biased weights, swapped gate/up,
transposed down, dropped shared branch, wrong tie order, weights not
renormalised, softmax without the max-shift being replaced by a wrong axis).
The same hand-worked fixtures that pin the oracle must reject every mutant.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import moe as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _route_biased_weights(L, K, bias, scale):
    s = om.sigmoid(L)
    b = s + bias
    idx = om.topk_desc(b, K)
    picked = b[np.arange(L.shape[0])[:, None], idx]
    return idx, scale * picked / picked.sum(1, keepdims=True)


def _route_no_renorm(L, K, bias, scale):
    s = om.sigmoid(L)
    idx = om.topk_desc(s + bias, K)
    return idx, scale * s[np.arange(L.shape[0])[:, None], idx]


def _route_unbiased_select(L, K, bias, scale):
    s = om.sigmoid(L)
    idx = om.topk_desc(s, K)
    picked = s[np.arange(L.shape[0])[:, None], idx]
    return idx, scale * picked / picked.sum(1, keepdims=True)


def _route_bias_on_logit(L, K, bias, scale):
    s = om.sigmoid(L)
    idx = om.topk_desc(om.sigmoid(L + bias), K)
    picked = s[np.arange(L.shape[0])[:, None], idx]
    return idx, scale * picked / picked.sum(1, keepdims=True)


@pytest.mark.parametrize("mutant", [_route_biased_weights, _route_no_renorm,
                                    _route_unbiased_select, _route_bias_on_logit])
def test_route_mutants_fail_golden(mutant):
    c = load("route_sigmoid_bias_hand.json")
    idx, w = mutant(np.array(c["logits"]), c["K"], np.array(c["bias"]), c["scale"])
    same = idx.tolist() == c["idx"] and np.allclose(w, c["weight"], atol=1e-9)
    assert not same


def _topk_ties_to_higher_index(score, k):
    E = score.shape[1]
    rev = np.argsort(-score[:, ::-1], axis=1, kind="stable")   # stable on reversed order
    return (E - 1 - rev)[:, :k]


def test_tie_order_mutant_fails_golden():
    c = load("route_sigmoid_ties_hand.json")
    L = np.array(c["logits"])
    for K in ("2", "3"):
        idx = _topk_ties_to_higher_index(om.sigmoid(L), int(K))
        assert idx.tolist() != c["by_K"][K]["idx"]


def _swiglu_swapped(a, wg, wu, wd):
    return om.swiglu_expert(a, wu, wg, wd)


def _swiglu_transposed_down(a, wg, wu, wd):
    return om.swiglu_expert(a, wg, wu, np.asarray(wd).T)


def _swiglu_transposed_gate(a, wg, wu, wd):
    return om.swiglu_expert(a, np.asarray(wg).T, wu, wd)


def _swiglu_plain_sigmoid(a, wg, wu, wd):
    g = a @ np.asarray(wg).T
    u = a @ np.asarray(wu).T
    return (om.sigmoid(g) * u) @ np.asarray(wd).T


@pytest.mark.parametrize("mutant", [_swiglu_swapped, _swiglu_transposed_down,
                                    _swiglu_transposed_gate, _swiglu_plain_sigmoid])
def test_swiglu_mutants_fail_golden(mutant):
    c = load("swiglu_hand.json")
    out = mutant(np.array(c["a"]), np.array(c["w_gate"]), np.array(c["w_up"]),
                 np.array(c["w_down"]))
    assert not np.allclose(out, c["out"], atol=1e-6)


def test_dropped_shared_branch_fails_golden():
    c = load("layer_hand.json")
    ex = [(np.array(d["gate"]), np.array(d["up"]), np.array(d["down"])) for d in c["experts"]]
    out, _ = oracle.forward(np.array(c["x"]), np.array(c["w_router"]), lambda e: ex[e], 3,
                            c["K"], None, oracle.ROUTE_SIGMOID_BIAS, np.array(c["bias"]),
                            c["scale"])
    assert not np.allclose(out, c["out"], atol=1e-6)


def test_scaled_shared_branch_fails_golden():
    c = load("layer_hand.json")
    ex = [(np.array(d["gate"]), np.array(d["up"]), np.array(d["down"])) for d in c["experts"]]
    sh = tuple(np.array(c["shared"][k]) for k in ("gate", "up", "down"))
    sh_scaled = (sh[0], sh[1], sh[2] * 2.826)
    out, _ = oracle.forward(np.array(c["x"]), np.array(c["w_router"]), lambda e: ex[e], 3,
                            c["K"], sh_scaled, oracle.ROUTE_SIGMOID_BIAS, np.array(c["bias"]),
                            c["scale"])
    assert not np.allclose(out, c["out"], atol=1e-6)


def test_softmax_wrong_axis_fails_golden():
    c = load("route_softmax_hand.json")
    L = np.array(c["logits"] * 2)            # two identical tokens
    z = L - L.max(axis=0, keepdims=True)
    p = np.exp(z) / np.exp(z).sum(axis=0, keepdims=True)      # normalised over tokens
    idx = om.topk_desc(p, 2)
    w = p[np.arange(2)[:, None], idx]
    w = w / w.sum(1, keepdims=True)
    e = c["by_K"]["2"]
    assert not (idx[:1].tolist() == e["idx"] and np.allclose(w[:1], e["weight"]))
