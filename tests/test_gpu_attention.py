"""Split-KV decode attention on the GPU against the float64 oracle
(oracle/attention.py): ragged batches that exercise empty requests, tails
and splits, the Hy3 shape (64 query / 8 KV heads, head_dim 128) on a mixed
batch and on one 128K-token request, and bitwise determinism.

Tolerance (derived): the inputs are bf16 values, scores, softmax and the
accumulation run in float32, and the output is rounded once to bf16 (half
an ulp: 2^-9 relative), so every element must satisfy |got - ref| <=
2^-8 |ref| + 1e-5 max|ref| and the relative L2 error must stay below 2^-8."""
import numpy as np
import pytest
import torch

import sparse_moe_amd as sm
from gpu_util import log
from oracle.attention import attention_decode
from synth.attention_inputs import attention_inputs, bits_to_f64, mixed_lengths

pytestmark = pytest.mark.gpu
SCALE = 1.0 / np.sqrt(128.0)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sm.load()
    return torch.device("cuda:0")


def bf16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def run(seed, kv_len, hkv, tile, workers, dev):
    qb, kb, vb = attention_inputs(seed, kv_len, hkv)
    plan = sm.attn_plan(kv_len, hkv, tile, workers)
    log(f"  B={len(kv_len)} sum L={sum(kv_len)} Hkv={hkv} tile={tile} workers={workers} "
        f"tasks={plan.tasks.shape[0]}")
    out = sm.attn_decode(bf16(qb, dev), bf16(kb, dev), bf16(vb, dev), kv_len, plan)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    return got, (qb, kb, vb)


def check(got, inputs, kv_len, what):
    qb, kb, vb = inputs
    ref = attention_decode(bits_to_f64(qb), bits_to_f64(kb), bits_to_f64(vb), kv_len, SCALE)
    top = float(np.abs(ref).max()) if ref.size else 0.0
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * top
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"  {what}: max_abs={err.max():.3e} rel_l2={rel:.3e} max|ref|={top:.3g}")
    bad = np.argwhere(err > bound)
    for i in bad[:3]:
        log(f"    {tuple(i)}: got {got[tuple(i)]:.6g} ref {ref[tuple(i)]:.6g}")
    assert bad.size == 0
    assert rel <= 2.0 ** -8
    return ref


@pytest.mark.parametrize("tile, workers", [(256, 7), (64, 13), (256, 512), (1000, 3)])
def test_ragged_batch(dev, tile, workers):
    kv_len = [0, 1, 63, 64, 65, 255, 256, 257, 1000, 3001]
    got, inp = run(1, kv_len, 2, tile, workers, dev)
    ref = check(got, inp, kv_len, f"ragged tile={tile} workers={workers}")
    np.testing.assert_array_equal(got[0], 0.0)   # no cached tokens
    assert np.isfinite(got).all() and ref.shape == got.shape


def test_hy3_mixed_batch(dev):
    kv_len = mixed_lengths(2, 8, 512, 32768)
    got, inp = run(2, kv_len, 8, 256, 512, dev)
    check(got, inp, kv_len, f"hy3 mixed {kv_len}")


def test_hy3_single_long_request(dev):
    kv_len = [131072]
    got, inp = run(3, kv_len, 8, 256, 512, dev)
    check(got, inp, kv_len, "hy3 single 128K")


def test_deterministic_bitwise(dev):
    kv_len = [5000, 17, 40000]
    a, _ = run(4, kv_len, 8, 256, 512, dev)
    b, _ = run(4, kv_len, 8, 256, 512, dev)
    np.testing.assert_array_equal(a, b)


def test_plan_for_longer_lengths_covers_the_cached_tokens(dev):
    """A plan made for lengths [1000, 500] run on caches of [300, 500]
    tokens: tasks past request 0's 300 tokens are empty splits (no loads),
    and the outputs are the attention over the cached tokens."""
    kv_len = [300, 500]
    qb, kb, vb = attention_inputs(6, kv_len, 8)
    plan = sm.attn_plan([1000, 500], 8, 256, 9)
    out = sm.attn_decode(bf16(qb, dev), bf16(kb, dev), bf16(vb, dev), kv_len, plan)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    check(got, (qb, kb, vb), kv_len, "plan for longer lengths")
