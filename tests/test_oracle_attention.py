"""Pins of the split-KV attention oracle against closed forms, a worked
planning example and identities of the softmax merge (CPU only)."""
import numpy as np
import pytest

from oracle.attention import (attention_decode, combine_splits, partial_attention,
                              plan_split_kv)

SCALE = 1.0 / np.sqrt(128.0)


def rand_case(rng, kv_len, Hq=16, Hkv=2, d=128):
    q = rng.standard_normal((len(kv_len), Hq, d))
    k = rng.standard_normal((Hkv, sum(kv_len), d))
    v = rng.standard_normal((Hkv, sum(kv_len), d))
    return q, k, v


def test_zero_query_gives_mean_of_values():
    """q = 0: all scores equal, so o is the plain mean of the request's V."""
    rng = np.random.default_rng(1)
    kv_len = [5, 17, 1]
    q, k, v = rand_case(rng, kv_len)
    q[:] = 0.0
    o = attention_decode(q, k, v, kv_len, SCALE)
    starts = np.cumsum([0] + kv_len)
    for b in range(3):
        for j in range(16):
            np.testing.assert_allclose(o[b, j], v[j // 8, starts[b]:starts[b + 1]].mean(0),
                                       rtol=0, atol=1e-13)


def test_single_token_returns_its_value_and_empty_gives_zero():
    rng = np.random.default_rng(2)
    kv_len = [1, 0, 1]
    q, k, v = rand_case(rng, kv_len)
    o = attention_decode(q, k, v, kv_len, SCALE)
    np.testing.assert_array_equal(o[1], 0.0)
    for j in range(16):
        np.testing.assert_allclose(o[0, j], v[j // 8, 0], atol=1e-15)
        np.testing.assert_allclose(o[2, j], v[j // 8, 1], atol=1e-15)


def test_two_keys_closed_form_with_large_scores():
    """Scores 1000 and 1000 - ln 3 (exp overflows without the max shift):
    weights 3/4 and 1/4."""
    d = 128
    q = np.zeros((1, 8, d)); q[0, :, 0] = 1.0
    k = np.zeros((1, 2, d))
    k[0, 0, 0] = 1000.0 / SCALE
    k[0, 1, 0] = (1000.0 - np.log(3.0)) / SCALE
    v = np.zeros((1, 2, d)); v[0, 0, 1] = 1.0; v[0, 1, 2] = 1.0
    o = attention_decode(q, k, v, [2], SCALE)
    assert np.isfinite(o).all()
    np.testing.assert_allclose(o[0, :, 1], 0.75, atol=1e-12)
    np.testing.assert_allclose(o[0, :, 2], 0.25, atol=1e-12)


def test_query_head_uses_its_group_kv_head():
    """Changing KV head 1's values changes exactly query heads 8..15."""
    rng = np.random.default_rng(3)
    kv_len = [9, 4]
    q, k, v = rand_case(rng, kv_len)
    o1 = attention_decode(q, k, v, kv_len, SCALE)
    v2 = v.copy(); v2[1] += 1.0
    o2 = attention_decode(q, k, v2, kv_len, SCALE)
    np.testing.assert_array_equal(o1[:, :8], o2[:, :8])
    np.testing.assert_allclose(o2[:, 8:] - o1[:, 8:], 1.0, atol=1e-12)   # rows of p sum to 1


def test_plan_worked_example():
    """L = [300, 700], 2 KV heads, tile 256, 3 workers: rows have 2, 2, 3, 3
    tiles (10), cap 4; worker 0 takes rows 0 and 1, worker 1 row 2 and the
    first tile of row 3, worker 2 the rest of row 3."""
    p = plan_split_kv([300, 700], 2, 256, 3)
    assert p.cap == 4
    assert p.tasks.tolist() == [[0, 0, 0, 2], [0, 1, 0, 2], [1, 0, 0, 3], [1, 1, 0, 1],
                                [1, 1, 1, 3]]
    assert p.worker_begin.tolist() == [0, 2, 4, 5]
    assert p.row_begin.tolist() == [0, 1, 2, 3, 5]


@pytest.mark.parametrize("kv_len, hkv, tile, workers", [
    ([131072], 8, 256, 512), ([0, 1, 255, 256, 257, 5000], 8, 256, 7),
    ([7] * 40, 8, 256, 512), ([100000, 3, 40000, 0, 9999], 8, 128, 300)])
def test_plan_properties(kv_len, hkv, tile, workers):
    """Every tile of every row exactly once; each worker holds cap tiles
    except the last one used; a row's tasks are consecutive and cover its
    tiles in order; at most workers + rows tasks."""
    p = plan_split_kv(kv_len, hkv, tile, workers)
    rows = len(kv_len) * hkv
    n_t = [-(-L // tile) for L in kv_len]
    total = hkv * sum(n_t)
    assert p.cap == max(1, -(-total // workers))
    seen = {}
    for b, h, t0, t1 in p.tasks.tolist():
        assert 0 <= t0 < t1 <= n_t[b]
        for t in range(t0, t1):
            assert (b, h, t) not in seen
            seen[(b, h, t)] = 1
    assert len(seen) == total
    loads = [int((p.tasks[p.worker_begin[w]:p.worker_begin[w + 1], 3] -
                  p.tasks[p.worker_begin[w]:p.worker_begin[w + 1], 2]).sum())
             for w in range(workers)]
    used = [x for x in loads if x]
    assert all(x == p.cap for x in used[:-1]) and 0 < used[-1] <= p.cap if used else total == 0
    assert len(p.row_begin) == rows + 1
    for r in range(rows):
        tt = p.tasks[p.row_begin[r]:p.row_begin[r + 1]]
        b, h = divmod(r, hkv)
        assert (tt[:, 0] == b).all() and (tt[:, 1] == h).all()
        if len(tt):
            assert tt[0, 2] == 0 and tt[-1, 3] == n_t[b]
            assert (tt[1:, 2] == tt[:-1, 3]).all()
    assert len(p.tasks) <= workers + rows


def test_merging_splits_equals_attention():
    """Cutting a row's keys at arbitrary points and merging the partial
    results reproduces the unsplit attention (the softmax merge identity)."""
    rng = np.random.default_rng(4)
    L = 1000
    q, k, v = rand_case(rng, [L], Hq=8, Hkv=1)
    ref = attention_decode(q, k, v, [L], SCALE)[0]
    for cuts in ([0, 1000], [0, 256, 512, 768, 1000], [0, 1, 2, 999, 1000], [0, 333, 1000]):
        parts = [partial_attention(q[0], k[0, a:b], v[0, a:b], SCALE)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        np.testing.assert_allclose(combine_splits(parts), ref, rtol=0, atol=1e-12)


def test_merge_of_two_single_keys_closed_form():
    """Two one-key splits with scores a, b: weights e^a / (e^a + e^b)."""
    d = 4
    q = np.array([[1.0, 0, 0, 0]])
    ka, kb = np.array([[2.0, 0, 0, 0]]), np.array([[-1.0, 0, 0, 0]])
    va, vb = np.array([[1.0, 0, 0, 0]]), np.array([[0, 1.0, 0, 0]])
    o = combine_splits([partial_attention(q, ka, va, 1.0), partial_attention(q, kb, vb, 1.0)])
    wa = np.exp(2.0) / (np.exp(2.0) + np.exp(-1.0))
    np.testing.assert_allclose(o[0], [wa, 1 - wa, 0, 0], atol=1e-15)
