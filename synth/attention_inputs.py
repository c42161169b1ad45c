"""Seeded synthetic inputs for split-KV decode attention (generation only).

Hy3 attention shape (CANN deployment article, section 一): 64 query heads
over 8 KV heads, head_dim 128.  q, k and v are bf16 N(0, 1) values; the
cached lengths either come from a stated list or, for a mixed batch, are
drawn log-uniformly between two bounds.  Cache layout: [KV head][token][128]
with request b's tokens after those of requests 0 .. b-1.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from .inputs import bf16_bits_to_f32, f32_to_bf16_bits

HY3_Q_HEADS, HY3_KV_HEADS, HEAD_DIM = 64, 8, 128


def mixed_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    rng = np.random.default_rng(np.random.SeedSequence([seed, 77]))
    return [int(x) for x in np.exp(rng.uniform(np.log(lo), np.log(hi), n)).astype(np.int64)]


def attention_inputs(seed: int, kv_len: Sequence[int], n_kv_heads: int = HY3_KV_HEADS,
                     group: int = 8, d: int = HEAD_DIM):
    """(q bits [B][Hq][d], k bits [Hkv][sum L][d], v bits) as uint16 bf16 bits."""
    B, total = len(kv_len), int(sum(kv_len))
    out = []
    for tid, shape in enumerate(((B, group * n_kv_heads, d), (n_kv_heads, total, d),
                                 (n_kv_heads, total, d))):
        rng = np.random.default_rng(np.random.SeedSequence([seed, 78, tid]))
        out.append(f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32)))
    return tuple(out)


def bits_to_f64(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(a).astype(np.float64)
