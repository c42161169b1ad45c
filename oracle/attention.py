"""Oracle for split-KV decode attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module; the product path never imports it.

What it follows: the Hy3 Preview inference case study, section "1.
Attention dynamic scheduling": every request's attention work is cut into
tiles of one size, the tiles are shared out over the workgroups by the
global tile count with a greedy fill, a task map is built before each
inference, the attention kernels take their tasks from it, and a combine
step merges the split-KV partial results.  The attention itself is the
model's GQA decode attention (CANN deployment article, section 一: 64 query
heads over 8 KV heads, head_dim 128): query head j of a request attends
with KV head j // (query heads per KV head) over that request's cached keys
and values,

    o = softmax(q K^T / sqrt(d)) V

computed here in float64 straight from the definition.  Readings where the
pages leave a step open (tile size, the fill rule, empty requests) are the
plainest ones and are listed with the design notes: the fill walks the
(request, KV head) rows in order and gives each worker consecutive tiles up
to ceil(total tiles / workers), so a worker's share of a row is one
contiguous range (a split); a request with no cached tokens yields zeros.
"""
from __future__ import annotations

import dataclasses
from typing import List, Sequence

import numpy as np


def attention_decode(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     kv_len: Sequence[int], scale: float) -> np.ndarray:
    """q [B][Hq][d]; k, v [Hkv][sum L][d] (request b's tokens at rows
    sum(L[:b]) .. +L[b] of every KV head); returns o [B][Hq][d] float64.
    softmax(scale q k^T) v per (request, query head); zeros when L[b] == 0."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[0]
    grp = Hq // Hkv
    out = np.zeros((B, Hq, d))
    start = 0
    for b, L in enumerate(kv_len):
        L = int(L)
        for j in range(Hq):
            if L == 0:
                continue
            kh = k[j // grp, start:start + L]
            vh = v[j // grp, start:start + L]
            s = scale * (kh @ q[b, j])
            p = np.exp(s - s.max())
            out[b, j] = (p / p.sum()) @ vh
        start += L
    return out


@dataclasses.dataclass
class Plan:
    """Task map.  tasks[i] = (request, kv head, first tile, end tile) of task
    i, in creation order; worker w runs tasks worker_begin[w] ..
    worker_begin[w+1]-1; row r = request * Hkv + kv head owns tasks
    row_begin[r] .. row_begin[r+1]-1 (its splits, in K order)."""
    tasks: np.ndarray          # [n_tasks][4] int
    worker_begin: np.ndarray   # [n_workers + 1]
    row_begin: np.ndarray      # [B * Hkv + 1]
    cap: int                   # tiles per worker


def plan_split_kv(kv_len: Sequence[int], n_kv_heads: int, tile: int, n_workers: int) -> Plan:
    """Greedy fill by the global tile count: row (b, h) has ceil(L[b] / tile)
    tiles; every worker takes consecutive tiles, rows in order, until it
    holds cap = ceil(total / n_workers) of them, then the next worker starts.
    A row split across workers gives one task per worker."""
    n_tiles = [-(-int(L) // tile) for L in kv_len]
    rows = [(b, h) for b in range(len(kv_len)) for h in range(n_kv_heads)]
    total = sum(n_tiles[b] for b, _ in rows)
    cap = max(1, -(-total // n_workers))
    tasks: List[tuple] = []
    worker_begin = [0]
    row_begin = []
    used = 0
    for b, h in rows:
        row_begin.append(len(tasks))
        t = 0
        while t < n_tiles[b]:
            take = min(cap - used, n_tiles[b] - t)
            tasks.append((b, h, t, t + take))
            t += take
            used += take
            if used == cap:
                worker_begin.append(len(tasks))
                used = 0
    row_begin.append(len(tasks))
    if used:
        worker_begin.append(len(tasks))
    while len(worker_begin) < n_workers + 1:
        worker_begin.append(len(tasks))
    return Plan(np.array(tasks, dtype=np.int64).reshape(-1, 4),
                np.array(worker_begin, dtype=np.int64),
                np.array(row_begin, dtype=np.int64), cap)


def partial_attention(q: np.ndarray, kh: np.ndarray, vh: np.ndarray, scale: float):
    """One split: over keys kh / values vh [n][d] (n >= 1) for query rows q
    [g][d]: (m, l, o) with m = max score, l = sum exp(s - m), o = sum
    exp(s - m) v / l, per query row, float64."""
    s = scale * (np.asarray(kh, np.float64) @ np.asarray(q, np.float64).T)   # [n][g]
    m = s.max(axis=0)
    p = np.exp(s - m)
    l = p.sum(axis=0)
    o = (p.T @ np.asarray(vh, np.float64)) / l[:, None]
    return m, l, o


def combine_splits(parts) -> np.ndarray:
    """Merge split results (m_i, l_i, o_i) of one row: with M = max m_i,
    o = sum_i l_i e^(m_i - M) o_i / sum_i l_i e^(m_i - M)."""
    M = np.max([m for m, _, _ in parts], axis=0)
    w = [l * np.exp(m - M) for m, l, _ in parts]
    num = sum(wi[:, None] * o for wi, (_, _, o) in zip(w, parts))
    return num / sum(w)[:, None]
