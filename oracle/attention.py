"""One-shot causal softmax attention in float64 (oracle; test infrastructure).

Source: zdszero "Chunked Prefill" notes, section "prefill as several resumable
extends". The equation for o_i defines the output of the extend token at global
position p = P_t + i as the softmax-weighted sum of v_j over keys j = 0..p
(inclusive), with weights exp(q_i . k_j / sqrt(d)). The same section states that
cutting a prefill into chunks changes only the floating-point summation order,
so the oracle is that definition with no chunking and no paging at all:

    s_j = scale * sum_d q[d] k_j[d]          for j = 0..p
    m   = max_j s_j
    w_j = exp(s_j - m),   l = sum_j w_j
    o   = sum_j w_j v_j / l,   lse = m + ln l

``lse`` is the natural-log log-sum-exp of the scaled scores (the pages name the
(m, l) statistics but define no exported value; this is the plain reading).
The softmax scale is an explicit argument; the pages use 1/sqrt(d).

Grouped-query attention (not on the pages): query head h reads KV head
h // (Hq / Hkv), contiguous groups.

The second half of the file restates the two-stage form of the same section
(stage 1: the whole prefix, unmasked; stage 2: the chunk, causal) and its merge
rule, m = max(m1, m2), o = (e^{m1-m} l1 o1 + e^{m2-m} l2 o2) / (e^{m1-m} l1 +
e^{m2-m} l2). Tests use it to check that the two-stage result equals the
one-shot definition; the GPU parity checks use only the one-shot definition.
"""

from __future__ import annotations

import numpy as np

_ROW_BLOCK = 256


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attend_rows(q_rows, k_ctx, v_ctx, positions, scale: float):
    """Causal attention for arbitrary query rows.

    q_rows:    [R, Hq, D] queries; row r sits at global position ``positions[r]``
    k_ctx:     [n_keys, Hkv, D] keys for global positions 0..n_keys-1
    v_ctx:     [n_keys, Hkv, D] values
    positions: [R] integers, each < n_keys; row r attends keys 0..positions[r]
    Returns ``(o [R, Hq, D], lse [R, Hq])`` in float64.
    """
    q = _as64(q_rows)
    k = _as64(k_ctx)
    v = _as64(v_ctx)
    pos = np.asarray(positions, dtype=np.int64)
    R, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if R and (pos.min() < 0 or pos.max() >= k.shape[0]):
        raise ValueError("positions out of range")
    group = hq // hkv
    o = np.zeros((R, hq, d))
    lse = np.zeros((R, hq))
    order = np.argsort(pos, kind="stable")
    for b0 in range(0, R, _ROW_BLOCK):
        rows = order[b0:b0 + _ROW_BLOCK]
        prow = pos[rows]
        n = int(prow.max()) + 1
        allowed = np.arange(n)[None, :] <= prow[:, None]           # j <= p, inclusive
        for h in range(hq):
            g = h // group
            s = scale * (q[rows, h, :] @ k[:n, g, :].T)               # [rows, n]
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            l = w.sum(axis=1, keepdims=True)
            o[rows, h, :] = (w @ v[:n, g, :]) / l
            lse[rows, h] = (m + np.log(l))[:, 0]
    return o, lse


def causal_attention(q, k, v, scale: float, rows=None):
    """One-shot causal attention over a whole sequence.

    q: [N, Hq, D], k, v: [N, Hkv, D]. Returns output and lse for the query
    positions in ``rows`` (default: all N).
    """
    n = np.asarray(q).shape[0]
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    return attend_rows(np.asarray(q)[rows], k, v, rows, scale)


# ---------------------------------------------------------------------------
# Two-stage form (rectangle + triangle) and the merge rule.
# ---------------------------------------------------------------------------

def _partial(q_row, k_set, v_set, scale: float):
    """Attention of one query head row over a key set: (normalised o, m, l).

    An empty key set gives m = -inf, l = 0 and o = 0 (it then carries no weight
    in the merge).
    """
    if k_set.shape[0] == 0:
        return np.zeros(q_row.shape[-1]), -np.inf, 0.0
    s = scale * (k_set @ q_row)
    m = s.max()
    w = np.exp(s - m)
    l = w.sum()
    return (w @ v_set) / l, m, l


def merge_two(o1, m1, l1, o2, m2, l2):
    """Merge two partial softmax results with their (m, l) statistics."""
    m = max(m1, m2)
    a1 = 0.0 if l1 == 0.0 else np.exp(m1 - m) * l1
    a2 = 0.0 if l2 == 0.0 else np.exp(m2 - m) * l2
    o = (a1 * np.asarray(o1) + a2 * np.asarray(o2)) / (a1 + a2)
    return o, m, a1 + a2


def rectangle_triangle(q_chunk, k_ctx, v_ctx, prefix_len: int, scale: float):
    """Extend attention of a chunk in two stages, merged.

    q_chunk: [E, Hq, D] queries at global positions prefix_len .. prefix_len+E-1.
    Stage 1 attends the whole prefix [0, prefix_len) with no mask; stage 2
    attends the chunk's own keys [prefix_len, prefix_len + i] causally.
    Returns (o [E, Hq, D], lse [E, Hq]).
    """
    q = _as64(q_chunk)
    k = _as64(k_ctx)
    v = _as64(v_ctx)
    e, hq, d = q.shape
    group = hq // k.shape[1]
    o = np.zeros((e, hq, d))
    lse = np.zeros((e, hq))
    for i in range(e):
        for h in range(hq):
            g = h // group
            o1, m1, l1 = _partial(q[i, h], k[:prefix_len, g], v[:prefix_len, g], scale)
            o2, m2, l2 = _partial(q[i, h], k[prefix_len:prefix_len + i + 1, g],
                                  v[prefix_len:prefix_len + i + 1, g], scale)
            oo, m, l = merge_two(o1, m1, l1, o2, m2, l2)
            o[i, h] = oo
            lse[i, h] = m + np.log(l)
    return o, lse


def lse_merge(parts):
    """Merge any number of normalised partials given as ``(o, lse)`` pairs.

    Each partial's (m, l) pair is represented by lse = m + ln l; the merged
    weight of part s is exp(lse_s - lse) with lse = ln sum_s exp(lse_s).
    """
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    top = lses.max(axis=0)
    w = np.exp(lses - top)
    total = w.sum(axis=0)
    o = sum(wi[..., None] * _as64(p[0]) for wi, p in zip(w, parts)) / total[..., None]
    return o, top + np.log(total)
