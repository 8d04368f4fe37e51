"""Pins for the oracle's attention (CPU only).

What fixes the values (zdszero "Chunked Prefill" notes, section "prefill as
several resumable extends"): the equation for o_i (softmax over keys 0..P_t+i,
inclusive), the statement that chunking changes only floating-point order, and
the two-stage merge rule. Pins, each able to catch a different plausible slip:
* brute-force scalar loops in pure Python (index or mask off-by-one, dropped scale);
* torch's scaled_dot_product_attention in float64 on the CPU with an explicit
  boolean mask (transposed operand, wrong softmax axis);
* closed-form special cases: q = 0 gives the mean of v and lse = ln(p+1); row 0
  gives v_0 and lse = scale q.k_0 (mask excludes the diagonal, wrong log base);
* shifting every key by one vector u shifts every score of a row by the same
  amount: o is unchanged and lse moves by scale q.u;
* the two-stage rectangle + triangle form, merged, equals one-shot (the page's
  identity), including an empty rectangle;
* GQA: replicating each KV head over its query-head group and running plain
  multi-head attention gives the same result (head mapping);
* the LSE merge of key-range partials equals the whole, in any grouping.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attend_rows, causal_attention, lse_merge, merge_two, rectangle_triangle
from oracle.attention import _partial


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def _brute(q, k, v, scale):
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    o = np.zeros((n, hq, d))
    lse = np.zeros((n, hq))
    for p in range(n):
        for h in range(hq):
            kh = h // g
            s = [scale * sum(q[p, h, t] * k[j, kh, t] for t in range(d)) for j in range(p + 1)]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            l = sum(w)
            for t in range(d):
                o[p, h, t] = sum(w[j] * v[j, kh, t] for j in range(p + 1)) / l
            lse[p, h] = m + math.log(l)
    return o, lse


@pytest.mark.parametrize("n,hq,hkv,d", [(9, 2, 1, 4), (12, 4, 2, 3), (7, 3, 3, 5)])
def test_brute_force(n, hq, hkv, d):
    q, k, v = _rand((n, hq, d), 1), _rand((n, hkv, d), 2), _rand((n, hkv, d), 3)
    scale = 1.0 / math.sqrt(d)
    o, lse = causal_attention(q, k, v, scale)
    ob, lb = _brute(q, k, v, scale)
    assert np.abs(o - ob).max() < 1e-12
    assert np.abs(lse - lb).max() < 1e-12


def test_brute_force_block_boundary():
    # more rows than the oracle's internal row block, so the block loop is exercised
    n, hq, hkv, d = 300, 1, 1, 2
    q, k, v = _rand((n, hq, d), 4), _rand((n, hkv, d), 5), _rand((n, hkv, d), 6)
    rows = np.array([0, 1, 255, 256, 257, 299])
    o, lse = causal_attention(q, k, v, 0.7, rows=rows)
    ob, lb = _brute(q[:300], k, v, 0.7)
    assert np.abs(o - ob[rows]).max() < 1e-12 and np.abs(lse - lb[rows]).max() < 1e-12


def test_matches_torch_sdpa_float64():
    n, hq, hkv, d = 70, 8, 2, 16
    q, k, v = _rand((n, hq, d), 7), _rand((n, hkv, d), 8), _rand((n, hkv, d), 9)
    scale = 0.3
    # a chunk of rows [40, 70) over keys [0, 70): explicit bottom-right mask
    rows = np.arange(40, 70)
    o, _ = causal_attention(q, k, v, scale, rows=rows)
    g = hq // hkv
    kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2)   # [hq, n, d]
    vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2)
    qt = torch.from_numpy(q[rows]).permute(1, 0, 2)
    mask = torch.from_numpy(np.arange(n)[None, :] <= rows[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    assert np.abs(o - ref.permute(1, 0, 2).numpy()).max() < 1e-12


def test_special_cases():
    n, d = 20, 6
    k, v = _rand((n, 1, d), 10), _rand((n, 1, d), 11)
    q0 = np.zeros((n, 1, d))
    o, lse = causal_attention(q0, k, v, 0.5)
    for p in range(n):
        assert np.allclose(o[p, 0], v[:p + 1, 0].mean(axis=0), atol=1e-13, rtol=0)
        assert abs(lse[p, 0] - math.log(p + 1)) < 1e-13
    q = _rand((n, 1, d), 12)
    o, lse = causal_attention(q, k, v, 0.5)
    assert np.abs(o[0, 0] - v[0, 0]).max() == 0.0
    assert abs(lse[0, 0] - 0.5 * float(q[0, 0] @ k[0, 0])) < 1e-13
    # identical keys: uniform weights whatever q is
    kk = np.repeat(k[:1], n, axis=0)
    o, lse = causal_attention(q, kk, v, 0.5)
    for p in (0, 5, 19):
        assert np.allclose(o[p, 0], v[:p + 1, 0].mean(axis=0), atol=1e-13, rtol=0)
        assert abs(lse[p, 0] - (0.5 * float(q[p, 0] @ k[0, 0]) + math.log(p + 1))) < 1e-12


def test_key_shift_invariance():
    n, hq, hkv, d = 33, 4, 2, 8
    q, k, v = _rand((n, hq, d), 13), _rand((n, hkv, d), 14), _rand((n, hkv, d), 15)
    u = _rand((1, hkv, d), 16) * 3.0
    o1, l1 = causal_attention(q, k, v, 0.25)
    o2, l2 = causal_attention(q, k + u, v, 0.25)
    g = hq // hkv
    shift = np.stack([0.25 * (q[:, h] @ u[0, h // g]) for h in range(hq)], axis=1)
    assert np.abs(o1 - o2).max() < 1e-12
    assert np.abs((l2 - l1) - shift).max() < 1e-11


@pytest.mark.parametrize("prefix,e", [(0, 7), (5, 1), (13, 6), (16, 16)])
def test_rectangle_triangle_equals_one_shot(prefix, e):
    hq, hkv, d = 4, 2, 8
    n = prefix + e
    q, k, v = _rand((n, hq, d), 17), _rand((n, hkv, d), 18), _rand((n, hkv, d), 19)
    o, lse = rectangle_triangle(q[prefix:], k, v, prefix, 0.35)
    o1, l1 = causal_attention(q, k, v, 0.35, rows=np.arange(prefix, n))
    assert np.abs(o - o1).max() < 1e-12
    assert np.abs(lse - l1).max() < 1e-12


def test_gqa_equals_replicated_mha():
    n, hq, hkv, d = 25, 8, 2, 4
    q, k, v = _rand((n, hq, d), 20), _rand((n, hkv, d), 21), _rand((n, hkv, d), 22)
    o, lse = causal_attention(q, k, v, 0.5)
    g = hq // hkv
    o2, lse2 = causal_attention(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), 0.5)
    assert np.abs(o - o2).max() == 0.0 and np.abs(lse - lse2).max() == 0.0


def test_lse_merge_of_key_ranges():
    d = 10
    q = _rand((d,), 23)
    k, v = _rand((40, d), 24), _rand((40, d), 25)
    whole, mw, lw = _partial(q, k, v, 0.4)
    cuts = [(0, 3), (3, 21), (21, 40)]
    parts = []
    for a, b in cuts:
        o, m, l = _partial(q, k[a:b], v[a:b], 0.4)
        parts.append((o, m + math.log(l)))
    o, lse = lse_merge(parts)
    assert np.abs(o - whole).max() < 1e-12 and abs(lse - (mw + math.log(lw))) < 1e-12
    # pairwise merge in two different groupings
    (o0, m0, l0), (o1, m1, l1), (o2, m2, l2) = [_partial(q, k[a:b], v[a:b], 0.4) for a, b in cuts]
    left = merge_two(*merge_two(o0, m0, l0, o1, m1, l1), o2, m2, l2)
    inner = merge_two(o1, m1, l1, o2, m2, l2)
    right = merge_two(o0, m0, l0, *inner)
    assert np.abs(left[0] - right[0]).max() < 1e-12
    lse_left = left[1] + math.log(left[2])
    assert abs(lse_left - np.logaddexp(m0 + math.log(l0), inner[1] + math.log(inner[2]))) < 1e-12
    assert abs(lse_left - (mw + math.log(lw))) < 1e-12


def test_decode_row_is_last_row_of_one_shot():
    n, hq, hkv, d = 50, 4, 1, 8
    q, k, v = _rand((n, hq, d), 26), _rand((n, hkv, d), 27), _rand((n, hkv, d), 28)
    o, lse = causal_attention(q, k, v, 0.3)
    od, ld = attend_rows(q[n - 1:], k, v, [n - 1], 0.3)
    assert np.abs(od[0] - o[-1]).max() < 1e-14 and np.abs(ld[0] - lse[-1]).max() < 1e-14
