"""Chunk tiles whose scores climb steeply along the keys (needs a gfx950 GPU).

The chunk kernel fixes its running max m at the first tile's exact row max and
lets later weights grow; a wave whose tile weights pass 2^64 against it redoes
its rows on an exact two-pass path (row max first, then the weights). Here the
keys carry a common offset that grows every 32 keys, so each tile's scores sit
about 12 (log2 units) above the tile before, some 190 to 360 above the first
tile in all: waves must take that path, and the status words count them. Both
outputs are compared with the exact fp64 oracle: ``out`` at the bf16 bar (max
2e-2, mean 2e-3) and ``lse`` at 1e-3 plus the fp32 spacing of lse itself
(1e-6 |lse|), since lse is the log-sum-exp of the scores the inputs define,
whatever their size.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_attention_extend_amd as ext
import oracle
from synth import custom_workload
from synth.workloads import round_to_bf16
from tests.harness import PagedCache, log

pytestmark = pytest.mark.gpu

D, HQ, HKV = 128, 8, 2
STEP = 1.47  # key offset added per 32 keys: about +12 in the scores (log2 units) per tile


def _inputs(seed: int, n: int):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, HQ, D)).astype(np.float32) * 0.5 + 0.5
    k = rng.standard_normal((n, HKV, D)).astype(np.float32) * 0.5
    k += (STEP * (np.arange(n) // 32)).astype(np.float32)[:, None, None]
    v = rng.standard_normal((n, HKV, D)).astype(np.float32) * 0.5
    return round_to_bf16(q)[0], round_to_bf16(k)[0], round_to_bf16(v)[0]


@pytest.mark.parametrize("prefix,extend,decode", [(0, 512, False), (960, 96, False), (960, 96, True)])
def test_rising_scores_take_the_exact_path(prefix, extend, decode):
    """decode=True adds a decode row (ordinary scores) to the launch, so the chunk rows
    run in the mixed kernel instead of the chunk-only one."""
    n = prefix + extend
    launches = [(prefix, extend)] + ([(300, 1)] if decode else [])
    w = custom_workload(900 + prefix, launches, HQ, HKV, D)
    q, k, v = _inputs(31 + prefix, n)
    log(f"rising scores: P={prefix}, E={extend}, {HQ}/{HKV} heads, D={D}, decode row: {decode}")
    cache = PagedCache(w)
    cache.expect_fast = False
    cache.append([0], [0], k, v, [n])
    q_all = q[prefix:]
    if decode:
        r = w.requests[1]
        cache.append([1], [0], w.k(r, 0, 301), w.v(r, 0, 301), [301])
        q_all = np.concatenate([q_all, w.q(r, 300, 301)])
    out, lse = cache.attend(list(range(len(launches))), [p for p, _ in launches], [e for _, e in launches], q_all)
    torch.cuda.synchronize()
    exact = ext.last_status()[2]
    log(f"  waves on the exact path: {exact}")
    assert exact > 0, "rising scores must push waves past the fast loop's bound"
    pos = np.arange(prefix, n)
    o_ref, lse_ref = oracle.attend_rows(q[prefix:], k, v, pos, w.scale)
    if decode:
        r = w.requests[1]
        o_d, l_d = oracle.attend_rows(w.q(r, 300, 301), w.k(r, 0, 301), w.v(r, 0, 301), np.array([300]), w.scale)
        o_ref, lse_ref = np.concatenate([o_ref, o_d]), np.concatenate([lse_ref, l_d])
    o = out.float().cpu().numpy().astype(np.float64)
    ls = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(ls).all()
    err = np.abs(o - o_ref)
    log(f"  out: max {err.max():.3e} mean {err.mean():.3e}; lse max {np.abs(ls - lse_ref).max():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    lerr = np.abs(ls - lse_ref)
    bar = 1e-3 + 1e-6 * np.abs(lse_ref)
    log(f"  lse: max error {lerr.max():.3e}, largest |lse| {np.abs(lse_ref).max():.1f}")
    assert (lerr <= bar).all(), f"lse error {lerr.max():.3e} above 1e-3 + 1e-6 |lse|"
