"""Chunk tiles whose scores climb steeply along the keys (needs a gfx950 GPU).

The chunk path keeps a running max m that is raised only when a tile's weights
would pass 2^12 (its rare rescale path). Here the keys carry a common offset
that grows every 32 keys, so each tile's scores sit about 12 (log2 units) above
the tile before, some 190 to 360 above the first tile in all: without the
rescale the weights would overflow fp32. ``out`` is compared with the oracle at
the bf16 bar (max 2e-2, mean 2e-3). ``lse`` is compared with the bound that the
bf16 rounding of the scaled query rows (q * scale * log2 e, relative error
<= 2^-9 per element) gives, scale * 2^-9 * max_j sum_d |q_d k_jd| (natural log
units) plus fp32 terms, since that error grows with the scores' size; and,
sharper, with the oracle evaluated on that effective query, where only fp32
terms remain.
"""
import numpy as np
import pytest
import torch

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


@pytest.mark.parametrize("prefix,extend", [(0, 512), (960, 96)])
def test_rising_scores_take_the_rescale_path(prefix, extend):
    n = prefix + extend
    w = custom_workload(900 + prefix, [(prefix, extend)], HQ, HKV, D)
    q, k, v = _inputs(31 + prefix, n)
    log(f"rising scores: P={prefix}, E={extend}, {HQ}/{HKV} heads, D={D}")
    cache = PagedCache(w)
    cache.append([0], [0], k, v, [n])
    out, lse = cache.attend([0], [prefix], [extend], q[prefix:])
    torch.cuda.synchronize()
    pos = np.arange(prefix, n)
    o_ref, lse_ref = oracle.attend_rows(q[prefix:], k, v, pos, w.scale)
    o = out.float().cpu().numpy().astype(np.float64)
    ls = lse.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(ls).all()
    err = np.abs(o - o_ref)
    log(f"  out: max {err.max():.3e} mean {err.mean():.3e}; lse max {np.abs(ls - lse_ref).max():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3
    # per (row, head): 2^-9 * scale * max over visible keys of sum_d |q_d k_d|
    g = np.arange(HQ) // (HQ // HKV)
    qa = np.abs(q[prefix:].astype(np.float64))            # [E, HQ, D]
    ka = np.abs(k.astype(np.float64))[:, g, :]             # [n, HQ, D]
    mag = np.einsum("rhd,jhd->rhj", qa, ka)                 # [E, HQ, n]
    mag = np.where(np.arange(n)[None, None, :] > pos[:, None, None], 0.0, mag)
    bound = 2.0 ** -9 * w.scale * mag.max(axis=2) + 1e-4 + 1e-6 * np.abs(lse_ref)
    excess = np.abs(ls - lse_ref) - bound
    assert excess.max() <= 0.0, f"lse error above its bound by {excess.max():.3e}"
    # sharper: the chunk path's result is the attention of the effective query
    # round_bf16(q * c) / c, c = scale * log2(e) as the library forms it in fp32
    c = np.float32(np.float32(w.scale) * np.float32(1.4426950408889634))
    q_eff = round_to_bf16(q[prefix:] * c)[0].astype(np.float64) / float(c)
    o_eff, lse_eff = oracle.attend_rows(q_eff, k, v, pos, w.scale)
    d_eff = np.abs(ls - lse_eff).max()
    log(f"  against the effective query: out max {np.abs(o - o_eff).max():.3e}, lse max {d_eff:.3e}")
    assert d_eff <= 2e-3 + 1e-6 * np.abs(lse_eff).max()
