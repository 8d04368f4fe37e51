"""Parity of the 128-chunk 128k sweep, every chunk (needs a gfx950 GPU).

The sweep's prompt (N = 131072, C = 1024, 64 query / 8 KV heads, D = 128, bf16)
is appended to the paged cache once; then every one of its 128 chunks runs as one
extend launch (P = 1024 t, E = 1024; keys past a chunk's rows are masked, so the
later tokens in the cache change nothing) and is compared with the fp64 oracle on
a declared row sample: rows {0, 1, E/2, E-2, E-1} of the chunk plus 27 seeded
random rows, all 64 heads. The identity under test is the zdszero notes' claim
(section "prefill as several resumable extends") that each chunk equals the
one-shot causal prefill's rows up to floating-point order. The 128 chunks are
split over four tests; the oracle work (about 9 TFLOP of fp64) runs on a pool of
host threads, one chunk per task.
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

import chunked_prefill_attention_extend_amd as ext
import oracle
from synth import make_workload
from tests.harness import TOL, PagedCache, log

pytestmark = pytest.mark.gpu

N_PARTS = 4
RANDOM_ROWS = 27


@pytest.fixture(scope="module")
def sweep():
    w = make_workload("sweep128k")
    n, c, h = w.plan
    plan = ext.chunk_plan(n, c, h)
    assert plan == oracle.chunk_plan(n, c, h), "chunk plan differs from the oracle"
    req = w.requests[0]
    log("sweep128k: drawing K/V for 131072 tokens and appending them")
    k = w.k(req, 0, n)
    v = w.v(req, 0, n)
    cache = PagedCache(w)
    cache.append([0], [0], k, v, [n])
    torch.cuda.synchronize()
    return {"w": w, "req": req, "chunks": plan["chunks"], "cache": cache,
            "k64": k.astype(np.float64), "v64": v.astype(np.float64)}


def _rows(t: int, e: int) -> np.ndarray:
    rng = np.random.default_rng(1000 + t)
    fixed = np.array(sorted({0, 1, e // 2, e - 2, e - 1}))
    rest = np.setdiff1d(np.arange(e), fixed)
    return np.sort(np.concatenate([fixed, rng.choice(rest, RANDOM_ROWS, replace=False)]))


def _oracle_chunk(args):
    q_rows, pos, k64, v64, scale = args
    n = int(pos.max()) + 1
    return oracle.attend_rows(q_rows, k64[:n], v64[:n], pos, scale)


@pytest.mark.parametrize("part", range(N_PARTS))
def test_sweep128k_every_chunk(sweep, part):
    w, req, cache = sweep["w"], sweep["req"], sweep["cache"]
    chunks = sweep["chunks"]
    per = len(chunks) // N_PARTS
    ts = list(range(part * per, (part + 1) * per))
    log(f"sweep128k chunks {ts[0]}..{ts[-1]}: 32 sampled rows each, all 64 heads")
    jobs, got = [], []
    for t in ts:
        p, e = chunks[t]
        q = w.q(req, p, p + e)
        out, lse = cache.attend([0], [p], [e], q)
        sel = _rows(t, e)
        got.append((t, p, e, out[torch.from_numpy(sel).to(out.device)].float().cpu().numpy().astype(np.float64),
                    lse[torch.from_numpy(sel).to(out.device)].cpu().numpy().astype(np.float64)))
        jobs.append((q[sel], p + sel, sweep["k64"], sweep["v64"], w.scale))
    torch.cuda.synchronize()
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        limit = None
    try:
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            refs = list(ex.map(_oracle_chunk, jobs))
    finally:
        if limit is not None:
            limit.unregister()
    tol = TOL["bf16"]
    worst = {"max": 0.0, "mean": 0.0, "lse": 0.0}
    for (t, p, e, o, ls), (o_ref, l_ref) in zip(got, refs):
        assert np.isfinite(o).all() and np.isfinite(ls).all(), f"chunk {t}: non-finite output"
        err = np.abs(o - o_ref)
        res = {"max": float(err.max()), "mean": float(err.mean()), "lse": float(np.abs(ls - l_ref).max())}
        log(f"  chunk {t:3d} (P={p}, E={e}): max {res['max']:.3e} mean {res['mean']:.3e} lse {res['lse']:.3e}")
        for key in worst:
            worst[key] = max(worst[key], res[key])
        assert res["max"] <= tol["max"], f"chunk {t}: max abs error {res['max']}"
        assert res["mean"] <= tol["mean"], f"chunk {t}: mean abs error {res['mean']}"
        assert res["lse"] <= tol["lse"], f"chunk {t}: lse error {res['lse']}"
    log(f"  worst over chunks {ts[0]}..{ts[-1]}: max {worst['max']:.3e} mean {worst['mean']:.3e} "
        f"lse {worst['lse']:.3e}")
