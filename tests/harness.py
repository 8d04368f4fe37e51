"""Shared GPU test plumbing: upload synthetic workloads, run the HIP library
through its binding, and compare with the CPU oracle.

Inputs come from ``synth`` (seeded). The GPU side receives them through
PyTorch tensors; the oracle receives the same values as float64. Nothing here
computes attention.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

import chunked_prefill_attention_extend_amd as ext
import oracle
from synth import Workload

TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}

# Tolerances. out: the required bars for bf16 inputs with fp32 accumulation
# (max abs 2e-2, mean abs 2e-3) and for fp32 (1e-5). lse (natural log): 1e-3 for
# bf16 inputs, 1e-5 for fp32, against the exact fp64 log-sum-exp of the scaled
# scores. The kernels form every score from the unmodified inputs and sum the
# fp32 weights before rounding them for the P.V product, so lse carries only fp32
# rounding (scale * log2 e to fp32, the exponent's fma, exp2 / log2, and the sum
# over up to 2^17 keys), far inside 1e-3 for the pages' score ranges; the largest
# |lse| seen by these tests is a few hundred, whose fp32 spacing is 3e-5.
TOL = {
    "bf16": {"max": 2e-2, "mean": 2e-3, "lse": 1e-3},
    "f32": {"max": 1e-5, "mean": 1e-5, "lse": 1e-5},
}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(vals: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Upload fp32 values that are exactly representable in ``dtype``."""
    return torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to(device).to(TORCH_DT[dtype])


class PagedCache:
    """Device paged cache for a workload, pre-filled with NaN so that unused
    slots would poison any result that read them."""

    def __init__(self, w: Workload, device="cuda", fill=float("nan"), block_table: np.ndarray | None = None):
        self.w = w
        self.expect_fast = True
        dt = TORCH_DT[w.dtype]
        self.k = torch.full((w.num_blocks, w.n_kv_heads, w.block_size, w.head_dim), fill, dtype=dt, device=device)
        self.v = torch.full((w.num_blocks, w.n_kv_heads, w.head_dim, w.block_size), fill, dtype=dt, device=device)
        bt = w.block_table() if block_table is None else block_table
        self.bt_host = bt
        self.bt = torch.from_numpy(np.ascontiguousarray(bt, dtype=np.int32)).to(device)

    def rows(self, idx: list[int]) -> torch.Tensor:
        return torch.from_numpy(np.ascontiguousarray(self.bt_host[idx], dtype=np.int32)).to(self.k.device)

    def append(self, req_idx: list[int], prefix: list[int], k_rows: np.ndarray, v_rows: np.ndarray,
               extend: list[int]) -> None:
        bt = self.bt if list(req_idx) == list(range(self.bt_host.shape[0])) else self.rows(req_idx)
        ext.kv_append(dev_tensor(k_rows, self.w.dtype), dev_tensor(v_rows, self.w.dtype), self.k, self.v, bt,
                      prefix, extend, check=True)

    def attend(self, req_idx: list[int], prefix: list[int], extend: list[int], q_rows: np.ndarray):
        w = self.w
        bt = self.bt if list(req_idx) == list(range(self.bt_host.shape[0])) else self.rows(req_idx)
        q = dev_tensor(q_rows, w.dtype)
        out = torch.empty_like(q)
        lse = torch.empty((q.shape[0], w.n_q_heads), dtype=torch.float32, device=q.device)
        ext.extend_attention(q, self.k, self.v, bt, prefix, extend, w.scale, out, lse, check=True)
        # the pages' workloads keep every tile's weights far inside the fast loop's
        # bound: no wave may take the exact two-pass path
        if self.expect_fast:
            assert ext.last_status()[2] == 0, f"{ext.last_status()[2]} waves took the exact path"
        return out, lse


def compare(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref: np.ndarray, lse_ref: np.ndarray, dtype: str,
            what: str = "") -> dict:
    o = o_gpu.float().cpu().numpy().astype(np.float64)
    ls = lse_gpu.cpu().numpy().astype(np.float64)
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    assert np.isfinite(ls).all(), f"{what}: non-finite lse"
    err = np.abs(o - o_ref)
    res = {"max": float(err.max()), "mean": float(err.mean()), "lse": float(np.abs(ls - lse_ref).max())}
    tol = TOL[dtype]
    log(f"  {what}: max {res['max']:.3e} mean {res['mean']:.3e} lse {res['lse']:.3e}")
    assert res["max"] <= tol["max"], f"{what}: max abs error {res['max']} > {tol['max']}"
    assert res["mean"] <= tol["mean"], f"{what}: mean abs error {res['mean']} > {tol['mean']}"
    assert res["lse"] <= tol["lse"], f"{what}: lse error {res['lse']} > {tol['lse']}"
    return res


def oracle_rows(w: Workload, req, positions: np.ndarray, q_rows: np.ndarray):
    """Oracle output for query rows of one request at the given global positions."""
    n = int(positions.max()) + 1
    k = w.k(req, 0, n)
    v = w.v(req, 0, n)
    return oracle.attend_rows(q_rows, k, v, positions, w.scale)


def run_planned(w: Workload, check_chunks=None, rows_per_chunk=None, seed: int = 0):
    """Run a single-request planned workload chunk by chunk (append, then attend).

    check_chunks: indices of chunks whose outputs are compared (default all).
    rows_per_chunk: None for every row, else the number of sampled rows
    (always including the first two and last two rows of the chunk).
    Returns the list of per-chunk comparison results.
    """
    n, c, h = w.plan
    plan = ext.chunk_plan(n, c, h)
    ref_plan = oracle.chunk_plan(n, c, h)
    assert plan == ref_plan, "chunk plan differs from the oracle"
    req = w.requests[0]
    cache = PagedCache(w)
    cached = plan["cached"]
    if cached:
        cache.append([0], [0], w.k(req, 0, cached), w.v(req, 0, cached), [cached])
    chunks = plan["chunks"]
    check = set(range(len(chunks)) if check_chunks is None else check_chunks)
    rng = np.random.default_rng(seed)
    results = []
    for t, (p, e) in enumerate(chunks):
        cache.append([0], [p], w.k(req, p, p + e), w.v(req, p, p + e), [e])
        if t not in check:
            continue
        q = w.q(req, p, p + e)
        out, lse = cache.attend([0], [p], [e], q)
        if rows_per_chunk is None or rows_per_chunk >= e:
            sel = np.arange(e)
        else:
            fixed = np.array(sorted({0, 1, e - 2, e - 1, e // 2}))
            extra = rng.choice(e, size=max(0, rows_per_chunk - len(fixed)), replace=False)
            sel = np.unique(np.concatenate([fixed, extra]))
        o_ref, lse_ref = oracle_rows(w, req, p + sel, q[sel])
        results.append(compare(out[sel], lse[sel], o_ref, lse_ref, w.dtype, f"{w.name} chunk {t} (P={p}, E={e})"))
    torch.cuda.synchronize()
    return results


def run_launch(w: Workload, order: list[int] | None = None, row_sample: dict | None = None):
    """Run one mixed launch of an explicit workload (each request's own (P, E)).

    All K/V (prefix and the chunk's own tokens) is appended first. ``order``
    permutes the requests inside the launch. ``row_sample`` maps request index
    to the chunk rows to compare (default all rows of every request).
    Returns (out, lse, q_off by request index).
    """
    reqs = w.requests if order is None else [w.requests[i] for i in order]
    idx = [r.index for r in reqs]
    prefix = [r.launch[0] for r in reqs]
    extend = [r.launch[1] for r in reqs]
    cache = PagedCache(w)
    # append everything the launch reads, request by request
    for r in reqs:
        p, e = r.launch
        cache.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    q = np.concatenate([w.q(r, r.launch[0], r.launch[0] + r.launch[1]) for r in reqs])
    out, lse = cache.attend(idx, prefix, extend, q)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(extend)[:-1]]).astype(int)
    q_off = {r.index: int(o) for r, o in zip(reqs, offs)}
    return out, lse, q_off, q


def check_launch(w: Workload, out, lse, q_off: dict, q: np.ndarray, row_sample: dict | None = None,
                 what: str = ""):
    o_all, l_all, ref_o, ref_l = [], [], [], []
    for r in w.requests:
        p, e = r.launch
        sel = np.arange(e) if row_sample is None or r.index not in row_sample else np.asarray(row_sample[r.index])
        rows = q_off[r.index] + sel
        o_ref, lse_ref = oracle_rows(w, r, p + sel, q[rows])
        o_all.append(out[torch.from_numpy(rows).to(out.device)])
        l_all.append(lse[torch.from_numpy(rows).to(out.device)])
        ref_o.append(o_ref)
        ref_l.append(lse_ref)
    return compare(torch.cat(o_all), torch.cat(l_all), np.concatenate(ref_o), np.concatenate(ref_l), w.dtype,
                   what or w.name)


def algorithmic_flops(prefix: list[int], extend: list[int], hq: int, d: int) -> int:
    """4 * D * Hq * (number of unmasked (query, key) pairs)."""
    pairs = sum(e * p + e * (e + 1) // 2 for p, e in zip(prefix, extend))
    return 4 * d * hq * pairs


def default_scale(d: int) -> float:
    return float(np.float32(1.0 / math.sqrt(d)))
