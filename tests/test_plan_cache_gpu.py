"""Launch plans taken from the library's plan table (needs a gfx950 GPU).

A launch whose plan comes from the table (sized first by workspace_bytes, then
repeated, evicted and rebuilt, shared between the plain and the fused-append
call of one shape) gives bit for bit the results of a launch planned from
scratch with the table off, and those match the oracle.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_attention_extend_amd as ext
from synth import custom_workload
from tests.harness import PagedCache, check_launch, dev_tensor, log

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def restore_table():
    yield
    ext.plan_cache_configure(256, 64 << 20)
    ext.plan_cache_clear()


def _launch(cache, w, q, prefix, extend, ws):
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], w.n_q_heads), dtype=torch.float32, device="cuda")
    ext.extend_attention(q, cache.k, cache.v, cache.bt, prefix, extend, w.scale, o, lse, workspace=ws)
    return o, lse


def test_cached_plans_give_the_same_results():
    launches = [(3000, 1), (900, 600), (4000, 5), (12, 1), (0, 300)]
    w = custom_workload(91, launches, 32, 8, 128)
    log(f"plan table: mixed launch {launches}")
    reqs = w.requests
    prefix = [r.launch[0] for r in reqs]
    extend = [r.launch[1] for r in reqs]
    cache = PagedCache(w)
    for r in reqs:
        p, e = r.launch
        cache.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    q_np = np.concatenate([w.q(r, p, p + e) for r, p, e in zip(reqs, prefix, extend)])
    q = dev_tensor(q_np, w.dtype)
    other = ([2000], [900])  # a second shape (within request 0's blocks) that evicts the first

    ext.plan_cache_configure(0)
    ext.plan_cache_clear()
    nbytes = ext.workspace_bytes(prefix, extend, 32, 8, 128, ext.EXTATTN_BF16)
    ws = torch.zeros(max(nbytes, ext.workspace_bytes(*other, 32, 8, 128, ext.EXTATTN_BF16)), dtype=torch.uint8,
                     device="cuda")
    o_ref, l_ref = _launch(cache, w, q, prefix, extend, ws)
    torch.cuda.synchronize()
    assert ext.plan_cache_stats()["entries"] == 0

    ext.plan_cache_configure(1)
    ext.plan_cache_clear()
    assert ext.workspace_bytes(prefix, extend, 32, 8, 128, ext.EXTATTN_BF16) == nbytes  # miss: plans, keeps
    results = [_launch(cache, w, q, prefix, extend, ws) for _ in range(2)]  # hits
    st = ext.plan_cache_stats()
    assert st["misses"] == 1 and st["hits"] == 2, st
    # evict with another shape (its launch reads request 0's blocks), then rebuild
    o_other = torch.empty((900, 32, 128), dtype=torch.bfloat16, device="cuda")
    ext.extend_attention(torch.zeros_like(o_other), cache.k, cache.v, cache.bt[:1], other[0], other[1], w.scale,
                         o_other, None, workspace=ws)
    results.append(_launch(cache, w, q, prefix, extend, ws))
    torch.cuda.synchronize()
    st = ext.plan_cache_stats()
    assert st["misses"] == 3 and st["hits"] == 2, st
    for i, (o, l) in enumerate(results):
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), f"launch {i} with a table plan differs"
    offs = np.concatenate([[0], np.cumsum(extend)[:-1]]).astype(int)
    check_launch(w, results[0][0], results[0][1], {r.index: int(o) for r, o in zip(reqs, offs)}, q_np,
                 what="table plan")


def test_plain_and_fused_calls_share_one_record():
    launches = [(2000, 1), (1500, 400), (0, 64)]
    w = custom_workload(92, launches, 32, 8, 128)
    log(f"plan table: plain and fused calls of {launches}")
    reqs = w.requests
    prefix = [r.launch[0] for r in reqs]
    extend = [r.launch[1] for r in reqs]
    q_np = np.concatenate([w.q(r, p, p + e) for r, p, e in zip(reqs, prefix, extend)])
    k_new = dev_tensor(np.concatenate([w.k(r, p, p + e) for r, p, e in zip(reqs, prefix, extend)]), w.dtype)
    v_new = dev_tensor(np.concatenate([w.v(r, p, p + e) for r, p, e in zip(reqs, prefix, extend)]), w.dtype)
    q = dev_tensor(q_np, w.dtype)
    ext.plan_cache_clear()
    ws = torch.zeros(ext.workspace_bytes(prefix, extend, 32, 8, 128, ext.EXTATTN_BF16), dtype=torch.uint8,
                     device="cuda")
    full = PagedCache(w)
    for r in reqs:
        p, e = r.launch
        full.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    o1, l1 = _launch(full, w, q, prefix, extend, ws)
    fused = PagedCache(w)
    for r in reqs:
        p, _ = r.launch
        if p:
            fused.append([r.index], [0], w.k(r, 0, p), w.v(r, 0, p), [p])
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(l1)
    ext.extend_attention_append(q, k_new, v_new, fused.k, fused.v, fused.bt, prefix, extend, w.scale, o2, l2,
                                workspace=ws)
    torch.cuda.synchronize()
    st = ext.plan_cache_stats()
    assert st["misses"] == 1 and st["hits"] == 2 and st["entries"] == 1, st
    assert ext.read_status(ws) == (0, 0, 0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "fused call with the shared record differs"
    offs = np.concatenate([[0], np.cumsum(extend)[:-1]]).astype(int)
    check_launch(w, o2, l2, {r.index: int(o) for r, o in zip(reqs, offs)}, q_np, what="shared record")
