"""The allocation-free entry point against extattn_extend_attention (needs a gfx950 GPU).

extattn_extend_attention_noalloc runs the same plan and kernels with the
library's static device scratch as the workspace. Two calls in a row (the second
with a smaller launch, so stale scratch contents from the first would show) must
give out / lse equal to the ordinary entry point's, bit for bit (and so within
the bf16 bars of the oracle comparison), with clean status words; a launch that
needs more than the scratch is refused before anything runs.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_attention_extend_amd as ext
from synth import custom_workload
from tests.harness import PagedCache, dev_tensor, log

pytestmark = pytest.mark.gpu


def _both(launches, hq, hkv, d, seed):
    w = custom_workload(seed, launches, hq, hkv, d)
    cache = PagedCache(w)
    for r in w.requests:
        p, e = r.launch
        cache.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    q = dev_tensor(np.concatenate([w.q(r, r.launch[0], r.launch[0] + r.launch[1]) for r in w.requests]), w.dtype)
    prefix = [r.launch[0] for r in w.requests]
    extend = [r.launch[1] for r in w.requests]
    o1, o2 = torch.empty_like(q), torch.full_like(q, float("nan"))
    l1 = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    l2 = torch.full_like(l1, float("nan"))
    ext.extend_attention(q, cache.k, cache.v, cache.bt, prefix, extend, w.scale, o1, l1, check=True)
    ext.extend_attention_noalloc(q, cache.k, cache.v, cache.bt, prefix, extend, w.scale, o2, l2)
    flags, bad, _ = ext.read_status(None)
    torch.cuda.synchronize()
    return o1, l1, o2, l2, flags, bad


def test_noalloc_matches_the_workspace_entry_point():
    cases = [
        # a mixed launch: decode rows (split items and their combine), a chunk cut into key pieces
        ([(3000, 1), (6000, 700), (40, 1), (900, 5)], 32, 8, 128, 31),
        # verify rows of 40-64 rows per KV head (the wide-split kernel), one context in two pieces
        ([(9000, 8), (3000, 5), (50, 1)], 64, 8, 128, 34),
        # then a smaller one: fewer items, no pieces
        ([(100, 50)], 16, 4, 64, 32),
    ]
    for launches, hq, hkv, d, seed in cases:
        log(f"no-alloc call: {launches} Hq={hq} Hkv={hkv} D={d}")
        o1, l1, o2, l2, flags, bad = _both(launches, hq, hkv, d, seed)
        assert flags == 0 and bad == 0, f"status {flags:#x} / {bad}"
        err = (o1.float() - o2.float()).abs().max().item()
        lerr = (l1 - l2).abs().max().item()
        log(f"  against extend_attention: out max {err:.3e}, lse max {lerr:.3e}")
        assert torch.isfinite(o2.float()).all() and torch.isfinite(l2).all()
        assert err <= 2e-2 and (o1.float() - o2.float()).abs().mean().item() <= 2e-3 and lerr <= 1e-3
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "the same plan and kernels must give the same bits"


def test_noalloc_refuses_launches_beyond_the_scratch():
    # 512 decode rows over 65536-key contexts: their split partials alone need far
    # more than the 64 MiB scratch, so the call fails before anything is enqueued
    n, ctx, hq, hkv, d = 512, 65536, 32, 8, 128
    need = ext.workspace_bytes([ctx - 1] * n, [1] * n, hq, hkv, d, ext.EXTATTN_BF16)
    assert need > 64 << 20
    q = torch.zeros((n, hq, d), dtype=torch.bfloat16, device="cuda")
    k_cache = torch.zeros((1, hkv, 16, d), dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros((1, hkv, d, 16), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((n, ctx // 16), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(ValueError, match="workspace too small"):
        ext.extend_attention_noalloc(q, k_cache, v_cache, bt, [ctx - 1] * n, [1] * n, 1.0 / np.sqrt(d), out)


def test_noalloc_under_graph_capture():
    """The allocation-free call captured in a HIP graph (torch.cuda.CUDAGraph) and
    replayed: its metadata travels in the captured kernels' arguments and the scratch
    is static, so every replay, with eager work and a synchronization between
    replays, gives the eager call's bits and clean status words."""
    launches, hq, hkv, d, seed = [(3000, 1), (2000, 300), (40, 1)], 32, 8, 128, 33
    w = custom_workload(seed, launches, hq, hkv, d)
    cache = PagedCache(w)
    for r in w.requests:
        p, e = r.launch
        cache.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    q = dev_tensor(np.concatenate([w.q(r, r.launch[0], r.launch[0] + r.launch[1]) for r in w.requests]), w.dtype)
    prefix = [r.launch[0] for r in w.requests]
    extend = [r.launch[1] for r in w.requests]
    o_ref = torch.empty_like(q)
    l_ref = torch.empty((q.shape[0], hq), dtype=torch.float32, device=q.device)
    log("graph capture: eager reference call")
    ext.extend_attention_noalloc(q, cache.k, cache.v, cache.bt, prefix, extend, w.scale, o_ref, l_ref, check=True)
    out = torch.full_like(q, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the side stream before capture
        ext.extend_attention_noalloc(q, cache.k, cache.v, cache.bt, prefix, extend, w.scale, out, lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    log("graph capture: capturing")
    with torch.cuda.graph(g):
        ext.extend_attention_noalloc(q, cache.k, cache.v, cache.bt, prefix, extend, w.scale, out, lse)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))  # eager work between the replays
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        log(f"graph capture: replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        flags, bad, _ = ext.read_status(None)
        assert flags == 0 and bad == 0, f"replay {rep}: status {flags:#x} / {bad}"
        assert torch.equal(out, o_ref) and torch.equal(lse, l_ref), f"replay {rep} differs from the eager call"
