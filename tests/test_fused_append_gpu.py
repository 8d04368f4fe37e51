"""KV append fused into the extend launch (needs a gfx950 GPU).

``extend_attention_append`` must leave the paged cache bit for bit as
``kv_append`` does and give the same ``out`` / ``lse`` bit for bit as
``kv_append`` followed by ``extend_attention`` (the attention work items are
the same; only where the new tokens' K/V come from in time differs), with no
status flag set. One case is also compared with the oracle directly.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_attention_extend_amd as ext
from synth import custom_workload
from tests.harness import PagedCache, check_launch, dev_tensor, log

pytestmark = pytest.mark.gpu


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _run_both(w):
    reqs = w.requests
    prefix = [r.launch[0] for r in reqs]
    extend = [r.launch[1] for r in reqs]
    idx = [r.index for r in reqs]
    q = np.concatenate([w.q(r, p, p + e) for r, p, e in zip(reqs, prefix, extend)])
    k_new = np.concatenate([w.k(r, p, p + e) for r, p, e in zip(reqs, prefix, extend)])
    v_new = np.concatenate([w.v(r, p, p + e) for r, p, e in zip(reqs, prefix, extend)])
    qd, kd, vd = dev_tensor(q, w.dtype), dev_tensor(k_new, w.dtype), dev_tensor(v_new, w.dtype)
    # separate: every token appended by kv_append, then attention
    sep = PagedCache(w)
    for r in reqs:
        p, e = r.launch
        sep.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    o1, l1 = sep.attend(idx, prefix, extend, q)
    # fused: prefixes appended beforehand, the new tokens by the attention launch
    fus = PagedCache(w)
    for r in reqs:
        p, _ = r.launch
        if p:
            fus.append([r.index], [0], w.k(r, 0, p), w.v(r, 0, p), [p])
    o2 = torch.empty_like(qd)
    l2 = torch.empty((qd.shape[0], w.n_q_heads), dtype=torch.float32, device="cuda")
    hkv, d = w.n_kv_heads, w.head_dim
    code = ext.EXTATTN_BF16 if w.dtype == "bf16" else ext.EXTATTN_F32
    ws = torch.zeros(ext.workspace_bytes(prefix, extend, w.n_q_heads, hkv, d, code), dtype=torch.uint8,
                     device="cuda")
    ext.extend_attention_append(qd, kd, vd, fus.k, fus.v, fus.bt, prefix, extend, w.scale, o2, l2, workspace=ws,
                                check=False)
    flags, _, exact = ext.read_status(ws)
    assert exact == 0, f"{exact} waves took the exact path"
    return (o1, l1, sep), (o2, l2, fus), flags, q


@pytest.mark.parametrize("case", [
    # (launches, Hq, Hkv, D, dtype)
    ([(3000, 1), (900, 600), (4000, 5), (12, 1), (0, 300)], 32, 8, 128, "bf16"),  # decode, verify, chunk, P=0
    ([(5000, 1024)], 64, 8, 128, "bf16"),   # one sweep-like chunk, prefix ending inside a block
    ([(6000, 700)], 32, 8, 128, "bf16"),    # chunk tiles cut into key pieces (pure-prefix pieces do not wait)
    ([(777, 40), (33, 1), (0, 17)], 16, 2, 64, "bf16"),  # D=64
    ([(3000, 5), (4000, 8), (12, 1), (9000, 7)], 64, 8, 128, "bf16"),  # 40-64 verify rows: wide kernel
    ([(50, 30), (129, 1)], 8, 2, 128, "f32"),  # fp32: append launch, then attention
    # copying workgroups take several 16-token groups each, none of them one whole cache
    # block (the prefix ends inside a block), the last group shared by two requests
    ([(37, 6003), (5000, 1)], 32, 8, 128, "bf16"),
    ([(40, 16)], 8, 8, 128, "bf16"),        # 8 work items, so 8 copying workgroups, 7 of them idle
])
def test_fused_append_matches_separate(case):
    launches, hq, hkv, d, dt = case
    w = custom_workload(700 + len(launches) + hq + d, launches, hq, hkv, d, dtype=dt,
                        mult=0.5 if dt == "bf16" else 1.0)
    log(f"fused append {launches} Hq={hq} Hkv={hkv} D={d} {dt}")
    (o1, l1, sep), (o2, l2, fus), err, q = _run_both(w)
    assert err == 0, f"status flags {err:#x}"
    assert torch.equal(_bits(sep.k), _bits(fus.k)), "K cache differs from kv_append's"
    assert torch.equal(_bits(sep.v), _bits(fus.v)), "V cache differs from kv_append's"
    assert torch.equal(o1, o2), "out differs from append + extend"
    assert torch.equal(l1, l2), "lse differs from append + extend"


def test_fused_append_against_oracle():
    w = custom_workload(777, [(2000, 1), (1500, 400), (0, 64)], 32, 8, 128)
    log("fused append against the oracle")
    _, (o2, l2, _), err, q = _run_both(w)
    assert err == 0
    offs = np.concatenate([[0], np.cumsum([r.launch[1] for r in w.requests])[:-1]]).astype(int)
    check_launch(w, o2, l2, {r.index: int(o) for r, o in zip(w.requests, offs)}, q, what="fused append")


def test_fused_append_invalid_block_ids_are_reported_not_written():
    """A new token whose block id is out of range is neither written nor read
    (the zero page stands in) and is reported in the status words; the other
    blocks are written as kv_append writes them. With the default check the
    call raises, also with a workspace of its own."""
    w = custom_workload(781, [(40, 24)], 8, 8, 128)
    r = w.requests[0]
    fus = PagedCache(w, fill=0.0)
    fus.append([0], [0], w.k(r, 0, 40), w.v(r, 0, 40), [40])
    bad = fus.bt.clone()
    bad[0, 3] = w.num_blocks + 1000      # block of positions 48..63 (new tokens 8..23)
    q = dev_tensor(w.q(r, 40, 64), w.dtype)
    kn = dev_tensor(w.k(r, 40, 64), w.dtype)
    vn = dev_tensor(w.v(r, 40, 64), w.dtype)
    out = torch.empty_like(q)
    ws = torch.zeros(ext.workspace_bytes([40], [24], 8, 8, 128, ext.EXTATTN_BF16), dtype=torch.uint8,
                     device="cuda")
    before = fus.k.clone()
    ext.extend_attention_append(q, kn, vn, fus.k, fus.v, bad, [40], [24], w.scale, out, None, workspace=ws,
                                check=False)
    flags, count, _ = ext.read_status(ws)
    assert flags == ext.STATUS_BAD_BLOCK and count > 0, f"status {flags:#x} / {count}"
    assert torch.isfinite(out.float()).all()
    blocks = [int(b) for b in r.blocks]
    # positions 40..47 (block 2) were written; nothing else changed
    assert not torch.equal(fus.k[blocks[2]], before[blocks[2]])
    others = [b for b in range(w.num_blocks) if b != blocks[2]]
    assert torch.equal(fus.k[others], before[others])
    with pytest.raises(ValueError, match="block id outside"):
        ext.extend_attention_append(q, kn, vn, fus.k, fus.v, bad, [40], [24], w.scale, out, None, workspace=ws)
    with pytest.raises(ValueError, match="block id outside"):
        ext.extend_attention_append(q, kn, vn, fus.k, fus.v, bad, [40], [24], w.scale, out, None)


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5, 6, 7, 8])
def test_fused_append_random_launches(seed):
    """Random mixed launches through the fused path: caches, out and lse bit for bit
    as kv_append followed by extend_attention."""
    rng = np.random.default_rng(2000 + seed)
    hq, hkv, d = [(32, 8, 128), (64, 8, 128), (16, 4, 64)][seed % 3]
    launches = []
    for _ in range(int(rng.integers(2, 7))):
        kind = int(rng.integers(0, 3))
        p = int(rng.integers(0, 5000))
        e = {0: 1, 1: int(rng.integers(2, 9)), 2: int(rng.integers(9, 900))}[kind]
        launches.append((p, e))
    w = custom_workload(3000 + seed, launches, hq, hkv, d)
    log(f"fused append, random launch {seed}: {launches} Hq={hq} Hkv={hkv} D={d}")
    (o1, l1, sep), (o2, l2, fus), err, q = _run_both(w)
    assert err == 0, f"error word {err:#x}"
    assert torch.equal(_bits(sep.k), _bits(fus.k)) and torch.equal(_bits(sep.v), _bits(fus.v))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
