"""Parity of the HIP library against the CPU oracle (needs a gfx950 GPU).

Every test calls the library through its C ABI (ctypes binding) on seeded
synthetic inputs and compares element by element with the fp64 oracle:
bf16 inputs with fp32 accumulation within max abs 2e-2 / mean abs 2e-3
(lse within 1e-3); fp32 within 1e-5. Chunk plans must match bit for bit.
"""
import numpy as np
import pytest
import torch

import chunked_prefill_attention_extend_amd as ext
from synth import custom_workload, make_workload
from tests.harness import PagedCache, check_launch, compare, dev_tensor, log, oracle_rows, run_launch, run_planned

pytestmark = pytest.mark.gpu


def test_tiny_f32_all_chunks():
    log("tiny_f32: 64 tokens, C=16, fp32")
    res = run_planned(make_workload("tiny_f32"))
    assert len(res) == 4


def test_prompt4000_all_chunks_all_rows():
    log("prompt4000: 8 chunks, every row")
    res = run_planned(make_workload("prompt4000"))
    assert len(res) == 8


def test_prefix_cache32k_sampled_rows():
    """Both chunks, rows {0, 1, E/2, E-2, E-1} and 251 seeded random rows each, all
    32 heads (the 128-chunk sweep has its own module, test_sweep_parity_gpu.py)."""
    log("prefix_cache32k: 2 chunks at P=16384/24576, 256 sampled rows each")
    res = run_planned(make_workload("prefix_cache32k"), rows_per_chunk=256)
    assert len(res) == 2


def test_mixed_budget2048():
    w = make_workload("mixed_budget2048")
    log("mixed_budget2048: 64 decode rows + 1984-row chunk in one launch")
    out, lse, q_off, q = run_launch(w)
    rng = np.random.default_rng(3)
    chunk_rows = np.unique(np.concatenate([[0, 1, 991, 1982, 1983], rng.choice(1984, 120, replace=False)]))
    check_launch(w, out, lse, q_off, q, row_sample={64: chunk_rows}, what="mixed step")


@pytest.mark.parametrize("case", [
    # (launches, Hq, Hkv, D)
    ([(37, 100)], 28, 4, 128),            # group of 7, ragged tile and ragged key tail
    ([(0, 1)], 8, 8, 128),                # first token of a prompt: one key
    ([(0, 333)], 16, 2, 64),              # head_dim 64, empty rectangle
    ([(1000, 3), (5, 4)], 32, 4, 128),    # verify rows of 24 and 32 rows (split path, two row blocks)
    ([(500, 2), (64, 3), (2047, 4)], 32, 8, 128),  # verify rows of 8, 12, 16 rows (split path, one row block)
    ([(777, 2)], 64, 8, 64),              # 16 split rows at two positions, D=64
    ([(500, 3), (31, 4)], 64, 8, 64),     # 24 and 32 split rows (two row blocks), D=64
    ([(77, 5)], 64, 8, 128),              # 40 rows: one partial chunk tile
    ([(3000, 9), (40, 8)], 64, 8, 64),    # 72 and 64 rows: partial chunk tiles, D=64
    ([(300, 17)], 64, 1, 128),            # one KV head for 64 query heads
    ([(4095, 1), (16, 1), (1, 1)], 32, 8, 64),  # decode rows, D=64
    ([(6000, 700)], 32, 8, 128),          # 88 chunk tiles: key ranges cut in 3 pieces and merged; ragged end
    ([(5000, 256)], 16, 2, 64),           # 16 chunk tiles, D=64: 2 pieces
])
def test_edge_cases(case):
    launches, hq, hkv, d = case
    w = custom_workload(len(launches) * 100 + hq + d, launches, hq, hkv, d)
    log(f"edge case {launches} Hq={hq} Hkv={hkv} D={d}")
    out, lse, q_off, q = run_launch(w)
    check_launch(w, out, lse, q_off, q, what=f"edge {launches}")


def test_verify_rows_long_contexts():
    """Verify rows of 1..16 tokens (4..64 rows per KV head, so the launch runs on the
    4-wave wide kernel: split items of one to four row blocks) over contexts long
    enough that the split pieces reach their longest (4096 keys there); ten
    requests compared."""
    rng = np.random.default_rng(41)
    n = 40
    ctx = rng.integers(4000, 9000, size=n, endpoint=True)
    e = rng.integers(1, 16, size=n, endpoint=True)
    e[:3] = [1, 8, 16]
    launches = [(int(L - x), int(x)) for L, x in zip(ctx, e)]
    w = custom_workload(51, launches, 64, 16, 64)
    log(f"verify rows: {n} requests, E 1..16, context 4000..9000, 64/16 heads, D=64")
    out, lse, q_off, q = run_launch(w)
    keep = set(range(3)) | set(rng.choice(np.arange(3, n), 7, replace=False).tolist())
    sub = custom_workload(51, launches, 64, 16, 64)
    sub.requests = [r for r in sub.requests if r.index in keep]
    check_launch(sub, out, lse, q_off, q, what="verify rows, long contexts")


@pytest.mark.parametrize("d", [128, 64])
def test_verify_rows_40_to_64(d):
    """Verify rows of 5..8 tokens with 64 query / 8 KV heads: 40, 48, 56 and 64 rows
    per KV head, past the 8-wave split items' 32, next to a decode row (8 rows) and
    a 3-token row (24): the launch runs every request as split items of the 4-wave
    wide kernel (one to four 16-row blocks per wave), key ranges cut into
    4096-key pieces merged by the combine kernel. Contexts from a few keys to
    several pieces; every row of every request is compared, and the measurement
    variant gives the same bits."""
    launches = [(3, 5), (1000, 6), (4090, 7), (9000, 8), (250, 8), (16000, 5), (7000, 1), (5000, 3)]
    w = custom_workload(71 + d, launches, 64, 8, d)
    log(f"verify rows of 40..64 rows per KV head, D={d}")
    out, lse, q_off, q = run_launch(w)
    check_launch(w, out, lse, q_off, q, what=f"verify rows 40..64, D={d}")
    cache = PagedCache(w)
    for r in w.requests:
        p, e = r.launch
        cache.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    qd = dev_tensor(q, w.dtype)
    o2 = torch.empty_like(qd)
    l2 = torch.empty_like(lse)
    _, st, _ = ext.extend_attention(qd, cache.k, cache.v, cache.bt, [p for p, _ in launches],
                                    [e for _, e in launches], w.scale, o2, l2, timed=True)
    torch.cuda.synchronize()
    assert set(st[:, 2].cpu().numpy().tolist()) == {1}, "rows of 40..64 run as split items"
    assert torch.equal(out, o2) and torch.equal(lse, l2)


@pytest.mark.parametrize("d", [128, 64])
def test_split_tiles_through_lds(d):
    """Decode and verify rows on the 8-wave kernel's split items (32 query / 8 KV
    heads, 1..8 tokens: 4..32 rows per KV head, one and two 16-row blocks), whose
    waves copy their K/V tiles into LDS slots and read them back in operand layout:
    contexts from 1 key to several key pieces (merged by the combine kernel), ends at
    and next to block (16), tile (32) and wave-round (256 keys) boundaries, waves
    with no tile at all. Every row of every request against the oracle."""
    ctx = [1, 13, 31, 32, 33, 255, 256, 257, 1000, 4099, 8191, 8193, 20000]
    es = [1, 2, 4, 5, 8, 1, 3, 6, 7, 8, 1, 4, 2]
    launches = [(L - e, e) for L, e in zip(ctx, es)]
    w = custom_workload(91 + d, launches, 32, 8, d)
    log(f"split tiles through LDS: {len(launches)} requests, contexts 1..20000, 32/8 heads, D={d}")
    out, lse, q_off, q = run_launch(w)
    check_launch(w, out, lse, q_off, q, what=f"split tiles through LDS, D={d}")


def test_long_chunk_from_empty_prefix():
    """The largest chunk of the pages' workloads and then some: one 32768-token prompt
    from an empty cache (32 / 8 heads: 512 tiles per KV head, keys up to 32768),
    compared on sampled rows spread over the whole chunk."""
    w = custom_workload(4242, [(0, 32768)], 32, 8, 128)
    log("long chunk: P=0, E=32768, 32/8 heads, D=128, sampled rows")
    out, lse, q_off, q = run_launch(w)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 16383, 32766, 32767], rng.choice(32768, 25, replace=False)]))
    check_launch(w, out, lse, q_off, q, row_sample={0: rows}, what="long chunk")


def test_many_decode_rows():
    """300 decode rows in one launch (contexts 1..3000 tokens: 2400 split items, one
    per request and KV head, many of them a single tile), 30 requests compared."""
    rng = np.random.default_rng(77)
    ctx = rng.integers(1, 3000, size=300, endpoint=True)
    ctx[:3] = [1, 2, 3000]
    launches = [(int(c - 1), 1) for c in ctx]
    w = custom_workload(77, launches, 32, 8, 128)
    log("many decode rows: 300 requests, context 1..3000, 32/8 heads, D=128")
    out, lse, q_off, q = run_launch(w)
    keep = set(range(3)) | set(rng.choice(np.arange(3, 300), 27, replace=False).tolist())
    sub = custom_workload(77, launches, 32, 8, 128)
    sub.requests = [r for r in sub.requests if r.index in keep]
    check_launch(sub, out, lse, q_off, q, what="many decode rows")


@pytest.mark.parametrize("seed", [1, 2, 3, 4, 5, 6])
def test_random_mixed_launches(seed):
    """Random launches: head layout, head_dim, and a mix of decode rows, verify rows,
    short and long chunks with random prefixes (ragged against blocks and tiles),
    compared with the oracle on up to 24 sampled rows per request."""
    rng = np.random.default_rng(1000 + seed)
    hq, hkv = [(32, 8), (64, 8), (16, 16), (28, 4), (8, 1)][seed % 5]
    d = 128 if seed % 3 else 64
    launches = []
    for _ in range(int(rng.integers(2, 9))):
        kind = int(rng.integers(0, 4))
        p = int(rng.integers(0, 6000))
        e = {0: 1, 1: int(rng.integers(2, 9)), 2: int(rng.integers(9, 300)), 3: int(rng.integers(300, 1500))}[kind]
        launches.append((p, e))
    w = custom_workload(5000 + seed, launches, hq, hkv, d)
    log(f"random launch {seed}: {launches} Hq={hq} Hkv={hkv} D={d}")
    out, lse, q_off, q = run_launch(w)
    sample = {r.index: np.unique(np.concatenate([[0, r.launch[1] - 1], rng.integers(0, r.launch[1], 22)]))
              for r in w.requests}
    check_launch(w, out, lse, q_off, q, row_sample=sample, what=f"random launch {seed}")


def test_timed_variant_same_results_and_sane_stamps():
    """The measurement variant gives bit-identical results and one
    {start, end, kind, request} record per work item."""
    launches = [(3000, 1), (900, 600), (4000, 5), (12, 1)]
    w = custom_workload(61, launches, 32, 8, 128)
    log("timed variant: mixed launch of decode, verify and chunk rows")
    out, lse, q_off, q = run_launch(w)
    cache = PagedCache(w)
    for r in w.requests:
        p, e = r.launch
        cache.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    qd = dev_tensor(q, w.dtype)
    o2 = torch.empty_like(qd)
    l2 = torch.empty_like(lse)
    prefix = [p for p, _ in launches]
    extend = [e for _, e in launches]
    _, st, hz = ext.extend_attention(qd, cache.k, cache.v, cache.bt, prefix, extend, w.scale, o2, l2, timed=True)
    torch.cuda.synchronize()
    if not (torch.equal(out, o2) and torch.equal(lse, l2)):
        d = (out.float() - o2.float()).abs()
        rows = torch.nonzero(d.nan_to_num(1e9).amax(dim=(1, 2)) > 0).flatten().tolist()
        dl = (lse - l2).abs().nan_to_num(1e9)
        lrows = torch.nonzero(dl.amax(dim=1) > 0).flatten().tolist()
        raise AssertionError(f"timed launch changed the results: out rows {rows[:16]} ({len(rows)}), max "
                             f"{float(d.nan_to_num(1e9).max())}, NaN {int(torch.isnan(out.float()).sum())}/"
                             f"{int(torch.isnan(o2.float()).sum())}; lse rows {lrows[:16]} ({len(lrows)})")
    st = st.cpu().numpy()
    assert hz > 0 and st.shape[1] == 6 and st.shape[0] > 0
    assert (st[:, 1] >= st[:, 0]).all() and (st[:, 0] > 0).all()
    # shader-clock cycles over wall-clock time: a clock between 0.5 and 3.5 GHz
    sclk = (st[:, 5] - st[:, 4]).sum() / ((st[:, 1] - st[:, 0]).sum() / hz)
    assert (st[:, 5] >= st[:, 4]).all() and 0.5e9 < sclk < 3.5e9, sclk
    assert set(st[:, 2].tolist()) == {0, 1}
    kinds = {int(r): int(k) for k, r in zip(st[:, 2], st[:, 3])}
    assert kinds == {0: 1, 1: 0, 2: 1, 3: 1}, kinds   # rows per KV head: 4, 2400, 20, 4
    assert (st[:, 1].max() - st[:, 0].min()) / hz < 1.0


def test_timed_launch_holds_its_workspace(monkeypatch):
    """A timed launch without a caller workspace keeps the workspace that the
    binding allocates referenced until both of its library calls have been made,
    so the stamp buffer allocated between them never takes that memory (stamps
    written over the workspace's zero page reach the values of padded key tiles)."""
    import weakref
    from chunked_prefill_attention_extend_amd import binding
    made = []
    real_ws = binding._workspace

    def spy(*args, **kw):
        t = real_ws(*args, **kw)
        made.append(weakref.ref(t))
        return t

    lib = binding.load_library()
    real_timed = lib.extattn_extend_attention_timed
    seen = []

    def timed(*args):  # args: the 20 launch arguments, then stamps, capacity, n_items, tick_hz
        seen.append((args[17], args[18], args[20], [r() is not None for r in made]))
        return real_timed(*args)

    monkeypatch.setattr(binding, "_workspace", spy)
    monkeypatch.setattr(lib, "extattn_extend_attention_timed", timed)
    launches = [(3000, 1), (900, 600), (12, 1)]
    w = custom_workload(62, launches, 32, 8, 128)
    log("timed variant: workspace lifetime")
    cache = PagedCache(w)
    for r in w.requests:
        p, e = r.launch
        cache.append([r.index], [0], w.k(r, 0, p + e), w.v(r, 0, p + e), [p + e])
    q = dev_tensor(np.concatenate([w.q(r, p, p + e) for r, (p, e) in zip(w.requests, launches)]), w.dtype)
    o = torch.empty_like(q)
    made.clear()  # the cache appends above allocated their own
    _, stamps, _ = ext.extend_attention(q, cache.k, cache.v, cache.bt, [p for p, _ in launches],
                                        [e for _, e in launches], w.scale, o, None, timed=True)
    torch.cuda.synchronize()
    assert len(made) == 1 and len(seen) == 2, (len(made), len(seen))
    assert all(all(alive) for *_, alive in seen), "the workspace was freed before the launch"
    ws_ptr, ws_bytes, st_ptr, _ = seen[1]
    st_bytes = stamps.numel() * stamps.element_size()
    assert st_ptr + st_bytes <= ws_ptr or st_ptr >= ws_ptr + ws_bytes, "stamps overlap the workspace"


def test_fp32_mixed_and_gqa():
    w = custom_workload(7, [(50, 30), (129, 1), (0, 70)], 8, 2, 128, dtype="f32", mult=1.0)
    log("fp32 mixed launch with GQA")
    out, lse, q_off, q = run_launch(w)
    check_launch(w, out, lse, q_off, q, what="fp32 mixed")


def test_request_order_invariance():
    w = custom_workload(11, [(500, 1), (200, 300), (31, 1), (1000, 129)], 32, 8, 128)
    o1, l1, off1, _ = run_launch(w)
    o2, l2, off2, _ = run_launch(w, order=[3, 1, 0, 2])
    for r in w.requests:
        e = r.launch[1]
        a = o1[off1[r.index]:off1[r.index] + e]
        b = o2[off2[r.index]:off2[r.index] + e]
        assert torch.equal(a, b), f"request {r.index} depends on its place in the launch"


def test_block_permutation_and_determinism():
    launches = [(700, 200), (65, 1)]
    w1 = custom_workload(21, launches, 32, 8, 128, permute=True)
    w2 = custom_workload(21, launches, 32, 8, 128, permute=False)
    o1, l1, _, _ = run_launch(w1)
    o1b, l1b, _, _ = run_launch(w1)
    o2, l2, _, _ = run_launch(w2)
    assert torch.equal(o1, o1b) and torch.equal(l1, l1b), "repeat run differs"
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "result depends on physical block placement"


def test_decode_row_batch_invariance():
    w = custom_workload(31, [(2000, 1), (900, 600)], 32, 8, 128)
    out, lse, q_off, q = run_launch(w)
    alone = custom_workload(31, [(2000, 1)], 32, 8, 128)
    o2, l2, _, _ = run_launch(alone)
    assert torch.equal(out[q_off[0]:q_off[0] + 1], o2), "decode row differs when launched with a chunk"


def test_kv_append_layout():
    w = custom_workload(41, [(10, 40)], 8, 4, 128, permute=True)
    r = w.requests[0]
    cache = PagedCache(w, fill=0.0)
    k = w.k(r, 0, 50)
    v = w.v(r, 0, 50)
    cache.append([0], [0], k[:10], v[:10], [10])
    cache.append([0], [10], k[10:], v[10:], [40])
    kc = cache.k.float().cpu().numpy()
    vc = cache.v.float().cpu().numpy()
    for p in range(50):
        b, s = r.blocks[p // 16], p % 16
        assert np.array_equal(kc[b, :, s, :], k[p]), f"K of token {p}"
        assert np.array_equal(vc[b, :, :, s], v[p]), f"V of token {p}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_kv_append_layout_whole_blocks(dtype):
    """Appends that start on a block boundary fill whole cache blocks (the kernel's
    wide-row V path), followed by a ragged tail: every token lands where the block
    table says, in both element types."""
    w = custom_workload(43, [(16, 53)], 8, 2, 128, dtype=dtype, mult=0.5 if dtype == "bf16" else 1.0,
                        permute=True)
    r = w.requests[0]
    cache = PagedCache(w, fill=0.0)
    k = w.k(r, 0, 69)
    v = w.v(r, 0, 69)
    cache.append([0], [0], k[:16], v[:16], [16])      # one whole block
    cache.append([0], [16], k[16:], v[16:], [53])     # three whole blocks and a 5-token tail
    kc = cache.k.float().cpu().numpy()
    vc = cache.v.float().cpu().numpy()
    for p in range(69):
        b, s = r.blocks[p // 16], p % 16
        assert np.array_equal(kc[b, :, s, :], k[p]), f"K of token {p}"
        assert np.array_equal(vc[b, :, :, s], v[p]), f"V of token {p}"


def test_invalid_block_ids_are_reported_not_read():
    """An out-of-range block id reads as zeros and is reported in the status words;
    with check=True the call raises, with a workspace of its own too, and kv_append
    reports one the same way."""
    w = custom_workload(51, [(40, 8)], 8, 8, 128)
    cache = PagedCache(w, fill=0.0)
    r = w.requests[0]
    cache.append([0], [0], w.k(r, 0, 48), w.v(r, 0, 48), [48])
    bad = cache.bt.clone()
    bad[0, 1] = w.num_blocks + 1000
    q = dev_tensor(w.q(r, 40, 48), w.dtype)
    out = torch.empty_like(q)
    nbytes = ext.workspace_bytes([40], [8], 8, 8, 128, ext.EXTATTN_BF16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    ext.extend_attention(q, cache.k, cache.v, bad, [40], [8], w.scale, out, None, workspace=ws)
    flags, count, _ = ext.read_status(ws)
    assert flags == ext.STATUS_BAD_BLOCK and count > 0, f"status {flags:#x} / {count}"
    assert torch.isfinite(out.float()).all()
    # the next call over a valid table clears the status
    ext.extend_attention(q, cache.k, cache.v, cache.bt, [40], [8], w.scale, out, None, workspace=ws)
    assert ext.read_status(ws) == (0, 0, 0)
    with pytest.raises(ValueError, match="block id outside"):
        ext.extend_attention(q, cache.k, cache.v, bad, [40], [8], w.scale, out, None, workspace=ws, check=True)
    with pytest.raises(ValueError, match="block id outside"):
        ext.extend_attention(q, cache.k, cache.v, bad, [40], [8], w.scale, out, None, check=True)
    # decode rows (split path) meet the bad id too
    qd = q[-1:].contiguous()
    with pytest.raises(ValueError, match="block id outside"):
        ext.extend_attention(qd, cache.k, cache.v, bad, [47], [1], w.scale, torch.empty_like(qd), None, check=True)
    kn = dev_tensor(w.k(r, 40, 48), w.dtype)
    with pytest.raises(ValueError, match="block id outside"):
        ext.kv_append(kn, kn, cache.k, cache.v, bad, [16], [8], check=True)


def test_invalid_block_ids_in_a_wide_split_launch():
    """Verify rows of 48 rows per KV head (64 q / 8 kv heads, 6 tokens) run on the
    4-wave wide-split kernel; an out-of-range block id there is read as zeros,
    counted in the status words and raised with check=True, and the rows stay
    finite."""
    w = custom_workload(52, [(40, 6)], 64, 8, 128)
    cache = PagedCache(w, fill=0.0)
    r = w.requests[0]
    cache.append([0], [0], w.k(r, 0, 46), w.v(r, 0, 46), [46])
    bad = cache.bt.clone()
    bad[0, 1] = w.num_blocks + 7
    q = dev_tensor(w.q(r, 40, 46), w.dtype)
    out = torch.empty_like(q)
    nbytes = ext.workspace_bytes([40], [6], 64, 8, 128, ext.EXTATTN_BF16)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    _, st, _ = ext.extend_attention(q, cache.k, cache.v, bad, [40], [6], w.scale, out, None, workspace=ws,
                                    timed=True)
    torch.cuda.synchronize()
    assert set(st[:, 2].cpu().numpy().tolist()) == {1}, "48 rows run as split items"
    flags, count, _ = ext.read_status(ws)
    assert flags == ext.STATUS_BAD_BLOCK and count > 0, f"status {flags:#x} / {count}"
    assert torch.isfinite(out.float()).all()
    with pytest.raises(ValueError, match="block id outside"):
        ext.extend_attention(q, cache.k, cache.v, bad, [40], [6], w.scale, out, None, check=True)
    ext.extend_attention(q, cache.k, cache.v, cache.bt, [40], [6], w.scale, out, None, workspace=ws)
    assert ext.read_status(ws) == (0, 0, 0)


def test_device_argument_errors():
    w = custom_workload(61, [(16, 16)], 8, 2, 128)
    cache = PagedCache(w, fill=0.0)
    q = torch.zeros((16, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(ValueError):
        ext.extend_attention(q, cache.k, cache.v, cache.bt, [16], [16], -1.0, out)
    with pytest.raises(ValueError):
        ext.extend_attention(q, cache.k, cache.v, cache.bt, [16000], [16], 0.1, out)
    small = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        ext.extend_attention(q, cache.k, cache.v, cache.bt, [16], [16], 0.1, out, workspace=small)


def test_planner_to_launch_budget2048():
    """A queue planned by the library's token-budget step (the token-budget blog's
    section-5 example: budget 2048, 8 decode rows, a running prefill needing 1440,
    a waiting 900-token prompt cut to 600) run as one launch and checked against
    the oracle."""
    running = [(1001 + 37 * i, 1000 + 37 * i) for i in range(8)] + [(3000, 1560)]
    waiting = [(900, 0), (500, 0)]
    entries, left = ext.token_budget_step(running, waiting, 2048)
    assert [e[3] for e in entries] == [1] * 8 + [1440, 600] and left == 0
    launches = [(e[2], e[3]) for e in entries]
    w = custom_workload(2048, launches, 32, 8, 128)
    log(f"planned launch {launches}")
    out, lse, q_off, q = run_launch(w)
    check_launch(w, out, lse, q_off, q, what="planned budget-2048 step")
