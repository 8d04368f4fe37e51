"""Benchmark of chunked-prefill extend attention on one MI355X.

A step is one pass of the whole hot path over the 128-chunk 128k-token sweep:
for each of the 128 chunks (P = 1024 t, E = 1024), append the chunk's K/V to the
paged cache, then run extend attention for its 1024 query rows over keys
0 .. P+i (64 query heads, 8 KV heads, head dim 128, bf16, block size 16,
seeded permuted block table). ``value`` is the sweep's algorithmic FLOPs
(4 * D * Hq * unmasked query-key pairs, 281.48 TFLOP) divided by the measured
step time, with all inputs resident in HBM before the timed region.

The JSON line also carries:
* roofline: the attention kernel's achieved TFLOP/s over its own launches
  (HIP events on the launch stream around every extend_attention call),
  against the bf16 dense MFMA peak, with the shader clock the kernel ran at
  (measured from one timed launch's per-workgroup cycle and wall-clock stamps);
* mixed_step: the 2048-token mixed step (64 decode rows + a 1984-row chunk in
  one launch); decode-row HBM GB/s measured on the same launch with the chunk
  request removed, against the 8 TB/s HBM peak;
* verify_rows: multi-token verify rows (E = 1..8) over the mixed step's contexts;
* config_table: GPU time of the three single-prompt workloads (tiny fp32, a
  4000-token prompt, 32768 tokens at hit rate 0.5);
* chunk_size_sweep: attention TFLOP/s of one 65536-token prompt at C = 256 .. 16384;
* cpu_baseline: the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4 SIMD x 1024 bf16 FLOP/clk x 2.4 GHz (dense)
PEAK_CLOCK_GHZ = 2.4
PEAK_HBM_GBS = 8000.0

SWEEP = dict(n=131072, chunk=1024, hq=64, hkv=8, d=128)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_bf16_sweep128k_traffic.json")
SWEEP_KERNEL = "chunk_bf16_kernel<128, 1, 8>"   # the attention kernel of the sweep's launches


def code_hash(files) -> str:
    """sha256 over the given sources with // comments and blank lines removed, so
    that only code changes (not comment edits) count as a changed kernel."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        for line in open(os.path.join(ROOT, f), encoding="utf-8"):
            code = re.sub(r"//.*", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE runs (copy-calibrated), or None when the kernel code changed
    since those counters were taken."""
    try:
        t = json.load(open(TRAFFIC_FILE))
        if code_hash(t["source_files"]) != t.get("code_sha256"):
            return None
    except (OSError, ValueError, KeyError):
        return None
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]


def sweep_flops(chunks, hq, d) -> int:
    return 4 * d * hq * sum(e * p + e * (e + 1) // 2 for p, e in chunks)


def setup_sweep(torch, ext, synth):
    n, c, hq, hkv, d = SWEEP["n"], SWEEP["chunk"], SWEEP["hq"], SWEEP["hkv"], SWEEP["d"]
    w = synth.make_workload("sweep128k")
    plan = ext.chunk_plan(n, c, 0.0)["chunks"]
    dev = "cuda"
    bf = torch.bfloat16
    q = synth.device_normal((n, hq, d), 5001, 0.5, bf)
    k_new = synth.device_normal((n, hkv, d), 5002, 0.5, bf)
    v_new = synth.device_normal((n, hkv, d), 5003, 0.5, bf)
    k_cache = torch.zeros((w.num_blocks, hkv, 16, d), dtype=bf, device=dev)
    v_cache = torch.zeros((w.num_blocks, hkv, d, 16), dtype=bf, device=dev)
    bt = torch.from_numpy(w.block_table()).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((n, hq), dtype=torch.float32, device=dev)
    ws_bytes = max(ext.workspace_bytes([p], [e], hq, hkv, d, ext.EXTATTN_BF16) for p, e in plan)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    kv_ws = torch.empty(4096, dtype=torch.uint8, device=dev)
    return dict(w=w, plan=plan, q=q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, bt=bt,
                out=out, lse=lse, ws=ws, kv_ws=kv_ws, scale=w.scale)


def sweep_step(ext, s, events=None, fused=False):
    """One pass over the 128 chunks. ``events``: list of (start, end) pairs
    recorded around each extend_attention call. ``fused``: each chunk's K/V
    append runs inside its attention launch (extend_attention_append)."""
    for t, (p, e) in enumerate(s["plan"]):
        if fused:
            if events is not None:
                events[t][0].record()
            ext.extend_attention_append(s["q"][p:p + e], s["k_new"][p:p + e], s["v_new"][p:p + e], s["k_cache"],
                                        s["v_cache"], s["bt"], [p], [e], s["scale"], s["out"][p:p + e],
                                        s["lse"][p:p + e], workspace=s["ws"], check=False)
            if events is not None:
                events[t][1].record()
            continue
        ext.kv_append(s["k_new"][p:p + e], s["v_new"][p:p + e], s["k_cache"], s["v_cache"], s["bt"], [p], [e],
                      workspace=s["kv_ws"])
        if events is not None:
            events[t][0].record()
        ext.extend_attention(s["q"][p:p + e], s["k_cache"], s["v_cache"], s["bt"], [p], [e], s["scale"],
                             s["out"][p:p + e], s["lse"][p:p + e], workspace=s["ws"])
        if events is not None:
            events[t][1].record()


def shader_clock(torch, ext, s, t: int = -1):
    """The shader clock the attention kernel runs at on sweep chunk t (the last,
    heaviest one by default): a timed launch of that chunk, whose per-workgroup
    stamps hold both shader-clock cycles and wall-clock ticks. Returns GHz, the
    cycle-weighted mean over the workgroups."""
    p, e = s["plan"][t]
    _, st, hz = ext.extend_attention(s["q"][p:p + e], s["k_cache"], s["v_cache"], s["bt"], [p], [e], s["scale"],
                                     s["out"][p:p + e], s["lse"][p:p + e], workspace=s["ws"], timed=True)
    torch.cuda.synchronize()
    st = st.cpu().numpy().astype(np.float64)
    return float((st[:, 5] - st[:, 4]).sum() / ((st[:, 1] - st[:, 0]).sum() / hz) / 1e9)


def check_status(ext, s) -> None:
    """Raise if the last launches left a status flag in their workspaces (an
    invalid block id, a fused-append wait that gave up): their timings would not
    stand for valid results."""
    for name, ws in (("attention", s["ws"]), ("kv_append", s["kv_ws"])):
        flags, count, exact = ext.read_status(ws)
        err = ext.status_error(flags, count, name)
        if err is not None:
            raise err


def mixed_step_bench(torch, ext, synth, reps: int = 10):
    """2048-token mixed step: one launch with 64 decode rows and a 1984-row chunk."""
    w = synth.make_workload("mixed_budget2048")
    dev = "cuda"
    bf = torch.bfloat16
    reqs = w.requests
    hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
    k_cache = torch.zeros((w.num_blocks, hkv, 16, d), dtype=bf, device=dev)
    v_cache = torch.zeros((w.num_blocks, hkv, d, 16), dtype=bf, device=dev)
    bt_all = w.block_table()
    # fill each request's context (untimed)
    for r in reqs:
        p, e = r.launch
        kk = synth.device_normal((p + e, hkv, d), 6000 + r.index, 0.5, bf)
        vv = synth.device_normal((p + e, hkv, d), 7000 + r.index, 0.5, bf)
        ext.kv_append(kk, vv, k_cache, v_cache, torch.from_numpy(bt_all[r.index:r.index + 1]).to(dev), [0], [p + e])
    prefix = [r.launch[0] for r in reqs]
    extend = [r.launch[1] for r in reqs]
    q = synth.device_normal((sum(extend), hq, d), 6999, 0.5, bf)
    out = torch.empty_like(q)
    lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=dev)
    bt = torch.from_numpy(bt_all).to(dev)
    dec = [i for i, r in enumerate(reqs) if r.launch[1] == 1]
    ci = [i for i in range(len(reqs)) if i not in dec]
    # one workspace for the three launches timed below (the whole step, its decode
    # rows alone, its chunk alone)
    ws_bytes = max(ext.workspace_bytes(prefix, extend, hq, hkv, d, ext.EXTATTN_BF16),
                   ext.workspace_bytes([prefix[i] for i in dec], [1] * len(dec), hq, hkv, d, ext.EXTATTN_BF16),
                   ext.workspace_bytes([prefix[i] for i in ci], [extend[i] for i in ci], hq, hkv, d,
                                       ext.EXTATTN_BF16))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    bt_dec = torch.from_numpy(bt_all[dec]).to(dev)
    q_dec = q[:len(dec)] if dec == list(range(len(dec))) else None
    assert q_dec is not None, "decode rows are expected first"
    out_dec = torch.empty_like(q_dec)
    lse_dec = torch.empty((len(dec), hq), dtype=torch.float32, device=dev)
    flush = torch.empty(512 * 2**20, dtype=torch.uint8, device=dev)

    def timed(fn):
        """GPU time of one call (its metadata copy and kernels), median over reps. The
        GPU is first given ~10 ms of fills so that the host enqueues every call ahead
        of the GPU: the events then bracket device work only, not host-side planning."""
        torch.cuda.synchronize()
        for _ in range(100):
            flush.fill_(0x5A)
        evs = []
        for i in range(reps + 2):
            flush.fill_(i & 0xFF)   # evict the 256 MB last-level cache between repetitions
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e-3 for a, b in evs[2:]]
        return float(np.median(ts)), float(np.min(ts))

    (t_mix, t_mix_min) = timed(lambda: ext.extend_attention(q, k_cache, v_cache, bt, prefix, extend, w.scale, out, lse,
                                               workspace=ws))
    (t_dec, t_dec_min) = timed(lambda: ext.extend_attention(q_dec, k_cache, v_cache, bt_dec, [prefix[i] for i in dec],
                                               [1] * len(dec), w.scale, out_dec, lse_dec, workspace=ws))
    c_off = sum(extend[i] for i in dec)   # the chunk's rows follow the decode rows
    q_chk = q[c_off:]
    out_chk = torch.empty_like(q_chk)
    lse_chk = torch.empty((q_chk.shape[0], hq), dtype=torch.float32, device=dev)
    bt_chk = torch.from_numpy(bt_all[ci]).to(dev)
    (t_chk, t_chk_min) = timed(lambda: ext.extend_attention(q_chk, k_cache, v_cache, bt_chk, [prefix[i] for i in ci],
                                               [extend[i] for i in ci], w.scale, out_chk, lse_chk, workspace=ws))
    dec_bytes = 0
    for i in dec:
        L = prefix[i] + 1
        dec_bytes += 2 * L * hkv * d * 2 + 2 * hq * d * 2 + 4 * hq + 4 * math.ceil(L / 16)
    # Inside the full mixed launch: per-workgroup wall-clock stamps (measurement
    # variant of the same launch), decode span = first decode workgroup start to
    # last decode workgroup end (the combine kernel after it is not included).
    spans = []
    for i in range(reps):
        flush.fill_(i & 0xFF)
        _, st, hz = ext.extend_attention(q, k_cache, v_cache, bt, prefix, extend, w.scale, out, lse, workspace=ws,
                                         timed=True)
        st = st.cpu().numpy()
        dsel, csel = st[:, 2] == 1, st[:, 2] == 0
        spans.append(((st[dsel, 1].max() - st[dsel, 0].min()) / hz, (st[csel, 1].max() - st[csel, 0].min()) / hz,
                      (st[:, 1].max() - st[:, 0].min()) / hz,
                      float((st[:, 5] - st[:, 4]).sum() / ((st[:, 1] - st[:, 0]).sum() / hz) / 1e9)))
    dspan, cspan, kspan, sclk = (float(np.median([x[j] for x in spans])) for j in range(4))
    chunk = [(p, e) for p, e in zip(prefix, extend) if e > 1]
    chunk_flops = sweep_flops(chunk, hq, d)
    return {
        "workload": "mixed_budget2048: 64 decode rows (context U{512..8192}) + 1984-row chunk at P=6144, "
                    "32 q / 8 kv heads, D=128, bf16, one launch",
        "timing": "GPU time per call (metadata copy + kernels), median of %d calls, host enqueued ahead" % reps,
        "ms_mixed_launch": t_mix * 1e3,
        "ms_mixed_launch_min": t_mix_min * 1e3,
        "ms_decode_rows_only": t_dec * 1e3,
        "ms_decode_rows_only_min": t_dec_min * 1e3,
        "decode_bytes": dec_bytes,
        "decode_GBps": dec_bytes / t_dec / 1e9,
        "decode_frac_hbm_peak": dec_bytes / t_dec / 1e9 / PEAK_HBM_GBS,
        "decode_span_in_mixed_ms": dspan * 1e3,
        "decode_GBps_in_mixed": dec_bytes / dspan / 1e9,
        "decode_frac_hbm_peak_in_mixed": dec_bytes / dspan / 1e9 / PEAK_HBM_GBS,
        "chunk_span_in_mixed_ms": cspan * 1e3,
        "attention_kernel_span_ms": kspan * 1e3,
        "span_note": "per-workgroup wall-clock stamps (measurement variant of the same launch), median of %d" % reps,
        "sclk_ghz_in_mixed": sclk,
        "chunk_flops": chunk_flops,
        "ms_chunk_rows_only": t_chk * 1e3,
        "chunk_tflops_alone": chunk_flops / t_chk / 1e12,
        "mixed_lower_bound_ms": max(chunk_flops / (PEAK_BF16_TFLOPS * 1e12), dec_bytes / (PEAK_HBM_GBS * 1e9)) * 1e3,
    }


def verify_rows_sweep(torch, ext, synth, reps: int = 10):
    """Multi-token verify rows (several candidate tokens per request, as in
    speculative decoding): the 64 requests of the mixed step (context L ~
    U{512..8192}, 32 or 64 q / 8 kv heads, D=128, bf16), each launched with its last E
    tokens as query rows (P = L - E) for E = 1..8. Like decode rows these are
    HBM-bound (up to G*E = 64 rows per KV head share one read of the context), so the
    figure is bytes / GPU time against the 8 TB/s peak."""
    w = synth.make_workload("mixed_budget2048")
    dev = "cuda"
    bf = torch.bfloat16
    reqs = [r for r in w.requests if r.launch[1] == 1]
    hkv, d = w.n_kv_heads, w.head_dim
    k_cache = torch.zeros((w.num_blocks, hkv, 16, d), dtype=bf, device=dev)
    v_cache = torch.zeros((w.num_blocks, hkv, d, 16), dtype=bf, device=dev)
    bt_all = w.block_table()
    ctx = [r.n_ctx for r in reqs]
    for r in reqs:
        kk = synth.device_normal((r.n_ctx, hkv, d), 6000 + r.index, 0.5, bf)
        vv = synth.device_normal((r.n_ctx, hkv, d), 7000 + r.index, 0.5, bf)
        ext.kv_append(kk, vv, k_cache, v_cache, torch.from_numpy(bt_all[r.index:r.index + 1]).to(dev), [0],
                      [r.n_ctx])
    bt = torch.from_numpy(bt_all[:len(reqs)]).to(dev)
    flush = torch.empty(512 * 2**20, dtype=torch.uint8, device=dev)
    rows = []
    for hq, e in [(h, x) for h in (32, 64) for x in range(1, 9)]:
        prefix = [L - e for L in ctx]
        extend = [e] * len(ctx)
        q = synth.device_normal((e * len(ctx), hq, d), 6900 + e, 0.5, bf)
        out = torch.empty_like(q)
        lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=dev)
        ws = torch.empty(ext.workspace_bytes(prefix, extend, hq, hkv, d, ext.EXTATTN_BF16), dtype=torch.uint8,
                         device=dev)
        torch.cuda.synchronize()
        for _ in range(100):
            flush.fill_(0x5A)
        evs = []
        for i in range(reps + 2):
            flush.fill_(i & 0xFF)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            ext.extend_attention(q, k_cache, v_cache, bt, prefix, extend, w.scale, out, lse, workspace=ws)
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        t = float(np.median([a.elapsed_time(b) * 1e-3 for a, b in evs[2:]]))
        nbytes = sum(2 * L * hkv * d * 2 + 2 * e * hq * d * 2 + 4 * e * hq + 4 * math.ceil(L / 16) for L in ctx)
        rows.append({"q_heads": hq, "E": e, "rows_per_kv_head": e * hq // hkv, "ms": t * 1e3, "bytes": nbytes,
                     "GBps": nbytes / t / 1e9, "frac_hbm_peak": nbytes / t / 1e9 / PEAK_HBM_GBS})
        log(f"verify Hq={hq} E={e}: {t * 1e3:.3f} ms, {nbytes / t / 1e9:.0f} GB/s")
    return {"workload": "64 requests, context U{512..8192} (the mixed step's decode contexts), last E tokens as "
                        "query rows, 32 or 64 q / 8 kv heads, D=128, bf16, one launch per (Hq, E)",
            "timing": "GPU time per call (metadata copy + kernels), median of %d calls, LLC flushed" % reps,
            "rows": rows}


def host_planning(ext, synth, n: int = 200):
    """Host time of planning a launch (workspace_bytes), planned afresh with the plan
    table off against a table hit, for the mixed step and the sweep's last chunk."""
    w = synth.make_workload("mixed_budget2048")
    shapes = {"mixed_budget2048": ([r.launch[0] for r in w.requests], [r.launch[1] for r in w.requests], 32, 8),
              "sweep128k_t127": ([130048], [1024], 64, 8)}
    import ctypes
    lib = ext.load_library()
    res = {}
    for name, (p, e, hq, hkv) in shapes.items():
        pa, ea = np.asarray(p, dtype=np.int32), np.asarray(e, dtype=np.int32)
        pp, ep = pa.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ea.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        out = ctypes.c_size_t()
        row = {}
        for mode, entries in (("planned_us", 0), ("table_hit_us", 256)):
            ext.plan_cache_configure(entries)
            lib.extattn_workspace_bytes(len(pa), pp, ep, hq, hkv, 128, ext.EXTATTN_BF16, ctypes.byref(out))
            t0 = time.perf_counter()
            for _ in range(n):
                lib.extattn_workspace_bytes(len(pa), pp, ep, hq, hkv, 128, ext.EXTATTN_BF16, ctypes.byref(out))
            row[mode] = (time.perf_counter() - t0) / n * 1e6
        res[name] = row
    ext.plan_cache_configure(256)
    ext.plan_cache_clear()
    res["note"] = ("one C-ABI call (ctypes) per launch shape; the attention call after sizing reuses the "
                   "record, so with the table a sized launch plans once")
    return res


def calibration(torch):
    """Reference rates on this GPU, for reading the rooflines: a vendor bf16 GEMM on
    random data (the practical matrix-core rate, which sits below the published dense
    peak when operands are random) and a plain device copy (HBM)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(77)
    n = 8192
    a = (torch.randn((n, n), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    b = (torch.randn((n, n), generator=g, device="cuda") * 0.5).to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    nb = 1 << 30
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy = 2.0 * nb * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return {"gemm_bf16_8192_random_tflops": gemm, "copy_1gib_read_plus_write_gbps": copy}


def chunk_size_sweep(torch, ext, synth, n: int = 65536, sizes=(256, 512, 1024, 2048, 4096, 8192, 16384),
                     reps: int = 3):
    """Attention TFLOP/s of one prompt of n tokens prefilled at each chunk size C
    (64 q / 8 kv heads, D=128, bf16, sweep-style inputs): the zdszero notes' claim
    that one forward's efficiency saturates past some size, measured for this
    kernel. The cache is filled once (the tokens are the same for every C);
    each chunk's attention launch is timed with HIP events, median of reps."""
    hq, hkv, d = SWEEP["hq"], SWEEP["hkv"], SWEEP["d"]
    bf = torch.bfloat16
    nb = n // 16
    q = synth.device_normal((n, hq, d), 5101, 0.5, bf)
    k_new = synth.device_normal((n, hkv, d), 5102, 0.5, bf)
    v_new = synth.device_normal((n, hkv, d), 5103, 0.5, bf)
    k_cache = torch.zeros((nb, hkv, 16, d), dtype=bf, device="cuda")
    v_cache = torch.zeros((nb, hkv, d, 16), dtype=bf, device="cuda")
    perm = np.random.default_rng(5104).permutation(nb).astype(np.int32)
    bt = torch.from_numpy(perm.reshape(1, nb)).cuda()
    ext.kv_append(k_new, v_new, k_cache, v_cache, bt, [0], [n])
    out = torch.empty_like(q)
    lse = torch.empty((n, hq), dtype=torch.float32, device="cuda")
    rows = []
    for c in sizes:
        plan = ext.chunk_plan(n, c, 0.0)["chunks"]
        ws = torch.empty(max(ext.workspace_bytes([p], [e], hq, hkv, d, ext.EXTATTN_BF16) for p, e in plan),
                         dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(reps + 1):
            evs = []
            for p, e in plan:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                ext.extend_attention(q[p:p + e], k_cache, v_cache, bt, [p], [e], 1.0 / math.sqrt(d),
                                     out[p:p + e], lse[p:p + e], workspace=ws)
                b.record()
                evs.append((a, b))
            torch.cuda.synchronize()
            times.append(sum(a.elapsed_time(b) for a, b in evs) * 1e-3)
        t = float(np.median(times[1:]))
        f = sweep_flops(plan, hq, d)
        rows.append({"chunk_size": c, "chunks": len(plan), "attention_ms": t * 1e3, "tflops": f / t / 1e12,
                     "ms_per_chunk": t * 1e3 / len(plan)})
        log(f"chunk size {c}: {len(plan)} chunks, {t * 1e3:.2f} ms, {f / t / 1e12:.0f} TFLOP/s")
    return {"workload": f"one prompt of {n} tokens, 64 q / 8 kv heads, D=128, bf16, paged block 16, permuted blocks",
            "flops": sweep_flops(ext.chunk_plan(n, sizes[0], 0.0)["chunks"], hq, d), "rows": rows}


def config_table(torch, ext, synth, reps: int = 5, compact: bool = False):
    """GPU time of the pages' single-prompt workloads (tiny fp32 64 tokens at C=16;
    a 4000-token prompt at C=512; 32768 tokens at hit rate 0.5 and C=8192): each
    planned chunk's K/V is appended, then its extend launch is timed with HIP
    events (median of reps). The mixed step and the 128k sweep are the default
    bench lines. ``compact`` leaves out the per-chunk rows."""
    out = []
    for name in ("tiny_f32", "prompt4000", "prefix_cache32k"):
        w = synth.make_workload(name)
        n, c, h = w.plan
        plan = ext.chunk_plan(n, c, h)
        hq, hkv, d = w.n_q_heads, w.n_kv_heads, w.head_dim
        dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        mult = w.mult
        q = synth.device_normal((n, hq, d), 8001, mult, dt)
        kn = synth.device_normal((n, hkv, d), 8002, mult, dt)
        vn = synth.device_normal((n, hkv, d), 8003, mult, dt)
        k_cache = torch.zeros((w.num_blocks, hkv, 16, d), dtype=dt, device="cuda")
        v_cache = torch.zeros((w.num_blocks, hkv, d, 16), dtype=dt, device="cuda")
        bt = torch.from_numpy(w.block_table()).cuda()
        out_t = torch.empty_like(q)
        lse = torch.empty((n, hq), dtype=torch.float32, device="cuda")
        cached = plan["cached"]
        if cached:
            ext.kv_append(kn[:cached], vn[:cached], k_cache, v_cache, bt, [0], [cached])
        chunks = []
        for p_, e_ in plan["chunks"]:
            ext.kv_append(kn[p_:p_ + e_], vn[p_:p_ + e_], k_cache, v_cache, bt, [p_], [e_])
            ts = []
            for _ in range(reps + 1):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                ext.extend_attention(q[p_:p_ + e_], k_cache, v_cache, bt, [p_], [e_], w.scale, out_t[p_:p_ + e_],
                                     lse[p_:p_ + e_])
                b.record()
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b) * 1e-3)
            t = float(np.median(ts[1:]))
            f = sweep_flops([(p_, e_)], hq, d)
            chunks.append({"prefix": p_, "extend": e_, "ms": t * 1e3, "tflops": f / t / 1e12})
        tot_f = sum(sweep_flops([(x["prefix"], x["extend"])], hq, d) for x in chunks)
        tot_t = sum(x["ms"] for x in chunks) * 1e-3
        row = {"workload": name, "dtype": w.dtype, "n_chunks": len(chunks), "flops": tot_f,
               "attention_ms": tot_t * 1e3, "tflops": tot_f / tot_t / 1e12}
        if not compact:
            row["chunks"] = chunks
        out.append(row)
        log(f"{name}: {len(chunks)} chunks, {tot_t * 1e3:.3f} ms, {tot_f / tot_t / 1e12:.1f} TFLOP/s")
    return out


def _oracle_rate(w, rows, n_rows: int, rng):
    """Time the CPU oracle on n_rows random rows of ``rows`` ((request, position)
    pairs, all query heads each), called once per request with all of that
    request's sampled rows (its intended use). Inputs are generated before timing.
    Returns (flops timed, seconds, rows timed)."""
    import oracle
    sample = [rows[i] for i in rng.permutation(len(rows))[:n_rows]]
    by_req = {}
    for ri, pos in sample:
        by_req.setdefault(ri, []).append(pos)
    args = []
    for ri, ps in by_req.items():
        req = w.requests[ri]
        m = max(ps) + 1
        q = np.concatenate([w.q(req, p_, p_ + 1) for p_ in ps])
        args.append((q, w.k(req, 0, m), w.v(req, 0, m), ps))
    t0 = time.perf_counter()
    for q, kk, vv, ps in args:
        oracle.attend_rows(q, kk, vv, ps, w.scale)
    dt = time.perf_counter() - t0
    f = sum(4 * w.head_dim * w.n_q_heads * (p_ + 1) for _, p_ in sample)
    return f, dt, len(sample)


def config_oracle_times(n_rows: int = 64):
    """The CPU oracle on each of the pages' five workloads (a timed random sample of
    the rows their launches compute, all heads): its rate, and its wall time for
    the whole workload extrapolated from that rate."""
    import oracle
    import synth
    rng = np.random.default_rng(1)
    res = []
    for name in ("tiny_f32", "prompt4000", "prefix_cache32k", "mixed_budget2048", "sweep128k"):
        w = synth.make_workload(name)
        if w.plan is not None:
            n, c, h = w.plan
            launches = [(0, p_, e_) for p_, e_ in oracle.chunk_plan(n, c, h)["chunks"]]
        else:
            launches = [(r.index, r.launch[0], r.launch[1]) for r in w.requests]
        total_f = sum(4 * w.head_dim * w.n_q_heads * (e_ * p_ + e_ * (e_ + 1) // 2) for _, p_, e_ in launches)
        rows = [(ri, p_ + i) for ri, p_, e_ in launches for i in range(e_)]
        f, dt, k = _oracle_rate(w, rows, n_rows, rng)
        rate = f / dt
        res.append({"workload": name, "rows_timed": k, "rows_total": len(rows), "oracle_gflops": rate / 1e9,
                    "seconds_timed": dt, "full_seconds_estimated": total_f / rate, "full": k == len(rows)})
        log(f"oracle {name}: {k}/{len(rows)} rows in {dt:.1f} s, {rate / 1e9:.2f} GFLOP/s")
    return res


def cpu_baseline(target_s: float = 15.0):
    """Time the CPU oracle on sampled rows of the sweep (chunk 64, P = 65536)."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    w = synth.make_workload("sweep128k")
    req = w.requests[0]
    p0 = 64 * 1024
    kk = w.k(req, 0, p0 + 1024)
    vv = w.v(req, 0, p0 + 1024)
    rng = np.random.default_rng(0)
    rows = p0 + rng.permutation(1024)
    qs = w.q(req, p0, p0 + 1024)
    flops = 0
    done = 0
    block = 16  # rows per oracle call (the oracle attends any set of rows in one call)
    t0 = time.perf_counter()
    for b in range(0, len(rows), block):
        pos = rows[b:b + block]
        oracle.attend_rows(qs[pos - p0], kk, vv, pos, w.scale)
        flops += sum(4 * w.head_dim * w.n_q_heads * (int(p_) + 1) for p_ in pos)
        done += len(pos)
        if time.perf_counter() - t0 > target_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} query rows (all 64 heads) of sweep chunk 64 (P=65536), {block} rows per oracle "
                      f"call, fp64 NumPy, {dt:.1f} s; affinity {len(os.sched_getaffinity(0))} cpus"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--only-mixed", action="store_true", help="run only the mixed-step measurement (for profiling)")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused append + attention steps")
    ap.add_argument("--no-tables", action="store_true", help="skip the config table and the chunk-size sweep")
    ap.add_argument("--config-table", action="store_true",
                    help="only time the pages' smaller workloads on the GPU and the oracle on all five")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="only measure attention TFLOP/s against the chunk size (one 64k prompt)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (3 launches), the reference for HBM byte counters")
    ap.add_argument("--verify-sweep", action="store_true",
                    help="only measure verify rows (E = 1..8 query rows per request) in HBM GB/s")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import chunked_prefill_attention_extend_amd as ext
    import synth

    ext.load_library()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_launch": n, "bytes_written_per_launch": n,
                                               "launches": 3}}), flush=True)
        return 0
    if args.chunk_sweep:
        print(json.dumps({"chunk_size_sweep": chunk_size_sweep(torch, ext, synth)}), flush=True)
        return 0
    if args.config_table:
        table = {"gpu": config_table(torch, ext, synth),
                 "oracle": None if args.no_cpu_baseline else config_oracle_times()}
        print(json.dumps({"config_table": table}), flush=True)
        return 0
    if args.verify_sweep:
        print(json.dumps({"verify_rows": verify_rows_sweep(torch, ext, synth)}), flush=True)
        return 0
    if args.only_mixed:
        print(json.dumps({"mixed_step": mixed_step_bench(torch, ext, synth)}), flush=True)
        return 0
    log("setting up the 128-chunk sweep")
    s = setup_sweep(torch, ext, synth)
    flops = sweep_flops(s["plan"], SWEEP["hq"], SWEEP["d"])
    nchunk = len(s["plan"])
    for i in range(args.warmup):
        sweep_step(ext, s)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    events = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(nchunk)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        sweep_step(ext, s, [list(p) for p in events[k]])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {dt:.3f} s")
    check_status(ext, s)
    kern_s = sum(a.elapsed_time(b) for step in events for a, b in step) * 1e-3 / args.steps
    per_launch_s = kern_s / nchunk
    achieved = flops / nchunk / per_launch_s / 1e12
    # per chunk: median over the timed steps
    med = [float(np.median([events[k][t][0].elapsed_time(events[k][t][1]) * 1e-3 for k in range(args.steps)]))
           for t in range(nchunk)]
    chunk_f = [sweep_flops([pe], SWEEP["hq"], SWEEP["d"]) for pe in s["plan"]]
    per_chunk = {f"t{t}": chunk_f[t] / med[t] / 1e12 for t in (0, 1, 3, 7, 15, 31, 63, 95, 127) if t < nchunk}
    aggregate = sum(chunk_f) / sum(med) / 1e12
    ms = dt / args.steps * 1e3
    value = flops / (dt / args.steps) / 1e12

    # The same steps with each chunk's append fused into its attention launch.
    fused = None
    if not args.no_fused:
        for i in range(args.warmup):
            sweep_step(ext, s, fused=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            sweep_step(ext, s, fused=True)
        torch.cuda.synchronize()
        dtf = time.perf_counter() - t0
        check_status(ext, s)
        fused = {"ms_per_step": dtf / args.steps * 1e3, "tflops": flops / (dtf / args.steps) / 1e12,
                 "note": "128 x extend_attention_append (append inside the attention launch)"}
        log(f"fused steps: {dtf / args.steps * 1e3:.1f} ms per step")

    sclk = shader_clock(torch, ext, s)
    log(f"shader clock on the last chunk: {sclk:.3f} GHz")

    mixed = None
    if not args.no_mixed:
        log("mixed step")
        mixed = mixed_step_bench(torch, ext, synth)
    verify = None
    if not args.no_mixed:
        log("verify rows")
        verify = verify_rows_sweep(torch, ext, synth)
    configs = chunk_sizes = None
    if not args.no_tables:
        log("config table")
        configs = config_table(torch, ext, synth, compact=True)
        log("chunk-size sweep")
        chunk_sizes = chunk_size_sweep(torch, ext, synth)
    log("calibration")
    calib = calibration(torch)
    planning = host_planning(ext, synth)
    base = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        base = cpu_baseline()

    line = {
        "metric": "extend-attn bf16 TFLOP/s & % MFMA peak; mixed-step decode HBM GB/s, 1 GPU",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "sweep128k: N=131072 tokens, C=1024 (128 chunks, P=1024t, E=1024), append + "
                               "extend per chunk, 64 q / 8 kv heads, D=128, bf16, paged block 16, permuted blocks",
                   "flops_per_step": flops, "chunks": nchunk},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                     "kernel": SWEEP_KERNEL,
                     "avg_launch_ms": per_launch_s * 1e3, "flops_per_launch": flops / nchunk,
                     "peak_clock_ghz": PEAK_CLOCK_GHZ, "sclk_ghz_measured": sclk,
                     "peak_at_measured_clock": PEAK_BF16_TFLOPS * sclk / PEAK_CLOCK_GHZ,
                     "clock_note": "peak = 256 CU x 4 SIMD x 1024 bf16 FLOP/clk at 2.4 GHz; sclk_ghz_measured: "
                                   "shader-clock cycles / wall-clock time of the workgroups of one timed launch "
                                   "of the last chunk"},
        "sweep_attention": {"aggregate_tflops": aggregate, "per_chunk_tflops": per_chunk,
                            "note": "attention launches only (kv_append excluded); sum(F) / sum(per-chunk median)"},
        "calibration": calib,
        "host_planning": planning,
        "fused_append_step": fused,
        "mixed_step": mixed,
        "verify_rows": verify,
        "config_table": configs,
        "chunk_size_sweep": chunk_sizes,
        "cpu_baseline": base,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
