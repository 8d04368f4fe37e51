"""Python binding of libextattn.so (argument marshalling only).

Every step of the computation runs in the HIP library; this module checks
tensor shapes and dtypes, pulls raw device pointers and the current stream
from PyTorch, and maps status codes to exceptions. If the library has not been
built it raises; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libextattn.so")

EXTATTN_OK, EXTATTN_EINVAL, EXTATTN_ENOSPC, EXTATTN_EUNSUPPORTED, EXTATTN_EHIP = 0, -1, -2, -3, -4
EXTATTN_BF16, EXTATTN_F32 = 0, 1
STATUS_BAD_BLOCK, STATUS_WAIT_TIMEOUT = 1, 2
STAMP_WORDS = 6  # per work item of a timed launch: start, end, kind, request, clk_start, clk_end
BLOCK_SIZE = 16

_lib = None

_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)


def load_library() -> ctypes.CDLL:
    """Load libextattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m chunked_prefill_attention_extend_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.extattn_last_error.restype = ctypes.c_char_p
    lib.extattn_last_error.argtypes = []
    lib.extattn_chunk_plan.restype = ctypes.c_int
    lib.extattn_chunk_plan.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_double, _c_i64p, _c_i64p,
                                       _c_i64p, _c_i64p, _c_i64p, ctypes.c_int64]
    _c_i32p_ = ctypes.POINTER(ctypes.c_int32)
    lib.extattn_token_budget_step.restype = ctypes.c_int
    lib.extattn_token_budget_step.argtypes = [ctypes.c_int32, _c_i64p, _c_i64p, ctypes.c_int32, _c_i64p, _c_i64p,
                                              ctypes.c_int64, _c_i32p_, _c_i64p, _c_i64p, ctypes.c_int32,
                                              _c_i32p_, _c_i64p]
    lib.extattn_mixed_chunk_step.restype = ctypes.c_int
    lib.extattn_mixed_chunk_step.argtypes = [ctypes.c_int32, _c_i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                             _c_i64p, _c_i64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                             _c_i32p_, _c_i32p_, _c_i64p, _c_i64p, ctypes.c_int32, _c_i32p_,
                                             _c_i64p, _c_i32p_, _c_i32p_, _c_i64p]
    lib.extattn_decode_first_with_slack.restype = ctypes.c_int
    lib.extattn_decode_first_with_slack.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                    _c_i64p, _c_i64p, _c_i64p]
    lib.extattn_workspace_bytes.restype = ctypes.c_int
    lib.extattn_workspace_bytes.argtypes = [ctypes.c_int32, _c_i32p, _c_i32p, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.extattn_kv_append_workspace_bytes.restype = ctypes.c_size_t
    lib.extattn_kv_append_workspace_bytes.argtypes = [ctypes.c_int32]
    lib.extattn_kv_append.restype = ctypes.c_int
    lib.extattn_kv_append.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, _c_i32p, _c_i32p,
                                      ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.extattn_extend_attention.restype = ctypes.c_int
    lib.extattn_extend_attention.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_int32, ctypes.c_int64, _c_i32p, _c_i32p, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_float, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.extattn_extend_attention_append.restype = ctypes.c_int
    lib.extattn_extend_attention_append.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                    *lib.extattn_extend_attention.argtypes[1:]]
    lib.extattn_extend_attention_timed.restype = ctypes.c_int
    lib.extattn_extend_attention_timed.argtypes = [*lib.extattn_extend_attention.argtypes, ctypes.c_void_p,
                                                   ctypes.c_int32, _c_i32p, ctypes.POINTER(ctypes.c_double)]
    lib.extattn_plan_cache_configure.restype = ctypes.c_int
    lib.extattn_plan_cache_configure.argtypes = [ctypes.c_int32, ctypes.c_int64]
    lib.extattn_plan_cache_stats.restype = ctypes.c_int
    lib.extattn_plan_cache_stats.argtypes = [_c_i64p, _c_i64p, _c_i32p, _c_i64p]
    lib.extattn_plan_cache_clear.restype = ctypes.c_int
    lib.extattn_plan_cache_clear.argtypes = []
    lib.extattn_extend_attention_noalloc.restype = ctypes.c_int
    lib.extattn_extend_attention_noalloc.argtypes = [*lib.extattn_extend_attention.argtypes[:17], ctypes.c_void_p]
    lib.extattn_read_status.restype = ctypes.c_int
    lib.extattn_read_status.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32), _c_i32p, _c_i32p,
                                        ctypes.c_void_p]
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc == EXTATTN_OK:
        return
    msg = load_library().extattn_last_error().decode(errors="replace")
    if rc == EXTATTN_EHIP:
        raise RuntimeError(f"extattn HIP failure: {msg}")
    kind = {EXTATTN_EINVAL: "invalid argument", EXTATTN_ENOSPC: "insufficient space",
            EXTATTN_EUNSUPPORTED: "unsupported"}.get(rc, f"status {rc}")
    raise ValueError(f"extattn {kind}: {msg}")


def status_error(flags: int, bad_block_reads: int, what: str = "launch"):
    """The exception that a non-zero status stands for, or None."""
    if flags & STATUS_WAIT_TIMEOUT:
        return RuntimeError(f"extattn {what}: a fused-append wait gave up; the results are not valid")
    if flags & STATUS_BAD_BLOCK:
        return ValueError(f"extattn {what}: {bad_block_reads} read(s) of a block id outside [0, num_blocks); "
                          "the results are not valid")
    if flags:
        return RuntimeError(f"extattn {what}: unknown status flags {flags:#x}")
    return None


_last_status = (0, 0, 0)


def read_status(workspace, stream=None) -> tuple[int, int, int]:
    """``(flags, bad_block_reads, exact_waves)`` left in ``workspace`` by the last
    call that used it (waits for ``stream``, default torch's current stream);
    ``workspace=None`` reads the allocation-free entry point's scratch."""
    global _last_status
    flags, count, exact = ctypes.c_uint32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    ws = workspace.data_ptr() if workspace is not None else None
    _check(load_library().extattn_read_status(ws, ctypes.byref(flags), ctypes.byref(count), ctypes.byref(exact),
                                              _stream_handle(stream)))
    _last_status = (flags.value, count.value, exact.value)
    return _last_status


def last_status() -> tuple[int, int, int]:
    """The status words of the most recent ``read_status`` (also the one a
    ``check=True`` call makes)."""
    return _last_status


def _raise_on_status(ws, stream, what: str) -> None:
    flags, count, _ = read_status(ws, stream)
    err = status_error(flags, count, what)
    if err is not None:
        raise err


def _host_i32(x: Sequence[int]) -> np.ndarray:
    if hasattr(x, "detach"):
        if x.is_cuda:
            raise ValueError("prefix_lens / extend_lens must be host (CPU) values")
        x = x.detach().numpy()
    arr = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    if arr.ndim != 1:
        raise ValueError("length arrays must be one-dimensional")
    if arr.size and (arr.min() < -2**31 or arr.max() > 2**31 - 1):
        raise ValueError("lengths must fit int32")
    return np.ascontiguousarray(arr.astype(np.int32))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_c_i32p)


def chunk_plan(n_tokens: int, chunk_size: int, hit_rate: float = 0.0) -> dict:
    """Chunk plan of one prompt: ``{"cached", "effective", "chunks": [(P_t, E_t), ...]}``."""
    lib = load_library()
    cached, eff, k = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    rc = lib.extattn_chunk_plan(int(n_tokens), int(chunk_size), float(hit_rate), ctypes.byref(cached),
                                ctypes.byref(eff), ctypes.byref(k), None, None, 0)
    if rc != EXTATTN_ENOSPC and rc != EXTATTN_OK:
        _check(rc)
    n = k.value
    p = np.zeros(max(n, 1), np.int64)
    e = np.zeros(max(n, 1), np.int64)
    _check(lib.extattn_chunk_plan(int(n_tokens), int(chunk_size), float(hit_rate), ctypes.byref(cached),
                                  ctypes.byref(eff), ctypes.byref(k), p.ctypes.data_as(_c_i64p),
                                  e.ctypes.data_as(_c_i64p), n))
    return {"cached": cached.value, "effective": eff.value,
            "chunks": [(int(p[t]), int(e[t])) for t in range(n)]}


def _i64(values) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(list(values), dtype=np.int64))
    return a if a.size else np.zeros(1, np.int64)


def token_budget_step(running, waiting, budget: int):
    """One mixed step under a token budget (see ``extattn_token_budget_step``).

    running: [(total_tokens, computed)], waiting: [(total_tokens, cached)].
    Returns ``(entries, budget_left)`` with entries ``(kind, index, prefix, extend)``,
    kind ``"running"`` or ``"waiting"``, in scheduling order."""
    lib = load_library()
    running, waiting = list(running), list(waiting)
    rt, rc_ = _i64(t for t, _ in running), _i64(c for _, c in running)
    wt, wc = _i64(t for t, _ in waiting), _i64(c for _, c in waiting)
    cap = len(running) + len(waiting)
    idx = np.zeros(max(cap, 1), np.int32)
    pre = np.zeros(max(cap, 1), np.int64)
    ext = np.zeros(max(cap, 1), np.int64)
    n, left = ctypes.c_int32(), ctypes.c_int64()
    _check(lib.extattn_token_budget_step(len(running), rt.ctypes.data_as(_c_i64p), rc_.ctypes.data_as(_c_i64p),
                                         len(waiting), wt.ctypes.data_as(_c_i64p), wc.ctypes.data_as(_c_i64p),
                                         int(budget), idx.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         pre.ctypes.data_as(_c_i64p), ext.ctypes.data_as(_c_i64p), cap,
                                         ctypes.byref(n), ctypes.byref(left)))
    out = []
    for k in range(n.value):
        i = int(idx[k])
        kind, j = ("running", i) if i < len(running) else ("waiting", i - len(running))
        out.append((kind, j, int(pre[k]), int(ext[k])))
    return out, left.value


_KINDS = {0: "decode", 1: "chunked", 2: "waiting"}


def mixed_chunk_step(decode_prefix, chunked, waiting, chunk_size: int, page_size: int = 1, mixed: bool = True):
    """One round of the mixed-chunk scheduler (see ``extattn_mixed_chunk_step``).

    decode_prefix: cached tokens of each decode row; chunked: None or (total, done);
    waiting: [(total_tokens, cached)]. Returns ``(entries, chunk_left, next_chunked)``:
    entries ``(kind, index, prefix, extend)``, kind "decode" | "chunked" | "waiting";
    next_chunked None or ``(kind, index, total, done)``."""
    lib = load_library()
    decode_prefix, waiting = list(decode_prefix), list(waiting)
    dp = _i64(decode_prefix)
    wt, wc = _i64(t for t, _ in waiting), _i64(c for _, c in waiting)
    ct, cd = (int(chunked[0]), int(chunked[1])) if chunked is not None else (0, 0)
    cap = len(decode_prefix) + 1 + len(waiting)
    i32p = ctypes.POINTER(ctypes.c_int32)
    kinds, idx = np.zeros(cap, np.int32), np.zeros(cap, np.int32)
    pre, ext = np.zeros(cap, np.int64), np.zeros(cap, np.int64)
    n, left, nk, ni, nd = ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib.extattn_mixed_chunk_step(len(decode_prefix), dp.ctypes.data_as(_c_i64p), ct, cd, len(waiting),
                                        wt.ctypes.data_as(_c_i64p), wc.ctypes.data_as(_c_i64p), int(chunk_size),
                                        int(page_size), 1 if mixed else 0, kinds.ctypes.data_as(i32p),
                                        idx.ctypes.data_as(i32p), pre.ctypes.data_as(_c_i64p),
                                        ext.ctypes.data_as(_c_i64p), cap, ctypes.byref(n), ctypes.byref(left),
                                        ctypes.byref(nk), ctypes.byref(ni), ctypes.byref(nd)))
    entries = [(_KINDS[int(kinds[k])], int(idx[k]), int(pre[k]), int(ext[k])) for k in range(n.value)]
    nxt = None
    if nk.value >= 0:
        total = ct if nk.value == 1 else int(waiting[ni.value][0])
        nxt = (_KINDS[nk.value], ni.value, total, nd.value)
    return entries, left.value, nxt


def decode_first_with_slack(ready_decode: int, pending_prefill: int, chunk_query_len: int,
                            max_batched_tokens: int):
    """``(p_step, d_step, limit)`` of the default mixed-step scheduler."""
    lib = load_library()
    p, d, lim = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib.extattn_decode_first_with_slack(int(ready_decode), int(pending_prefill), int(chunk_query_len),
                                               int(max_batched_tokens), ctypes.byref(p), ctypes.byref(d),
                                               ctypes.byref(lim)))
    return p.value, d.value, lim.value


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return EXTATTN_BF16
    if t.dtype == torch.float32:
        return EXTATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def workspace_bytes(prefix_lens, extend_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    dtype_code: int) -> int:
    lib = load_library()
    p, e = _host_i32(prefix_lens), _host_i32(extend_lens)
    if p.shape != e.shape:
        raise ValueError("prefix_lens and extend_lens differ in length")
    out = ctypes.c_size_t()
    _check(lib.extattn_workspace_bytes(len(p), _ptr(p), _ptr(e), num_q_heads, num_kv_heads, head_dim,
                                       dtype_code, ctypes.byref(out)))
    return out.value


def plan_cache_configure(max_entries: int, max_bytes: int = 64 << 20) -> None:
    """Bound the library's launch-plan table (0 entries turns it off)."""
    _check(load_library().extattn_plan_cache_configure(int(max_entries), int(max_bytes)))


def plan_cache_stats() -> dict:
    """Hits and misses since the last clear, records held and their host bytes."""
    h, m, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    n = ctypes.c_int32()
    _check(load_library().extattn_plan_cache_stats(ctypes.byref(h), ctypes.byref(m), ctypes.byref(n),
                                                   ctypes.byref(b)))
    return {"hits": h.value, "misses": m.value, "entries": n.value, "bytes": b.value}


def plan_cache_clear() -> None:
    """Drop every launch-plan record and zero the counters."""
    _check(load_library().extattn_plan_cache_clear())


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _check_cache(k_cache, v_cache, block_table):
    import torch
    if k_cache.dim() != 4 or v_cache.dim() != 4:
        raise ValueError("k_cache must be [num_blocks, Hkv, block, D] and v_cache [num_blocks, Hkv, D, block]")
    nb, hkv, bs, d = k_cache.shape
    if tuple(v_cache.shape) != (nb, hkv, d, bs):
        raise ValueError("v_cache must be [num_blocks, Hkv, D, block] (slot-minor)")
    if not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("caches must be contiguous")
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [num_seqs, max_blocks] tensor")
    if not (k_cache.is_cuda and v_cache.is_cuda and block_table.is_cuda):
        raise ValueError("caches and block_table must be device tensors")
    return nb, hkv, bs, d


def _workspace(nbytes: int, device, workspace, stream=None):
    """The caller's workspace, or a new one. A new one must stay referenced until
    every launch that uses it has been enqueued: once freed, torch's caching
    allocator may hand its memory to the next allocation (it did to the stamp
    buffer of a timed launch, whose stamps then overwrote the zero page). On a
    stream other than torch's current one it is also marked as in use there, so
    that the allocator waits for that stream's work before reusing it."""
    import torch
    if workspace is None:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        if stream is not None:
            ws.record_stream(stream)
        return ws
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError("workspace too small")
    return workspace


def kv_append(k_new, v_new, k_cache, v_cache, block_table, prefix_lens, extend_lens,
              workspace=None, stream=None, check: bool = False) -> None:
    """Write each request's new K/V rows ``[sum(E), Hkv, D]`` into the paged cache.
    With ``check`` the call waits for the stream and raises if a block id was
    outside ``[0, num_blocks)``."""
    lib = load_library()
    nb, hkv, bs, d = _check_cache(k_cache, v_cache, block_table)
    p, e = _host_i32(prefix_lens), _host_i32(extend_lens)
    if p.shape != e.shape or len(p) != block_table.shape[0]:
        raise ValueError("length arrays must have one entry per block_table row")
    total = int(e.sum())
    for t in (k_new, v_new):
        if tuple(t.shape) != (total, hkv, d) or t.dtype != k_cache.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError("k_new / v_new must be contiguous device tensors [sum(E), Hkv, D] of the cache dtype")
    need = lib.extattn_kv_append_workspace_bytes(len(p))
    ws = _workspace(need, k_cache.device, workspace, stream)
    _check(lib.extattn_kv_append(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                 block_table.data_ptr(), block_table.shape[1], nb, _ptr(p), _ptr(e), len(p),
                                 hkv, d, bs, _dtype_code(k_cache), ws.data_ptr(),
                                 ws.numel() * ws.element_size(), _stream_handle(stream)))
    if check:
        _raise_on_status(ws, stream, "kv_append")


_NO_WORKSPACE = object()  # marks the allocation-free call in _extend_args


def _extend_args(q, k_cache, v_cache, block_table, prefix_lens, extend_lens, scale, out, lse, workspace, stream):
    """Checks shared by the extend-attention entry points; returns (lib, p, e, hkv, d, ws, args).
    The caller holds ``ws`` (the workspace, maybe allocated here) until its launches are enqueued."""
    import torch
    lib = load_library()
    nb, hkv, bs, d = _check_cache(k_cache, v_cache, block_table)
    p, e = _host_i32(prefix_lens), _host_i32(extend_lens)
    if p.shape != e.shape or len(p) != block_table.shape[0]:
        raise ValueError("length arrays must have one entry per block_table row")
    total = int(e.sum())
    if q.dim() != 3 or q.shape[0] != total or q.shape[2] != d:
        raise ValueError("q must be [sum(E), Hq, D]")
    hq = q.shape[1]
    if q.dtype != k_cache.dtype or not q.is_contiguous() or not q.is_cuda:
        raise ValueError("q must be a contiguous device tensor of the cache dtype")
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must match q")
    if lse is not None and (tuple(lse.shape) != (total, hq) or lse.dtype != torch.float32
                            or not lse.is_contiguous()):
        raise ValueError("lse must be a contiguous float32 [sum(E), Hq] tensor")
    code = _dtype_code(q)
    if workspace is _NO_WORKSPACE:  # the allocation-free entry point: nothing is allocated here either
        ws = None
    elif workspace is None:
        ws = _workspace(workspace_bytes(p, e, hq, hkv, d, code), q.device, None, stream)
    else:  # the library checks the size itself (EXTATTN_ENOSPC): no second planning pass here
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or not workspace.is_cuda:
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        ws = workspace
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(), block_table.shape[1], nb,
            _ptr(p), _ptr(e), len(p), hq, hkv, d, bs, float(scale), code, out.data_ptr(),
            lse.data_ptr() if lse is not None else None, ws.data_ptr() if ws is not None else None,
            ws.numel() * ws.element_size() if ws is not None else 0, _stream_handle(stream))
    return lib, p, e, hkv, d, ws, args


def extend_attention(q, k_cache, v_cache, block_table, prefix_lens, extend_lens, scale: float, out,
                     lse=None, workspace=None, stream=None, timed: bool = False, check: bool = False):
    """Chunked-prefill extend attention over the paged cache.

    q, out: device ``[sum(E), Hq, D]``; lse: device float32 ``[sum(E), Hq]`` or None;
    prefix_lens / extend_lens: host, one entry per block_table row.
    Returns ``out``; with ``timed`` (bf16 only) the measurement variant runs and
    ``(out, stamps, tick_hz)`` is returned, ``stamps`` a device int64 ``[items, 6]``
    of {start, end, kind (0 chunk, 1 decode / verify), request, clk_start, clk_end}
    per work item (start / end in wall-clock ticks, clk in shader-clock cycles).
    With ``check`` the call waits for the stream and raises if the launch met a
    block id outside ``[0, num_blocks)`` (``ValueError``). Without it the status
    stays in the workspace (``read_status``); a workspace allocated here is
    dropped with it.
    """
    import torch
    lib, p, e, _, _, ws, args = _extend_args(q, k_cache, v_cache, block_table, prefix_lens, extend_lens, scale,
                                             out, lse, workspace, stream)
    if not timed:
        _check(lib.extattn_extend_attention(*args))
        if check:
            _raise_on_status(ws, stream, "extend_attention")
        return out
    n = ctypes.c_int32(0)
    hz = ctypes.c_double(0.0)
    rc = lib.extattn_extend_attention_timed(*args, None, 0, ctypes.byref(n), ctypes.byref(hz))
    if rc != EXTATTN_ENOSPC or n.value < 1:
        _check(rc)
        raise RuntimeError("timed launch: no work items")
    stamps = torch.empty((n.value, STAMP_WORDS), dtype=torch.int64, device=q.device)
    _check(lib.extattn_extend_attention_timed(*args, stamps.data_ptr(), n.value, ctypes.byref(n), ctypes.byref(hz)))
    if check:
        _raise_on_status(ws, stream, "extend_attention (timed)")
    del ws, p, e  # enqueued: stream order now protects the workspace
    return out, stamps, hz.value


def extend_attention_append(q, k_new, v_new, k_cache, v_cache, block_table, prefix_lens, extend_lens,
                            scale: float, out, lse=None, workspace=None, stream=None, check: bool = True):
    """KV append fused into the extend launch: writes k_new / v_new (device
    ``[sum(E), Hkv, D]``) into the paged cache at positions prefix + t and computes
    the same attention as ``extend_attention``, in one attention launch. Returns ``out``.

    ``check`` (default on) waits for the stream and raises if the launch's wait for
    its appends gave up (``RuntimeError``) or a block id was outside
    ``[0, num_blocks)`` (``ValueError``). A caller that turns it off to keep the
    host ahead of the GPU passes its own ``workspace`` and calls ``read_status``
    on it later."""
    lib, p, e, hkv, d, ws, args = _extend_args(q, k_cache, v_cache, block_table, prefix_lens, extend_lens, scale,
                                               out, lse, workspace, stream)
    total = int(e.sum())
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (total, hkv, d) or t.dtype != q.dtype or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous device [sum(E), Hkv, D] tensor of q's dtype")
    _check(lib.extattn_extend_attention_append(args[0], k_new.data_ptr(), v_new.data_ptr(), *args[1:]))
    if check:
        _raise_on_status(ws, stream, "extend_attention_append")
    return out


def extend_attention_noalloc(q, k_cache, v_cache, block_table, prefix_lens, extend_lens, scale: float, out,
                             lse=None, stream=None, check: bool = False):
    """``extend_attention`` through the allocation-free entry point: the library's
    static 64 MiB device scratch is the workspace, so nothing is allocated (calls on
    one GPU share it and must not overlap). Returns ``out``."""
    lib, p, e, _, _, ws, args = _extend_args(q, k_cache, v_cache, block_table, prefix_lens, extend_lens, scale,
                                             out, lse, _NO_WORKSPACE, stream)
    _check(lib.extattn_extend_attention_noalloc(*args[:17], args[19]))
    if check:
        _raise_on_status(None, stream, "extend_attention_noalloc")
    return out
