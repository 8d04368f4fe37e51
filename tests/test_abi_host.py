"""The C-ABI library on the host (no GPU needed).

* The library loads and exports every function the public header declares.
* The chunk plan is bit-exact against the oracle on the pages' examples and
  on random (N, C, hit rate) triples.
* Argument checks return the documented status before anything is enqueued.
"""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import chunked_prefill_attention_extend_amd as ext
from chunked_prefill_attention_extend_amd import binding as B
import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "extattn.h")


def test_library_exports_every_declared_symbol():
    lib = ext.load_library()
    declared = set(re.findall(r"\b(extattn_\w+)\s*\(", open(HEADER).read()))
    assert declared >= {"extattn_chunk_plan", "extattn_extend_attention", "extattn_kv_append",
                        "extattn_workspace_bytes", "extattn_last_error"}
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} not exported"


def test_chunk_plan_page_examples():
    for n, c, h in [(4000, 512, 0.0), (32768, 8192, 0.5), (131072, 1024, 0.0), (4096, 8192, 0.0),
                    (32768, 8192, 0.0), (10000, 4096, 0.0), (1024, 128, 0.0), (64, 16, 0.0)]:
        assert ext.chunk_plan(n, c, h) == oracle.chunk_plan(n, c, h)


def test_chunk_plan_random_bit_exact():
    rng = random.Random(5)
    for _ in range(10000):
        n = rng.randint(1, 2_000_000)
        c = rng.randint(1, 50_000)
        h = rng.choice([0.0, 1.0 - 1e-9, rng.random(), round(rng.random(), 2)])
        try:
            want = oracle.chunk_plan(n, c, h)
        except ValueError:
            with pytest.raises(ValueError):
                ext.chunk_plan(n, c, h)
            continue
        assert ext.chunk_plan(n, c, h) == want, (n, c, h)


def test_chunk_plan_double_rounding_case():
    assert ext.chunk_plan(10, 4, 0.7)["cached"] == 7
    assert ext.chunk_plan(100, 50, 0.29)["cached"] == 28


@pytest.mark.parametrize("args", [(0, 16, 0.0), (10, 0, 0.0), (10, -1, 0.0), (10, 4, float("nan")),
                                  (10, 4, -0.5), (10, 4, 1.5), (10, 4, 1.0)])
def test_chunk_plan_errors(args):
    with pytest.raises(ValueError):
        ext.chunk_plan(*args)


def test_chunk_plan_capacity():
    lib = ext.load_library()
    c, e, k = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    p = np.zeros(3, np.int64)
    x = np.zeros(3, np.int64)
    rc = lib.extattn_chunk_plan(4000, 512, 0.0, ctypes.byref(c), ctypes.byref(e), ctypes.byref(k),
                                p.ctypes.data_as(B._c_i64p), x.ctypes.data_as(B._c_i64p), 3)
    assert rc == B.EXTATTN_ENOSPC and k.value == 8
    assert b"capacity" in lib.extattn_last_error()


def _i32(xs):
    a = np.asarray(xs, dtype=np.int32)
    return a, a.ctypes.data_as(B._c_i32p)


FAKE = 0x10000  # never dereferenced: every call below fails its argument checks


@pytest.mark.parametrize("kw,code", [
    (dict(num_seqs=0), B.EXTATTN_EINVAL),
    (dict(extend=[0]), B.EXTATTN_EINVAL),
    (dict(prefix=[-1]), B.EXTATTN_EINVAL),
    (dict(hq=6, hkv=4), B.EXTATTN_EINVAL),
    (dict(d=96), B.EXTATTN_EUNSUPPORTED),
    (dict(block_size=32), B.EXTATTN_EUNSUPPORTED),
    (dict(dtype=7), B.EXTATTN_EUNSUPPORTED),
    (dict(max_blocks=1), B.EXTATTN_EINVAL),
    (dict(scale=float("inf")), B.EXTATTN_EINVAL),
    (dict(scale=0.0), B.EXTATTN_EINVAL),
    (dict(q=0), B.EXTATTN_EINVAL),
    (dict(ws_bytes=16), B.EXTATTN_ENOSPC),
    (dict(ws=FAKE + 8), B.EXTATTN_EINVAL),
])
def test_extend_attention_argument_errors(kw, code):
    lib = ext.load_library()
    prefix, pp = _i32(kw.get("prefix", [20]))
    extend, ep = _i32(kw.get("extend", [12]))
    rc = lib.extattn_extend_attention(
        kw.get("q", FAKE), FAKE, FAKE, FAKE, kw.get("max_blocks", 4), 100, pp, ep, kw.get("num_seqs", 1),
        kw.get("hq", 8), kw.get("hkv", 2), kw.get("d", 128), kw.get("block_size", 16),
        kw.get("scale", 0.125), kw.get("dtype", 0), FAKE, None, kw.get("ws", FAKE),
        kw.get("ws_bytes", 1 << 30), None)
    assert rc == code
    assert lib.extattn_last_error()


def test_workspace_bytes_grows_with_decode_rows():
    small = ext.workspace_bytes([100], [1], 32, 8, 128, ext.EXTATTN_BF16)
    big = ext.workspace_bytes([100, 50000], [1, 1], 32, 8, 128, ext.EXTATTN_BF16)
    assert big > small > 0


def test_kv_append_argument_errors():
    lib = ext.load_library()
    prefix, pp = _i32([0])
    extend, ep = _i32([40])
    # request needs 3 blocks, table has 2
    rc = lib.extattn_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, pp, ep, 1, 8, 128, 16, 0, FAKE, 1 << 20, None)
    assert rc == B.EXTATTN_EINVAL
    rc = lib.extattn_kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 10, pp, ep, 1, 8, 128, 16, 0, FAKE, 8, None)
    assert rc == B.EXTATTN_ENOSPC


def test_binding_rejects_device_lengths_and_bad_shapes():
    import torch
    with pytest.raises(ValueError):
        B._host_i32(np.zeros((2, 2)))
    with pytest.raises(ValueError):
        ext.workspace_bytes([1, 2], [1], 8, 8, 128, 0)
    assert B._host_i32(torch.tensor([1, 2, 3])).tolist() == [1, 2, 3]


@pytest.fixture
def fresh_plan_cache():
    ext.plan_cache_clear()
    ext.plan_cache_configure(256, 64 << 20)
    yield
    ext.plan_cache_configure(256, 64 << 20)
    ext.plan_cache_clear()


def test_plan_cache_through_the_abi(fresh_plan_cache):
    """Sizing a workspace plans once per shape; the table's bounds and counters."""
    mixed = ([100, 2000, 5], [1, 300, 1])
    size = ext.workspace_bytes(*mixed, 32, 8, 128, ext.EXTATTN_BF16)
    assert ext.plan_cache_stats()["misses"] == 1 and ext.plan_cache_stats()["entries"] == 1
    assert ext.workspace_bytes(*mixed, 32, 8, 128, ext.EXTATTN_BF16) == size
    st = ext.plan_cache_stats()
    assert st["hits"] == 1 and st["misses"] == 1 and st["bytes"] > 0
    ext.workspace_bytes([100, 2000, 5], [1, 301, 1], 32, 8, 128, ext.EXTATTN_BF16)
    ext.workspace_bytes(*mixed, 64, 8, 128, ext.EXTATTN_BF16)
    assert ext.plan_cache_stats()["misses"] == 3
    # off: same sizes, nothing kept
    ext.plan_cache_configure(0)
    assert ext.plan_cache_stats()["entries"] == 0
    assert ext.workspace_bytes(*mixed, 32, 8, 128, ext.EXTATTN_BF16) == size
    assert ext.plan_cache_stats()["entries"] == 0
    with pytest.raises(ValueError):
        ext.plan_cache_configure(-1)
    lib = ext.load_library()
    assert lib.extattn_plan_cache_stats(None, None, None, None) == B.EXTATTN_EINVAL
    ext.plan_cache_clear()
    assert ext.plan_cache_stats() == {"hits": 0, "misses": 0, "entries": 0, "bytes": 0}


def test_plan_cache_many_threads_same_sizes(fresh_plan_cache):
    """Concurrent sizing calls (ctypes drops the GIL) through a table smaller than the
    set of shapes return what a cold, single-threaded call returns."""
    import threading
    rng = random.Random(11)
    shapes = []
    for i in range(20):
        n = rng.randint(1, 8)
        shapes.append(([rng.randint(0, 9000) + (i if j == 0 else 0) for j in range(n)],
                       [rng.choice([1, 1, 3, 700]) for _ in range(n)]))
    ext.plan_cache_configure(0)
    want = [ext.workspace_bytes(p, e, 32, 8, 128, ext.EXTATTN_BF16) for p, e in shapes]
    ext.plan_cache_configure(6)
    ext.plan_cache_clear()
    bad = []

    def worker(seed):
        r = random.Random(seed)
        for _ in range(200):
            i = r.randrange(len(shapes))
            if ext.workspace_bytes(*shapes[i], 32, 8, 128, ext.EXTATTN_BF16) != want[i]:
                bad.append(i)

    th = [threading.Thread(target=worker, args=(s,)) for s in range(6)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not bad
    st = ext.plan_cache_stats()
    assert st["hits"] + st["misses"] == 1200 and st["entries"] <= 6
