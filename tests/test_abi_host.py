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
