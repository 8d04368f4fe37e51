"""Pins for the oracle's chunk plan (CPU only).

The printed examples in tests/golden/chunk_plan_examples.txt come from the
pages (each line names its page and section). The closed form of the zdszero
notes (section "prefill as several resumable extends": P_t = min(tC, N),
E_t = min(C, N - P_t), ceil(N/C) rounds) is checked against the oracle's cursor
walk on random inputs, and the floor of the hit-rate product is checked against
exact rational arithmetic rounded once to double.
"""
import math
import os
import random
from fractions import Fraction

import pytest

from oracle import chunk_plan, effective_length

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "chunk_plan_examples.txt")


def _golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        args, exp, src = [x.strip() for x in line.split("|")]
        n, c, h = args.split()
        cached, eff, k, lens = exp.split()
        ext = []
        for part in lens.split(","):
            if "*" in part:
                val, rep = part.split("*")
                ext += [int(val)] * int(rep)
            else:
                ext.append(int(part))
        rows.append((int(n), int(c), float(h), int(cached), int(eff), int(k), ext, src))
    return rows


@pytest.mark.parametrize("row", _golden(), ids=lambda r: f"{r[0]}@{r[1]}h{r[2]}")
def test_printed_examples(row):
    n, c, h, cached, eff, k, ext, _src = row
    plan = chunk_plan(n, c, h)
    assert plan["cached"] == cached
    assert plan["effective"] == eff
    assert len(plan["chunks"]) == k
    assert [e for _, e in plan["chunks"]] == ext
    # the cursor starts at the cached prefix and advances by each chunk
    assert plan["chunks"][0][0] == cached
    for (p0, e0), (p1, _) in zip(plan["chunks"], plan["chunks"][1:]):
        assert p1 == p0 + e0


def test_sweep_seq_lens_printed():
    # latency-table RFC, section 1.2: (query_len=1k, seq_len=1k), (1k, 2k), ..., (1k, 128k)
    plan = chunk_plan(131072, 1024, 0.0)
    assert [p + e for p, e in plan["chunks"]] == [1024 * (t + 1) for t in range(128)]
    assert all(e == 1024 for _, e in plan["chunks"])


def test_prefix_cache_prefixes():
    # kernel-space prefixes for the 32768 / 0.5 / 8192 example: the cached 16384 tokens come first
    assert chunk_plan(32768, 8192, 0.5)["chunks"] == [(16384, 8192), (24576, 8192)]


def test_single_chunk_when_effective_fits():
    # chunked-prefill RFC, section 1.3 / 3.1.2: effective <= budget keeps one chunk equal to the full prefill
    for n in (1, 2, 100, 8191, 8192):
        assert chunk_plan(n, 8192, 0.0)["chunks"] == [(0, n)]


def test_closed_form_agrees_with_cursor_walk():
    rng = random.Random(7)
    for _ in range(3000):
        n = rng.randint(1, 300000)
        c = rng.randint(1, 20000)
        plan = chunk_plan(n, c, 0.0)
        rounds = -(-n // c)
        expect = []
        for t in range(rounds):
            p = min(t * c, n)
            expect.append((p, min(c, n - p)))
        assert plan["chunks"] == expect
        assert sum(e for _, e in plan["chunks"]) == n
        assert all(e == c for _, e in plan["chunks"][:-1]) and 1 <= plan["chunks"][-1][1] <= c


def test_floor_of_hit_rate_product_is_one_double_multiply():
    # A double multiply rounds the exact product of the two doubles once to nearest.
    # 10 * 0.7: the exact product lies 2^-51 below 7, exactly half-way between two
    # doubles, and rounds to 7.0 (ties to even); the exact real floor would be 6.
    exact = Fraction(10) * Fraction(0.7)
    assert math.floor(exact) == 6
    assert math.floor(float(exact)) == 7
    assert effective_length(10, 0.7) == (7, 3)
    assert effective_length(100, 0.29) == (28, 72)
    rng = random.Random(11)
    for _ in range(5000):
        n = rng.randint(1, 10 ** 7)
        h = rng.random()
        want = math.floor(float(Fraction(n) * Fraction(h)))
        if n - want < 1:
            continue
        assert effective_length(n, h)[0] == want


@pytest.mark.parametrize("args", [(0, 16, 0.0), (-1, 16, 0.0), (10, 0, 0.0), (10, -5, 0.0),
                                  (10, 4, float("nan")), (10, 4, -0.1), (10, 4, 1.5), (10, 4, 1.0),
                                  (1, 1, 1.0)])
def test_invalid_arguments_raise(args):
    # chunked-prefill RFC, section 2.4: a non-positive budget is rejected at the entry;
    # an effective length below 1 is an error as well.
    with pytest.raises(ValueError):
        chunk_plan(*args)
