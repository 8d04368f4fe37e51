"""Pins of the mixed-step planning oracle (oracle/budget.py): the pages' worked
examples (tests/golden/budget_examples.jsonl, each line cited) and invariants
that hold for any queue."""
import json
import os
import random
from fractions import Fraction

import pytest

import oracle.budget as ob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "budget_examples.jsonl")


def golden():
    with open(GOLDEN) as f:
        return [json.loads(line) for line in f if line.strip()]


@pytest.mark.parametrize("ex", golden(), ids=lambda e: e["policy"])
def test_golden_examples(ex):
    pol = ex["policy"]
    if pol == "token_budget":
        entries, left = ob.token_budget_step([tuple(r) for r in ex["running"]], [tuple(w) for w in ex["waiting"]],
                                             ex["budget"])
        assert [e[3] for e in entries] == ex["expect_extend"]
        assert left == ex["expect_left"]
    elif pol == "mixed_chunk":
        entries, left, nc = ob.mixed_chunk_step(ex["decode"], tuple(ex["chunked"]) if ex["chunked"] else None,
                                                [tuple(w) for w in ex["waiting"]], ex["chunk_size"],
                                                ex["page_size"], ex["mixed"])
        assert left == ex["expect_left"]
        if "expect_entries" in ex:
            assert [list(e) for e in entries] == ex["expect_entries"]
            assert (list(nc) if nc else None) == ex["expect_new_chunked"]
        if "expect_chunk_extend" in ex:
            assert [e[3] for e in entries if e[0] == "chunked"] == [ex["expect_chunk_extend"]]
            assert sum(1 for e in entries if e[0] == "decode") == len(ex["decode"])
    elif pol == "decode_first":
        p, d = ob.decode_first_with_slack(ex["ready_decode"], ex["pending_prefill"], ex["chunk_query_len"],
                                          ex["max_batched_tokens"])
        assert (p, d) == (ex["expect_p"], ex["expect_d"])
        assert ob.slack_limit(ex["max_batched_tokens"]) == ex["expect_limit"]
    elif pol == "slack_limit":
        assert ob.slack_limit(ex["max_batched_tokens"]) == ex["expect_limit"]
    else:
        raise AssertionError(pol)


def test_slack_limit_against_exact_rounding():
    # the double product is within one unit of the exact rational product, and equal
    # to it whenever B * 1.15 is exactly representable after rounding
    for b in range(1, 20001):
        exact = Fraction(b) * Fraction("1.15")
        lim = ob.slack_limit(b)
        assert lim in (int(exact) - 1, int(exact))
        assert lim == int(Fraction(float(b) * 1.15))
    assert sum(ob.slack_limit(b) != int(Fraction(b) * Fraction("1.15")) for b in range(1, 2001)) > 0


def rand_queues(rng):
    running = []
    for _ in range(rng.randrange(0, 12)):
        c = rng.randrange(0, 5000)
        running.append((c + (1 if rng.random() < 0.6 else rng.randrange(1, 3000)), c))
    waiting = []
    for _ in range(rng.randrange(0, 8)):
        t = rng.randrange(1, 6000)
        waiting.append((t, rng.randrange(0, t)))
    return running, waiting


def test_token_budget_invariants():
    rng = random.Random(11)
    for _ in range(3000):
        running, waiting = rand_queues(rng)
        budget = rng.randrange(1, 6000)
        entries, left = ob.token_budget_step(running, waiting, budget)
        queue = [("running", i, c, t - c) for i, (t, c) in enumerate(running)] + \
                [("waiting", i, c, t - c) for i, (t, c) in enumerate(waiting)]
        # a prefix of the queue, in order, running first
        assert [e[:3] for e in entries] == [q[:3] for q in queue[:len(entries)]]
        # every entry but the last takes its whole need; the last takes what is left
        for e, q in zip(entries[:-1], queue):
            assert e[3] == q[3]
        if entries:
            assert 1 <= entries[-1][3] <= queue[len(entries) - 1][3]
        assert sum(e[3] for e in entries) + left == budget
        assert left == 0 or len(entries) == len(queue)
        assert left >= 0


def test_mixed_chunk_invariants():
    rng = random.Random(12)
    unaligned_continuations = 0
    for _ in range(3000):
        decode = [rng.randrange(0, 9000) for _ in range(rng.randrange(0, 40))]
        chunked = None
        if rng.random() < 0.5:
            t = rng.randrange(2, 20000)
            chunked = (t, rng.randrange(0, t))
        waiting = [(t, rng.randrange(0, t)) for t in (rng.randrange(1, 5000) for _ in range(rng.randrange(0, 6)))]
        size = rng.randrange(1, 6000)
        page = rng.choice([1, 16, 64])
        mixed = rng.random() < 0.8
        entries, left, nc = ob.mixed_chunk_step(decode, chunked, waiting, size, page, mixed)
        dec = [e for e in entries if e[0] == "decode"]
        pre = [e for e in entries if e[0] != "decode"]
        assert dec == ([("decode", i, p, 1) for i, p in enumerate(decode)] if mixed else [])
        budget = max(size - len(decode), 0) if mixed else size
        assert sum(e[3] for e in pre) + left == budget and left >= 0
        if chunked is not None and pre:
            assert pre[0][0] == "chunked" and pre[0][2] == chunked[1]
        if chunked is not None:
            # a continuation takes min(budget, rest of the request), page aligned or not
            take = min(budget, chunked[0] - chunked[1])
            assert [e[3] for e in pre if e[0] == "chunked"] == ([take] if take > 0 else [])
            unaligned_continuations += page > 1 and take % page != 0
        cut = [e for e in pre if e[0] == "waiting" and e[3] < waiting[e[1]][0] - waiting[e[1]][1]]
        assert len(cut) <= 1
        if cut:  # a first cut ends on a page boundary and is the last entry
            assert (cut[0][2] + cut[0][3]) % page == 0 and cut[0] == pre[-1]
            assert nc == ("waiting", cut[0][1], waiting[cut[0][1]][0], cut[0][2] + cut[0][3])
    assert unaligned_continuations > 100  # the branch the goldens with page_size > 1 pin


def test_decode_first_invariants():
    rng = random.Random(13)
    for _ in range(5000):
        b = rng.randrange(1, 20000)
        r, pend, q = rng.randrange(0, 30000), rng.randrange(0, 50), rng.randrange(1, 20000)
        p, d = ob.decode_first_with_slack(r, pend, q, b)
        lim = ob.slack_limit(b)
        assert d == min(r, b)
        assert 0 <= p <= pend
        if p > 0:
            assert p * q + d <= lim
        assert p == pend or (p + 1) * q + d > lim


def test_errors():
    with pytest.raises(ValueError):
        ob.token_budget_step([], [], 0)
    with pytest.raises(ValueError):
        ob.token_budget_step([(5, 5)], [], 10)     # a running request with nothing left
    with pytest.raises(ValueError):
        ob.decode_first_with_slack(1, 1, 0, 100)   # chunk_query_len must be >= 1
    with pytest.raises(ValueError):
        ob.slack_limit(0)
