"""The library's mixed-step planners (host code behind the C ABI) against the
oracle: exact on the pages' worked examples and on random queues; error codes.
CPU only: these entry points do not touch the GPU."""
import json
import os
import random

import pytest

import chunked_prefill_attention_extend_amd as ext
import oracle.budget as ob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "budget_examples.jsonl")


def golden():
    with open(GOLDEN) as f:
        return [json.loads(line) for line in f if line.strip()]


@pytest.mark.parametrize("ex", golden(), ids=lambda e: e["policy"])
def test_golden_examples(ex):
    pol = ex["policy"]
    if pol == "token_budget":
        entries, left = ext.token_budget_step([tuple(r) for r in ex["running"]], [tuple(w) for w in ex["waiting"]],
                                              ex["budget"])
        assert [e[3] for e in entries] == ex["expect_extend"] and left == ex["expect_left"]
    elif pol == "mixed_chunk":
        entries, left, nc = ext.mixed_chunk_step(ex["decode"], tuple(ex["chunked"]) if ex["chunked"] else None,
                                                 [tuple(w) for w in ex["waiting"]], ex["chunk_size"],
                                                 ex["page_size"], ex["mixed"])
        assert left == ex["expect_left"]
        if "expect_entries" in ex:
            assert [list(e) for e in entries] == ex["expect_entries"]
            assert (list(nc) if nc else None) == ex["expect_new_chunked"]
        if "expect_chunk_extend" in ex:
            assert [e[3] for e in entries if e[0] == "chunked"] == [ex["expect_chunk_extend"]]
    elif pol == "decode_first":
        p, d, lim = ext.decode_first_with_slack(ex["ready_decode"], ex["pending_prefill"], ex["chunk_query_len"],
                                                ex["max_batched_tokens"])
        assert (p, d, lim) == (ex["expect_p"], ex["expect_d"], ex["expect_limit"])
    elif pol == "slack_limit":
        assert ext.decode_first_with_slack(0, 0, 1, ex["max_batched_tokens"])[2] == ex["expect_limit"]


def test_token_budget_matches_oracle():
    rng = random.Random(21)
    for _ in range(2000):
        running = []
        for _ in range(rng.randrange(0, 12)):
            c = rng.randrange(0, 5000)
            running.append((c + (1 if rng.random() < 0.6 else rng.randrange(1, 3000)), c))
        waiting = [(t, rng.randrange(0, t)) for t in (rng.randrange(1, 6000) for _ in range(rng.randrange(0, 8)))]
        budget = rng.randrange(1, 9000)
        assert ext.token_budget_step(running, waiting, budget) == ob.token_budget_step(running, waiting, budget)


def test_mixed_chunk_matches_oracle():
    rng = random.Random(22)
    for _ in range(2000):
        decode = [rng.randrange(0, 9000) for _ in range(rng.randrange(0, 40))]
        chunked = None
        if rng.random() < 0.5:
            t = rng.randrange(2, 20000)
            chunked = (t, rng.randrange(0, t))
        waiting = [(t, rng.randrange(0, t)) for t in (rng.randrange(1, 5000) for _ in range(rng.randrange(0, 6)))]
        size = rng.randrange(1, 6000)
        page = rng.choice([1, 16, 64])
        mixed = rng.random() < 0.8
        got = ext.mixed_chunk_step(decode, chunked, waiting, size, page, mixed)
        want = ob.mixed_chunk_step(decode, chunked, waiting, size, page, mixed)
        assert got == want


def test_decode_first_matches_oracle():
    rng = random.Random(23)
    for _ in range(20000):
        b = rng.randrange(1, 1 << 20)
        r, pend, q = rng.randrange(0, 1 << 20), rng.randrange(0, 100), rng.randrange(1, 1 << 16)
        p, d, lim = ext.decode_first_with_slack(r, pend, q, b)
        assert (p, d) == ob.decode_first_with_slack(r, pend, q, b)
        assert lim == ob.slack_limit(b)


def test_errors():
    with pytest.raises(ValueError):
        ext.token_budget_step([], [], 0)
    with pytest.raises(ValueError):
        ext.token_budget_step([(5, 5)], [], 10)
    with pytest.raises(ValueError):
        ext.mixed_chunk_step([], (10, 10), [], 100)
    with pytest.raises(ValueError):
        ext.mixed_chunk_step([], None, [], 0)
    with pytest.raises(ValueError):
        ext.decode_first_with_slack(1, 1, 0, 100)
    with pytest.raises(ValueError):
        ext.decode_first_with_slack(1, 1, 10, 0)
