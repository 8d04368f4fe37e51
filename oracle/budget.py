"""Mixed-step token-budget planning, written out on Python integers (oracle; test infrastructure).

Three ways the pages turn queues of requests into one forward's work list, each
returning the (prefix, extend) pairs of one launch:

* ``token_budget_step`` -- the token-budget blog ("2.4 Chunked Prefill and the
  unified token budget"), section 4 (one map {request: tokens this step} with a
  sum bounded by the budget) and section 5 (how the budget cuts chunks): running
  requests are served first, each with min(what it still needs, budget left);
  then waiting requests are admitted in queue order the same way, after their
  prefix-cache hits, until the budget is used up. A long prompt is cut into a
  chunk simply because the budget runs out.
* ``mixed_chunk_step`` -- the zdszero "Chunked Prefill" notes, sections on
  scheduling ("only one half-finished request", "four things per round"),
  "mixed chunk" and "page alignment only at the first cut": decode rows take one
  token each and are taken out of the chunk budget first (chunk = size minus the
  running batch), the half-finished request continues before anything new, new
  requests then fill what is left in queue order, and the one that does not fit
  is cut and becomes the next half-finished request; only that first cut of a new
  request is aligned to the page size.
* ``decode_first_with_slack`` -- msmodeling chunked-prefill RFC, section 3.1.4
  (the default mixed-step scheduler): all ready decode rows up to the budget, then
  as many whole prefill chunks as fit under floor(budget * 1.15).

Readings (where the pages leave a step open):
* KV-cache allocation, preemption and the memory budget are left out: every
  allocation succeeds (those branches belong to the cache manager, not the plan).
* floor(budget * 1.15) is one IEEE-754 double multiply followed by floor, as the
  printed scheduler writes it (slack_ratio = 1.15 times an integer): it gives 114
  for a budget of 100 and 3449 for 3000 (the exact products are 115 and 3450).
* In the mixed-chunk step a first cut whose page-aligned length would be zero
  admits nothing; the request waits for the next round.
"""

from __future__ import annotations

import math


def _check_int(name, v, lo):
    if not isinstance(v, int) or isinstance(v, bool) or v < lo:
        raise ValueError(f"{name} must be an integer >= {lo}")


def token_budget_step(running, waiting, budget):
    """One scheduling step under a token budget.

    running: list of (total_tokens, computed): requests already running (decode rows
        have total = computed + 1; an unfinished prefill has more left).
    waiting: list of (total_tokens, cached): queued requests with their prefix-cache hits.
    Returns (entries, budget_left) where entries is a list of (kind, index, prefix, extend)
    in scheduling order, kind "running" or "waiting".
    """
    _check_int("budget", budget, 1)
    entries = []
    left = budget
    for i, (total, computed) in enumerate(running):
        _check_int("computed", computed, 0)
        _check_int("total", total, computed + 1)
        if left == 0:
            break
        take = min(total - computed, left)
        entries.append(("running", i, computed, take))
        left -= take
    for i, (total, cached) in enumerate(waiting):
        _check_int("cached", cached, 0)
        _check_int("total", total, cached + 1)
        if left == 0:
            break
        take = min(total - cached, left)
        entries.append(("waiting", i, cached, take))
        left -= take
    return entries, left


def mixed_chunk_step(decode_prefix, chunked, waiting, chunk_size, page_size=1, mixed=True):
    """One round of the mixed-chunk scheduler.

    decode_prefix: context tokens already cached for each running decode row (each
        decodes one token: prefix = that count, extend = 1).
    chunked: None or (total_tokens, done): the half-finished request.
    waiting: list of (total_tokens, cached) in queue order.
    Returns (entries, chunk_left, new_chunked) where entries are (kind, index, prefix,
    extend) with kind "decode", "chunked" or "waiting"; new_chunked is None or
    ("chunked" | "waiting", index, total, done_after_this_round).
    """
    _check_int("chunk_size", chunk_size, 1)
    _check_int("page_size", page_size, 1)
    entries = []
    left = chunk_size
    if mixed:
        for i, p in enumerate(decode_prefix):
            _check_int("decode prefix", p, 0)
            entries.append(("decode", i, p, 1))
        left = chunk_size - len(decode_prefix)
        if left < 0:
            left = 0
    new_chunked = None
    if chunked is not None:
        total, done = chunked
        _check_int("done", done, 0)
        _check_int("total", total, done + 1)
        take = min(total - done, left)  # continuation cuts are not page-aligned
        if take > 0:
            entries.append(("chunked", 0, done, take))
            left -= take
        if done + take < total:
            return entries, left, ("chunked", 0, total, done + take)
    for i, (total, cached) in enumerate(waiting):
        _check_int("cached", cached, 0)
        _check_int("total", total, cached + 1)
        if left == 0:
            break
        need = total - cached
        if need <= left:
            entries.append(("waiting", i, cached, need))
            left -= need
            continue
        # first cut of a new request: its end is aligned down to a whole page
        end = (cached + left) // page_size * page_size
        take = end - cached
        if take > 0:
            entries.append(("waiting", i, cached, take))
            left -= take
            new_chunked = ("waiting", i, total, cached + take)
        break
    return entries, left, new_chunked


def slack_limit(max_batched_tokens, slack_ratio=1.15):
    """floor(max_batched_tokens * slack_ratio), one double multiply."""
    _check_int("max_batched_tokens", max_batched_tokens, 1)
    return math.floor(float(max_batched_tokens) * float(slack_ratio))


def decode_first_with_slack(ready_decode, pending_prefill, chunk_query_len, max_batched_tokens,
                            slack_ratio=1.15):
    """(p_step, d_step): decode rows first, then whole prefill chunks under the slack limit."""
    _check_int("ready_decode", ready_decode, 0)
    _check_int("pending_prefill", pending_prefill, 0)
    _check_int("chunk_query_len", chunk_query_len, 1)
    limit = slack_limit(max_batched_tokens, slack_ratio)
    d = min(ready_decode, max_batched_tokens)
    room = limit - d
    p = max(0, min(pending_prefill, room // chunk_query_len if room >= 0 else 0))
    return p, d
