"""Chunk-plan arithmetic, written out on Python integers (oracle; test infrastructure).

Sources:
* zdszero "Chunked Prefill" notes, section "prefill as several resumable
  extends": a request of N tokens cut at chunk size C takes ceil(N/C) rounds;
  round t has prefix P_t = min(tC, N) and extend length E_t = min(C, N - P_t).
* msmodeling chunked-prefill RFC, section 2.2 (prefix cache with chunked
  prefill): cached tokens = floor(N * hit_rate), and chunking applies to the
  remaining effective length N - cached.
* the same RFC, section 3.1.3 (chunk plan) and section 4 (tests): a chunk
  advances a cursor by min(C, remaining); the cursor starts at the cached
  prefix in kernel space (the cached tokens are "just a prefix" to the kernel,
  zdszero notes, same section).

Readings (where the pages leave a step open):
* floor(N * hit_rate) is one IEEE-754 double multiply (round to nearest even)
  followed by floor; the pages name no numeric type.
* Returned prefixes are kernel-space prefixes: P_t counts the cached tokens.
* Errors follow the RFC's validation rules: a non-positive chunk size and an
  effective length below 1 are errors; so are N < 1 and a hit rate that is NaN
  or outside [0, 1].
"""

from __future__ import annotations

import math


def effective_length(n_tokens: int, hit_rate: float) -> tuple[int, int]:
    """``(cached, effective)`` for a prompt of ``n_tokens`` at ``hit_rate``."""
    if not isinstance(n_tokens, int) or n_tokens < 1:
        raise ValueError("n_tokens must be an integer >= 1")
    h = float(hit_rate)
    if math.isnan(h) or h < 0.0 or h > 1.0:
        raise ValueError("hit_rate must lie in [0, 1]")
    product = float(n_tokens) * h          # one double multiply
    cached = math.floor(product)
    effective = n_tokens - cached
    if effective < 1:
        raise ValueError("effective length after prefix-cache hits must be >= 1")
    return cached, effective


def chunk_plan(n_tokens: int, chunk_size: int, hit_rate: float = 0.0) -> dict:
    """The chunk plan as ``{"cached", "effective", "chunks": [(P_t, E_t), ...]}``.

    The cursor walk: start at the cached prefix, take ``min(C, remaining)`` new
    tokens per round until the effective tokens are used up.
    """
    if not isinstance(chunk_size, int) or chunk_size <= 0:
        raise ValueError("chunk_size must be an integer >= 1")
    cached, effective = effective_length(n_tokens, hit_rate)
    chunks = []
    consumed = 0
    while consumed < effective:
        take = min(chunk_size, effective - consumed)
        chunks.append((cached + consumed, take))
        consumed += take
    return {"cached": cached, "effective": effective, "chunks": chunks}
