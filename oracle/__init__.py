"""CPU oracle for chunked-prefill extend attention (TEST INFRASTRUCTURE ONLY).

This package is the plain, slow, obviously correct definition of what the GPU
path computes, written from the pages in float64 NumPy and Python integers. It
exists to check the HIP library: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call it. The product path
never routes through it, and it shares no code, constants or helpers with the
HIP library; the only thing both sides share is the seeded input generator in
``synth/``, which holds none of the method's arithmetic.

Every function is pinned by ``-m "not gpu"`` tests against values the pages
print, closed forms, special cases, brute force and a library routine; no
function here is "parity unpinned".
"""

from .chunk_plan import chunk_plan, effective_length  # noqa: F401
from .budget import decode_first_with_slack, mixed_chunk_step, slack_limit, token_budget_step  # noqa: F401
from .attention import (  # noqa: F401
    attend_rows,
    causal_attention,
    lse_merge,
    merge_two,
    rectangle_triangle,
)
