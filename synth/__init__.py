"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This package holds random-number generation, dtype rounding of the generated
values, and the structure of each workload (token counts, head counts, block
permutations, decode context lengths). It holds none of the attention method's
arithmetic: no chunk plan, no scores, no softmax. Both sides of every parity
check (the HIP library and the CPU oracle) receive the arrays made here.
"""

from .workloads import (  # noqa: F401
    GEN_BLOCK,
    WORKLOADS,
    Request,
    Workload,
    bf16_bits_to_f32,
    block_permutation,
    custom_workload,
    decode_context_lengths,
    device_normal,
    make_workload,
    round_to_bf16,
    token_values,
)
