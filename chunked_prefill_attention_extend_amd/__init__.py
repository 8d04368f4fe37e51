"""Chunked-prefill extend attention for AMD MI355X (gfx950).

The computation lives in the HIP library ``libextattn.so`` (C ABI declared in
``include/extattn.h``); this package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    BLOCK_SIZE,
    EXTATTN_BF16,
    EXTATTN_F32,
    LIB_PATH,
    STATUS_BAD_BLOCK,
    STATUS_WAIT_TIMEOUT,
    chunk_plan,
    decode_first_with_slack,
    extend_attention,
    extend_attention_append,
    extend_attention_noalloc,
    kv_append,
    last_status,
    load_library,
    mixed_chunk_step,
    plan_cache_clear,
    plan_cache_configure,
    plan_cache_stats,
    read_status,
    status_error,
    token_budget_step,
    workspace_bytes,
)
