"""Chunked-prefill extend attention for AMD MI355X (gfx950).

The computation lives in the HIP library ``libextattn.so`` (C ABI declared in
``include/extattn.h``); this package is its thin Python binding.
"""

from .binding import (  # noqa: F401
    BLOCK_SIZE,
    EXTATTN_BF16,
    EXTATTN_F32,
    LIB_PATH,
    chunk_plan,
    extend_attention,
    kv_append,
    load_library,
    workspace_bytes,
)
