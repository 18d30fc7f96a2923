"""Rotated INT2 KV cache for MI355X: append quantiser and INT2 paged decode
attention as hand-written gfx950 HIP kernels behind the C ABI in include/kvq.h.
"""
from ._lib import (  # noqa: F401
    KVQ_BF16,
    KVQ_F32,
    LIB_PATH,
    STAGE_ALL,
    STAGE_MERGE,
    STAGE_PREPARE,
    STAGE_SPLITS,
    KvqError,
    append,
    append_decode,
    append_decode_window,
    decode,
    decode_noalloc,
    SCRATCH_BYTES,
    decode_window,
    decode_workspace_bytes,
    lib,
    page_bytes,
    status_string,
    new_window,
    window_bytes,
    window_write,
    WINDOW_SINK,
    WINDOW_RECENT,
)
