"""Causal MHA/GQA attention for MI355X (gfx950): bf16 MFMA prefill (dense, ragged over packed tokens, or
chunked over a paged cache, alone or fused with the chunk's KV append), paged split-KV decode (bf16 or FP8 E4M3
cache, bf16 optionally with the newest token's append fused), and the paged-cache KV append.

The compute lives in ``libattn.so`` (hand-written HIP kernels behind the C ABI
declared in ``include/attn.h``); this package is its ctypes binding, with the
same function names.  ``synth`` draws the seeded synthetic inputs the tests and
the benchmark use.
"""

from ._binding import (  # noqa: F401
    ATTN_BF16,
    ATTN_ERR_HIP,
    ATTN_ERR_INVALID_ARG,
    ATTN_ERR_UNSUPPORTED,
    ATTN_ERR_WORKSPACE,
    ATTN_F32,
    ATTN_OK,
    LIB_PATH,
    AttnError,
    attn_decode_num_splits,
    attn_decode_paged,
    attn_decode_paged_append,
    attn_decode_paged_fp8,
    attn_decode_paged_noalloc,
    attn_decode_workspace_bytes,
    attn_kv_append,
    attn_last_error_message,
    attn_prefill,
    attn_prefill_paged,
    attn_prefill_paged_append,
    attn_prefill_varlen,
    attn_status_string,
    attn_validate_chunk_metadata,
    attn_validate_paged_metadata,
    attn_validate_varlen_metadata,
    load_library,
)
