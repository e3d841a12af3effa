"""Paged-KV attention step for AMD MI355X (gfx950): store_kvcache, varlen causal prefill and decode over a
block-paged cache, plus the fused q/k norm, rotary embedding and store step before attention and the next-token
sampler after it, as hand-written HIP kernels behind a C ABI (include/pa.h, libpa.so).

The Python functions below only marshal torch tensors into the C calls; see binding.py.
"""

from .binding import (  # noqa: F401
    CHECK_KINDS,
    PAError,
    PAIndexError,
    build_metadata,
    build_metadata_store,
    check_indices,
    checked_mode,
    decode,
    decode_append,
    decode_append_noalloc,
    decode_split_tokens,
    decode_workspace_bytes,
    lib,
    norm_rope_store_kvcache,
    prefill_varlen,
    prefill_workspace_bytes,
    sample,
    sample_workspace_bytes,
    status_str,
    store_kvcache,
)

__all__ = [
    "CHECK_KINDS", "PAError", "PAIndexError", "build_metadata", "build_metadata_store", "check_indices",
    "checked_mode", "decode", "decode_append", "decode_append_noalloc", "decode_split_tokens",
    "decode_workspace_bytes", "lib", "norm_rope_store_kvcache", "prefill_varlen", "prefill_workspace_bytes", "sample",
    "sample_workspace_bytes", "status_str", "store_kvcache",
]
