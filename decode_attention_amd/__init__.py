"""Paged decode attention for AMD MI355X (gfx950).

The compute lives in ``libdecode_attn.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/decode_attn.h``). ``binding`` marshals torch
tensors into that ABI; nothing in this package computes attention itself.
"""

from .binding import (  # noqa: F401
    DecodeAttnError,
    attn_decode_sliding,
    attn_decode_global,
    attn_decode_global_workspace_bytes,
    attn_decode_global_noalloc,
    attn_decode_sliding_gated,
    attn_decode_global_gated,
    attn_decode_global_prenorm,
    attn_kv_append_sliding,
    attn_kv_append_global,
    attn_kv_append_global_prenorm,
    attn_multiquery_sliding,
    attn_multiquery_global,
    attn_multiquery_workspace_bytes,
    attn_status_string,
    bind,
    library_path,
    load_library,
)
