"""Paged GQA split-KV decode attention for MI355X (gfx950).

The compute path is the C-ABI library ``libdecode_attn.so`` (hand-written HIP kernels, declared in
``include/decode_attn.h``). ``paged_gqa_kv_attn_amd.binding`` marshals arguments to it with ctypes;
PyTorch only supplies device memory and the current stream. The library is loaded on first use
and a missing or unloadable library raises an error: there is no fallback.
"""
from .binding import (  # noqa: F401
    NORM_QK,
    NORM_V,
    DecodeAttnError,
    Plan,
    PreparedCall,
    decode_attn_append_kv,
    decode_attn_append_kv_rope,
    decode_attn_global,
    decode_attn_layer_noalloc,
    decode_attn_plan,
    decode_attn_rope_cache,
    decode_attn_sliding,
    decode_attn_stage1,
    decode_attn_stage2,
    decode_attn_status_str,
    decode_attn_version,
    library_path,
    load_library,
)
