"""paged_kv_attention_pkv_amd -- attention over a paged KV cache on MI355X (gfx950).

The compute path is the C-ABI library ``libpkv.so`` (hand-written HIP kernels,
declared in ``include/pkv.h``).  This package is its thin Python binding:
argument marshalling from torch tensors (device memory and streams) to the C
entry points, nothing else.  The library is loaded on first use and a missing
or unloadable library raises immediately; there is no fallback path.
"""
from .api import (  # noqa: F401
    EXPORTED,
    PkvError,
    cache_desc,
    append,
    append_decode_attn,
    append_decode_attn_noalloc,
    append_rope,
    decode_attn,
    decode_plan,
    decode_workspace_bytes,
    decode_workspace_reset,
    lib_path,
    mixed_attn,
    mixed_workspace_bytes,
    prefill_attn,
    prefill_workspace_bytes,
    route,
    validate_append_host,
    validate_decode_step_host,
    validate_host,
)
