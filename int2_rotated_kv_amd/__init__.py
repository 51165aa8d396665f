"""MI355X (gfx950) rotated INT2 KV cache: quantize-write and decode attention.

The compute runs in libkvq.so (hand-written HIP kernels behind a C ABI,
include/kvq.h); this package is the thin Python binding over it.
"""
from .kvq import (  # noqa: F401
    Int2Cache, PagedCache, KvqError, kvq_quantize, kvq_decode_attention,
    kvq_quantize_paged, kvq_decode_attention_paged, kvq_decode_attention_noalloc,
    kvq_quantize_prerope, kvq_decode_attention_prerope, kvq_decode_workspace_bytes_prerope,
    kvq_decode_workspace_bytes, kvq_status_str, kvq_abi_version, load_library,
    library_path, EXPORTED_SYMBOLS,
)
