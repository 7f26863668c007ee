"""pkv: attention over a paged KV cache on MI355X (gfx950).

The compute lives in libpkv.so (hand-written HIP); this package only binds
it.  Importing the package loads the library and fails if it is not built.
"""
from ._lib import (  # noqa: F401
    BF16, F16, F32, FP8, I8, PAGE_SIZE, PkvError, load_library, paged_attn_decode,
    paged_attn_decode_append, paged_attn_decode_noalloc,
    paged_attn_decode_workspace_bytes, paged_attn_mixed, paged_attn_mixed_workspace_bytes,
    paged_attn_prefill_chunk, paged_attn_prefill_workspace_bytes, paged_kv_append,
    paged_kv_append_rope,
    pkv_abi_version, pkv_status_string,
)

load_library()
