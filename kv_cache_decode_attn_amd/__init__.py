"""kv_cache_decode_attn_amd - KV-cache attention for MI355X (gfx950).

Decode (split-K over the cache), prefill (tiled, causal/padding masked),
the cache append, batch/beam reorder and copy-on-write block copies, as
hand-written HIP kernels behind a C ABI (include/kvattn.h, libkvattn.so),
with a host block pool (free list and reference counts) in the same library.
This package is the thin Python binding (`api`), the seeded synthetic-input
generators (`synth`) and the paging fragmentation study (`fragmentation`).
"""
from ._lib import (BF16, BLOCK_TOKENS, CONTIGUOUS, EINVAL, ELAUNCH, ENOSPACE, EUNSUPPORTED, EWORKSPACE, F32, FP8_E4M3,
                   NOALLOC_SCRATCH_BYTES, OK, PAGED, VALIDATE_BLOCK_RANGE, VALIDATE_LEN_RANGE, VALIDATE_POSITION,
                   KvattnError)
from .api import (BlockPool, KVCache, attn_decode, attn_decode_append, attn_decode_append_noalloc, attn_decode_multi,
                  attn_prefill, cache_bytes, copy_blocks, stream_read, decode_default_part_tokens, decode_workspace,
                  decode_workspace_bytes, kv_append, reorder_cache, reorder_rows, validate, version)

__all__ = [
    "KVCache", "attn_decode", "attn_decode_append", "attn_decode_append_noalloc", "attn_decode_multi", "attn_prefill",
    "cache_bytes",
    "decode_default_part_tokens", "decode_workspace", "decode_workspace_bytes", "kv_append", "validate", "version",
    "KvattnError", "reorder_rows", "reorder_cache", "copy_blocks", "stream_read", "BlockPool",
    "F32", "BF16", "FP8_E4M3", "CONTIGUOUS", "PAGED", "BLOCK_TOKENS",
]
