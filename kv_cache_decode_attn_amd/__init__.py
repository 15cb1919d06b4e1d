"""kv_cache_decode_attn_amd - KV-cache attention for MI355X (gfx950).

Decode (split-K over the cache), prefill (tiled, causal/padding masked) and
the cache append, as hand-written HIP kernels behind a C ABI
(include/kvattn.h, libkvattn.so).  This package is the thin Python binding
(`api`) plus the seeded synthetic-input generators (`synth`).
"""
from ._lib import (BF16, BLOCK_TOKENS, CONTIGUOUS, EINVAL, ELAUNCH, EUNSUPPORTED, EWORKSPACE, F32, FP8_E4M3, OK,
                   PAGED, VALIDATE_BLOCK_RANGE, VALIDATE_LEN_RANGE, VALIDATE_POSITION, KvattnError)
from .api import (KVCache, attn_decode, attn_decode_append, attn_prefill, cache_bytes, decode_default_part_tokens,
                  decode_workspace, decode_workspace_bytes, kv_append, validate, version)

__all__ = [
    "KVCache", "attn_decode", "attn_decode_append", "attn_prefill", "cache_bytes", "decode_default_part_tokens",
    "decode_workspace", "decode_workspace_bytes", "kv_append", "validate", "version", "KvattnError",
    "F32", "BF16", "FP8_E4M3", "CONTIGUOUS", "PAGED", "BLOCK_TOKENS",
]
