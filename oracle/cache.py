"""The KV cache itself: logical contents, append contract, physical layouts,
byte closed forms.

Test infrastructure (see the package docstring).  Sources are cited by the
short keys [P1]..[P4] defined there.

Physical layouts predicted here (storage units are raw: uint32 words of fp32,
uint16 words of bf16, uint8 codes of fp8 E4M3FN):
  contiguous: [rows, Hkv, capacity, d]   - the [batch, kv_heads, seq,
              head_dim] shape of [P3] section "Tensor" and [P4] section
              "Cache shape and memory calculation";
  paged:      [num_blocks, Hkv, 16, d] with block_table[b][j] the physical
              block holding positions 16j .. 16j+15 of sequence b - the
              16-token blocks and page table of [P1] section
              "PagedAttention" and [P2] section "(4) PagedAttention".  The
              in-block order [Hkv, 16, d] is our reading (the pages fix only
              the 16-token granularity).
"""
import numpy as np

from . import codec

BLOCK_TOKENS = 16

F32, BF16, FP8_E4M3 = 0, 1, 2
_STORAGE = {F32: np.uint32, BF16: np.uint16, FP8_E4M3: np.uint8}
ELEM_BYTES = {F32: 4, BF16: 2, FP8_E4M3: 1}


def cache_bytes(layers, batch, kv_heads, seq, head_dim, elem_bytes):
    """Exact KV-cache size in bytes: 2 (K and V) x layers x batch x kv_heads
    x seq x head_dim x bytes per element.

    [P4] section "Cache shape and memory calculation" (the product formula
    and its 17,179,869,184-byte example); [P2] section "KV cache memory size
    calculation"; [P1] section "KV cache math".
    """
    return 2 * int(layers) * int(batch) * int(kv_heads) * int(seq) * int(head_dim) * int(elem_bytes)


def op_counts(n_tokens):
    """Attention query-rows computed to generate n tokens: the naive decoder
    recomputes every earlier row at each step (1 + 2 + ... + n), the cached
    decoder computes one new row per step ([P1] section "Build it", Step 3)."""
    n = int(n_tokens)
    return n * (n + 1) // 2, n


def to_f64(storage, dtype, scale=None):
    """Decode raw cache storage to fp64 values (fp8: times the dequant scale)."""
    if dtype == F32:
        return np.asarray(storage, dtype=np.uint32).view(np.float32).astype(np.float64)
    if dtype == BF16:
        return codec.bf16_bits_to_f64(storage)
    if dtype == FP8_E4M3:
        v = codec.e4m3_decode(storage)
        return v if scale is None else v * np.float64(np.float32(scale))
    raise ValueError(dtype)


def encode_rows(x_storage, in_dtype, cache_dtype, scale=None):
    """Convert new K/V rows from the input storage format to the cache's.

    Same format: the same bits.  f32/bf16 input -> fp8 cache: the fp32 value
    divided by the fp32 scale, rounded to E4M3FN ([P2] section "(1) FP8
    quantization": the cache is stored at 8 bits).  f32 -> bf16 is not a
    supported conversion (the library copies, it does not round).
    """
    if in_dtype == cache_dtype:
        return np.array(x_storage, dtype=_STORAGE[cache_dtype], copy=True)
    if cache_dtype == FP8_E4M3 and in_dtype in (F32, BF16):
        xf = to_f64(x_storage, in_dtype).astype(np.float32)  # exact
        return codec.e4m3_quantize(xf, scale)
    raise ValueError("unsupported conversion %r -> %r" % (in_dtype, cache_dtype))


class SequenceStore:
    """Logical contents of one layer's cache: per sequence, an fp64 array
    [Hkv, stored length, d] for K and one for V, in position order, with the
    append contract.

    [P3] section "Tensor" (the cache of one layer is [batch, kv_heads, seq,
    head_dim]; here each sequence keeps its own seq extent); [P4] section
    "Position IDs and the append contract" (new rows go in at cache_position
    equal to the current stored length, positions 0-based; anything else is
    an error).
    """

    def __init__(self, batch, kv_heads, head_dim):
        empty = np.zeros((kv_heads, 0, head_dim), dtype=np.float64)
        self.k = [empty.copy() for _ in range(batch)]
        self.v = [empty.copy() for _ in range(batch)]

    def stored(self, b):
        """Positions stored for sequence b."""
        return self.k[b].shape[1]

    def store(self, b, position, k_rows, v_rows):
        """k_rows, v_rows: [Hkv, n, d] values of n new tokens at positions
        position .. position + n - 1 of sequence b."""
        if position != self.stored(b):
            raise ValueError("store at position %d, stored length %d" % (position, self.stored(b)))
        self.k[b] = np.concatenate([self.k[b], np.asarray(k_rows, dtype=np.float64)], axis=1)
        self.v[b] = np.concatenate([self.v[b], np.asarray(v_rows, dtype=np.float64)], axis=1)

    def head(self, b, g):
        """([len, d], [len, d]) arrays of sequence b, KV head g."""
        return self.k[b][g], self.v[b][g]


def predict_append(cache_k, cache_v, k_new, v_new, positions, n_new, paged,
                   block_table=None, in_dtype=BF16, cache_dtype=BF16,
                   k_scale=None, v_scale=None, n_valid=None):
    """Physical cache contents after an append (the kv_append step).

    For token i < n_valid[b] (default n_new) of sequence b, position
    p = positions[b] + i:
        contiguous: cache[b, g, p, :]                        <- encode(x[b, g, i, :])
        paged:      pool[block_table[b][p // 16], g, p % 16, :] <- encode(x[b, g, i, :])
    Every other slot keeps its bytes.  cache_k/cache_v: raw storage arrays
    (not modified); k_new/v_new: [B, Hkv, n_new, d] raw input storage.
    Returns new (cache_k, cache_v) arrays.
    """
    ck = np.array(cache_k, copy=True)
    cv = np.array(cache_v, copy=True)
    B, Hkv = k_new.shape[0], k_new.shape[1]
    for b in range(B):
        nb = n_new if n_valid is None else int(n_valid[b])
        for i in range(nb):
            p = int(positions[b]) + i
            for g in range(Hkv):
                ks = None if k_scale is None else k_scale[g]
                vs = None if v_scale is None else v_scale[g]
                kr = encode_rows(k_new[b, g, i], in_dtype, cache_dtype, ks)
                vr = encode_rows(v_new[b, g, i], in_dtype, cache_dtype, vs)
                if paged:
                    blk = int(block_table[b][p // BLOCK_TOKENS])
                    ck[blk, g, p % BLOCK_TOKENS] = kr
                    cv[blk, g, p % BLOCK_TOKENS] = vr
                else:
                    ck[b, g, p] = kr
                    cv[b, g, p] = vr
    return ck, cv


def gather_sequence(cache, paged, b, g, length, block_table=None):
    """Raw storage rows of positions 0 .. length-1 of sequence b, KV head g,
    read through the block table when paged."""
    rows = []
    for p in range(int(length)):
        if paged:
            rows.append(cache[int(block_table[b][p // BLOCK_TOKENS]), g, p % BLOCK_TOKENS])
        else:
            rows.append(cache[b, g, p])
    if not rows:
        return np.zeros((0,) + tuple(cache.shape[3:]), dtype=cache.dtype)
    return np.stack(rows)


def beam_reorder(rows, perm):
    """Rows of the cache after a batch/beam reorder: new row i is old row
    perm[i] ([P4] section "Batch and beam reorder": [A0, A1, B0] sorted to
    [B0, A1, A0] uses the permutation [2, 1, 0])."""
    return [rows[int(i)] for i in perm]
