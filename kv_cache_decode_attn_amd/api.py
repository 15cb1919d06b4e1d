"""Torch-facing binding of libkvattn: the same calls as include/kvattn.h.

Argument marshalling only - tensors become device pointers, the current
torch stream becomes the HIP stream, and every step of the computation runs
in the library's HIP kernels.  PyTorch provides device memory (outputs and
workspaces are allocated here when the caller does not pass them).  There is
no fallback: without the built library or on CPU tensors these raise.
"""
import ctypes
import math

import numpy as np
import torch

from . import _lib
from ._lib import BF16, CONTIGUOUS, F32, FP8_E4M3, PAGED, BLOCK_TOKENS, check, lib

_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3: torch.uint8}
_CODE = {torch.float32: F32, torch.bfloat16: BF16}


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device (cuda/hip) tensor, got %s" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _i32(t, name):
    t = _dev(t, name)
    if t is not None and t.dtype != torch.int32:
        raise TypeError("%s must be int32" % name)
    return t


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class KVCache:
    """One layer's KV cache in device memory plus its layout.

    contiguous: k, v of shape [rows, num_kv_heads, capacity, head_dim]
    paged:      k, v of shape [num_blocks, num_kv_heads, 16, head_dim]
    dtype is F32, BF16 or FP8_E4M3 (fp8 codes are stored in uint8 tensors and
    need k_scale / v_scale, fp32 [num_kv_heads]).
    """

    def __init__(self, k, v, layout, dtype, k_scale=None, v_scale=None):
        _dev(k, "k")
        _dev(v, "v")
        if k.shape != v.shape or k.dim() != 4:
            raise ValueError("k and v must be 4-D tensors of one shape")
        if k.dtype != _TORCH_DTYPE[dtype] or v.dtype != _TORCH_DTYPE[dtype]:
            raise TypeError("storage dtype %s does not match cache dtype %d" % (k.dtype, dtype))
        if dtype == FP8_E4M3:
            for s, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
                _dev(s, n)
                if s is None or s.dtype != torch.float32 or s.numel() != k.shape[1]:
                    raise ValueError("%s must be fp32 [num_kv_heads]" % n)
        self.k, self.v, self.layout, self.dtype = k, v, layout, dtype
        self.k_scale, self.v_scale = k_scale, v_scale
        self.num_kv_heads = k.shape[1]
        self.head_dim = k.shape[3]
        if layout == PAGED and k.shape[2] != BLOCK_TOKENS:
            raise ValueError("paged pools hold 16 positions per block")

    @classmethod
    def contiguous(cls, rows, num_kv_heads, capacity, head_dim, dtype, device="cuda", k_scale=None,
                   v_scale=None, fill=None):
        shape = (rows, num_kv_heads, capacity, head_dim)
        k = torch.empty(shape, dtype=_TORCH_DTYPE[dtype], device=device)
        v = torch.empty(shape, dtype=_TORCH_DTYPE[dtype], device=device)
        if fill is not None:
            k.fill_(fill)
            v.fill_(fill)
        return cls(k, v, CONTIGUOUS, dtype, k_scale, v_scale)

    @classmethod
    def paged(cls, num_blocks, num_kv_heads, head_dim, dtype, device="cuda", k_scale=None, v_scale=None,
              fill=None):
        shape = (num_blocks, num_kv_heads, BLOCK_TOKENS, head_dim)
        k = torch.empty(shape, dtype=_TORCH_DTYPE[dtype], device=device)
        v = torch.empty(shape, dtype=_TORCH_DTYPE[dtype], device=device)
        if fill is not None:
            k.fill_(fill)
            v.fill_(fill)
        return cls(k, v, PAGED, dtype, k_scale, v_scale)

    @property
    def device(self):
        return self.k.device

    def desc(self):
        d = _lib.KvattnCache()
        d.dtype = self.dtype
        d.layout = self.layout
        d.num_kv_heads = self.num_kv_heads
        d.head_dim = self.head_dim
        if self.layout == CONTIGUOUS:
            d.capacity = self.k.shape[2]
            d.num_rows = self.k.shape[0]
        else:
            d.num_blocks = self.k.shape[0]
        d.k = self.k.data_ptr()
        d.v = self.v.data_ptr()
        d.k_scale = self.k_scale.data_ptr() if self.k_scale is not None else None
        d.v_scale = self.v_scale.data_ptr() if self.v_scale is not None else None
        return d


def version():
    return lib().kvattn_version().decode()


def cache_bytes(layers, batch, kv_heads, seq, head_dim, elem_bytes):
    return int(lib().kvattn_cache_bytes(layers, batch, kv_heads, seq, head_dim, elem_bytes))


def kv_append(cache, k_new, v_new, positions, block_table=None, n_valid=None):
    """Write k_new/v_new [B, Hkv, n_new, d] at positions[b] + i (kvattn_kv_append)."""
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    _i32(positions, "positions")
    _i32(block_table, "block_table")
    _i32(n_valid, "n_valid")
    if k_new.dtype not in _CODE or v_new.dtype != k_new.dtype or k_new.shape != v_new.shape:
        raise TypeError("k_new/v_new must be matching f32 or bf16 tensors")
    B, H, n, d = k_new.shape
    if H != cache.num_kv_heads or d != cache.head_dim:
        raise ValueError("k_new shape %s does not match the cache" % (tuple(k_new.shape),))
    mb = block_table.shape[1] if block_table is not None else 0
    check(lib().kvattn_kv_append(ctypes.byref(cache.desc()), B, n, _ptr(k_new), _ptr(v_new), _CODE[k_new.dtype],
                                 _ptr(positions), _ptr(n_valid), _ptr(block_table), mb, _stream(k_new.device)))


def decode_default_part_tokens(cache_dtype, batch, num_q_heads, num_kv_heads, max_seq_len):
    return int(lib().kvattn_decode_default_part_tokens(cache_dtype, batch, num_q_heads, num_kv_heads, max_seq_len))


def decode_workspace_bytes(cache_dtype, batch, num_q_heads, num_kv_heads, head_dim, max_seq_len, part_tokens=0):
    return int(lib().kvattn_decode_workspace_bytes(cache_dtype, batch, num_q_heads, num_kv_heads, head_dim,
                                                   max_seq_len, part_tokens))


def decode_workspace(cache, batch, num_q_heads, max_seq_len, part_tokens=0):
    """A workspace tensor large enough for attn_decode with these sizes."""
    n = decode_workspace_bytes(cache.dtype, batch, num_q_heads, cache.num_kv_heads, cache.head_dim, max_seq_len,
                               part_tokens)
    return torch.empty(max(n, 16) // 4 + 4, dtype=torch.float32, device=cache.device)


def _decode_args(cache, q, seq_lens, max_seq_len, block_table, key_mask, scale, out, workspace, part_tokens):
    _dev(q, "q")
    _i32(seq_lens, "seq_lens")
    _i32(block_table, "block_table")
    _dev(key_mask, "key_mask")
    if key_mask is not None and key_mask.dtype != torch.uint8:
        raise TypeError("key_mask must be uint8")
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _dev(out, "out")
    if workspace is None:
        workspace = decode_workspace(cache, B, Hq, max_seq_len, part_tokens)
    _dev(workspace, "workspace")
    mb = block_table.shape[1] if block_table is not None else 0
    stride = key_mask.shape[1] if key_mask is not None else 0
    return B, Hq, float(scale), out, workspace, mb, stride


def attn_decode(cache, q, seq_lens, max_seq_len, block_table=None, key_mask=None, scale=None, out=None,
                workspace=None, part_tokens=0):
    """One query token per sequence against the cache (kvattn_attn_decode).

    q: [B, Hq, d] (f32 for an f32 cache, bf16 otherwise); seq_lens int32 [B]
    counts keys including the appended token; key_mask uint8 [B, >= max_seq_len]
    (1 = attend) or None.  Returns fp32 [B, Hq, d].
    """
    B, Hq, scale, out, workspace, mb, stride = _decode_args(cache, q, seq_lens, max_seq_len, block_table, key_mask,
                                                            scale, out, workspace, part_tokens)
    check(lib().kvattn_attn_decode(ctypes.byref(cache.desc()), B, Hq, _ptr(q), _CODE.get(q.dtype, -1), _ptr(seq_lens),
                                   int(max_seq_len), _ptr(block_table), mb, _ptr(key_mask), stride, scale, _ptr(out),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), int(part_tokens),
                                   _stream(q.device)))
    return out


def attn_decode_append(cache, q, k_new, v_new, seq_lens, max_seq_len, block_table=None, key_mask=None, scale=None,
                       out=None, workspace=None, part_tokens=0):
    """One decode step (kvattn_attn_decode_append): k_new/v_new [B, Hkv, d]
    (f32 or bf16) are stored at position seq_lens[b] - 1, then q attends the
    cache as in attn_decode.  Returns fp32 [B, Hq, d]."""
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    if k_new.dtype not in _CODE or v_new.dtype != k_new.dtype or k_new.shape != v_new.shape:
        raise TypeError("k_new/v_new must be matching f32 or bf16 tensors")
    if k_new.dim() != 3 or k_new.shape[1] != cache.num_kv_heads or k_new.shape[2] != cache.head_dim:
        raise ValueError("k_new shape %s does not match the cache" % (tuple(k_new.shape),))
    if k_new.shape[0] != q.shape[0]:
        raise ValueError("k_new batch %d differs from q batch %d" % (k_new.shape[0], q.shape[0]))
    B, Hq, scale, out, workspace, mb, stride = _decode_args(cache, q, seq_lens, max_seq_len, block_table, key_mask,
                                                            scale, out, workspace, part_tokens)
    check(lib().kvattn_attn_decode_append(ctypes.byref(cache.desc()), B, Hq, _ptr(q), _CODE.get(q.dtype, -1),
                                          _ptr(k_new), _ptr(v_new), _CODE[k_new.dtype], _ptr(seq_lens),
                                          int(max_seq_len), _ptr(block_table), mb, _ptr(key_mask), stride, scale,
                                          _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          int(part_tokens), _stream(q.device)))
    return out



def attn_decode_append_noalloc(cache, q, k_new, v_new, seq_lens, max_seq_len, block_table=None, key_mask=None,
                               scale=None, out=None, part_tokens=0):
    """attn_decode_append without a workspace (kvattn_attn_decode_append_noalloc):
    the split-K partials go to the library's static per-GPU scratch array
    (NOALLOC_SCRATCH_BYTES).  `out` must be given for a call that allocates
    nothing at all (else it is allocated here).  Calls on one GPU share the
    array: do not overlap them."""
    _dev(q, "q")
    _dev(k_new, "k_new")
    _dev(v_new, "v_new")
    _i32(seq_lens, "seq_lens")
    _i32(block_table, "block_table")
    _dev(key_mask, "key_mask")
    if key_mask is not None and key_mask.dtype != torch.uint8:
        raise TypeError("key_mask must be uint8")
    if k_new.dtype not in _CODE or v_new.dtype != k_new.dtype or k_new.shape != v_new.shape:
        raise TypeError("k_new/v_new must be matching f32 or bf16 tensors")
    B, Hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    _dev(out, "out")
    mb = block_table.shape[1] if block_table is not None else 0
    stride = key_mask.shape[1] if key_mask is not None else 0
    check(lib().kvattn_attn_decode_append_noalloc(ctypes.byref(cache.desc()), B, Hq, _ptr(q), _CODE.get(q.dtype, -1),
                                                  _ptr(k_new), _ptr(v_new), _CODE[k_new.dtype], _ptr(seq_lens),
                                                  int(max_seq_len), _ptr(block_table), mb, _ptr(key_mask), stride,
                                                  float(scale), _ptr(out), int(part_tokens), _stream(q.device)))
    return out



def attn_decode_multi(cache, q, seq_lens, max_seq_len, k_new=None, v_new=None, block_table=None, key_mask=None,
                      scale=None, out=None, workspace=None, part_tokens=0):
    """n_q query tokens per sequence against the cache (kvattn_attn_decode_multi):
    q [B, Hq, n_q, d]; their K/V are the last n_q positions below seq_lens[b],
    stored by this call when k_new/v_new [B, Hkv, n_q, d] (f32 or bf16) are
    given.  Query i sees the keys below seq_lens[b] - (n_q - 1 - i).  Returns
    fp32 [B, Hq, n_q, d]."""
    _dev(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be [B, Hq, n_q, d]")
    B, Hq, nq, d = q.shape
    in_code = -1
    if k_new is not None or v_new is not None:
        _dev(k_new, "k_new")
        _dev(v_new, "v_new")
        if k_new.dtype not in _CODE or v_new.dtype != k_new.dtype or k_new.shape != v_new.shape:
            raise TypeError("k_new/v_new must be matching f32 or bf16 tensors")
        if tuple(k_new.shape) != (B, cache.num_kv_heads, nq, cache.head_dim):
            raise ValueError("k_new shape %s does not match [B, Hkv, n_q, d]" % (tuple(k_new.shape),))
        in_code = _CODE[k_new.dtype]
    if out is None:
        out = torch.empty((B, Hq, nq, d), dtype=torch.float32, device=q.device)
    # query i of head h is column h * n_q + i: q and out viewed as [B, Hq * n_q, d]
    _, _, scale, _, workspace, mb, stride = _decode_args(cache, q.view(B, Hq * nq, d), seq_lens, max_seq_len,
                                                         block_table, key_mask, scale, out.view(B, Hq * nq, d),
                                                         workspace, part_tokens)
    check(lib().kvattn_attn_decode_multi(ctypes.byref(cache.desc()), B, Hq, nq, _ptr(q), _CODE.get(q.dtype, -1),
                                         _ptr(k_new), _ptr(v_new), in_code, _ptr(seq_lens), int(max_seq_len),
                                         _ptr(block_table), mb, _ptr(key_mask), stride, scale, _ptr(out),
                                         _ptr(workspace), workspace.numel() * workspace.element_size(),
                                         int(part_tokens), _stream(q.device)))
    return out

def attn_prefill(q, k, v, cache=None, positions=None, q_lens=None, block_table=None, key_mask=None, causal=True,
                 attend_prefix=False, scale=None, out=None):
    """Attention of n_max new tokens per sequence (kvattn_attn_prefill).

    q: [B, Hq, n_max, d]; k, v: [B, Hkv, n_max, d] (f32 or bf16).  With a cache
    the new K/V are written at positions[b] + t; attend_prefix also attends
    the cached positions < positions[b].  Returns fp32 [B, Hq, n_max, d].
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    _i32(positions, "positions")
    _i32(q_lens, "q_lens")
    _i32(block_table, "block_table")
    _dev(key_mask, "key_mask")
    if key_mask is not None and key_mask.dtype != torch.uint8:
        raise TypeError("key_mask must be uint8")
    if q.dtype not in _CODE or k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share one dtype, f32 or bf16")
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, n, d) or v.shape != k.shape:
        raise ValueError("k/v shape %s incompatible with q %s" % (tuple(k.shape), tuple(q.shape)))
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, n, d), dtype=torch.float32, device=q.device)
    _dev(out, "out")
    desc = ctypes.byref(cache.desc()) if cache is not None else None
    mb = block_table.shape[1] if block_table is not None else 0
    stride = key_mask.shape[1] if key_mask is not None else 0
    check(lib().kvattn_attn_prefill(desc, B, Hq, Hkv, d, n, _ptr(q), _ptr(k), _ptr(v), _CODE[q.dtype], _ptr(positions),
                                    _ptr(q_lens), _ptr(block_table), mb, _ptr(key_mask), stride, int(bool(causal)),
                                    int(bool(attend_prefix)), float(scale), _ptr(out), _stream(q.device)))
    return out


def validate(cache, seq_lens, max_seq_len, positions=None, block_table=None):
    """Device check of the cache metadata contract (kvattn_validate).
    Returns the OR of VALIDATE_* bits (synchronises the stream to read it)."""
    _i32(seq_lens, "seq_lens")
    _i32(positions, "positions")
    _i32(block_table, "block_table")
    err = torch.zeros(1, dtype=torch.int32, device=seq_lens.device)
    mb = block_table.shape[1] if block_table is not None else 0
    check(lib().kvattn_validate(ctypes.byref(cache.desc()), seq_lens.shape[0], _ptr(seq_lens), int(max_seq_len),
                                _ptr(positions), _ptr(block_table), mb, _ptr(err), _stream(seq_lens.device)))
    return int(err.item())


# ------------------------------------------------ cache reorder and sharing ---

def reorder_rows(perm, src_table, src_lens=None, dst_table=None, dst_lens=None):
    """Batch/beam reorder of a paged cache's block table (kvattn_reorder_rows):
    row i of the result is row perm[i].  Device int32 tensors; returns
    (dst_table, dst_lens or None)."""
    _i32(perm, "perm")
    _i32(src_table, "src_table")
    _i32(src_lens, "src_lens")
    n = perm.shape[0]
    rows, mb = src_table.shape
    if dst_table is None:
        dst_table = torch.empty((n, mb), dtype=torch.int32, device=src_table.device)
    if src_lens is not None and dst_lens is None:
        dst_lens = torch.empty(n, dtype=torch.int32, device=src_table.device)
    _i32(dst_table, "dst_table")
    _i32(dst_lens, "dst_lens")
    check(lib().kvattn_reorder_rows(n, _ptr(perm), rows, _ptr(src_table), _ptr(src_lens), mb, _ptr(dst_table),
                                    _ptr(dst_lens), _stream(src_table.device)))
    return dst_table, dst_lens


def reorder_cache(src, dst, perm, src_lens=None, dst_lens=None):
    """Batch/beam reorder of a contiguous cache (kvattn_reorder_cache): dst
    row i receives the first src_lens[perm[i]] positions (all, without
    src_lens) of src row perm[i].  Returns dst_lens (or None)."""
    _i32(perm, "perm")
    _i32(src_lens, "src_lens")
    _i32(dst_lens, "dst_lens")
    check(lib().kvattn_reorder_cache(ctypes.byref(src.desc()), ctypes.byref(dst.desc()), perm.shape[0], _ptr(perm),
                                     _ptr(src_lens), _ptr(dst_lens), _stream(perm.device)))
    return dst_lens


def copy_blocks(cache, src_blocks, dst_blocks):
    """Copy whole physical blocks of a paged cache, K and V
    (kvattn_copy_blocks): block dst_blocks[i] receives block src_blocks[i]."""
    _i32(src_blocks, "src_blocks")
    _i32(dst_blocks, "dst_blocks")
    if src_blocks.shape != dst_blocks.shape or src_blocks.dim() != 1:
        raise ValueError("src_blocks and dst_blocks must be 1-D of one length")
    check(lib().kvattn_copy_blocks(ctypes.byref(cache.desc()), src_blocks.shape[0], _ptr(src_blocks),
                                   _ptr(dst_blocks), _stream(cache.device)))


def stream_read(x, sink=None):
    """One plain streaming read of the device tensor x (kvattn_stream_read, a
    measurement helper): returns sink, an int32 [1] tensor (allocated as 0
    when None) XORed with the XOR of all 32-bit words of x."""
    _dev(x, "x")
    nbytes = x.numel() * x.element_size()
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=x.device)
    _i32(sink, "sink")
    check(lib().kvattn_stream_read(_ptr(x), nbytes, _ptr(sink), _stream(x.device)))
    return sink


def _host_i32(a, name, writable=False):
    if not isinstance(a, np.ndarray) or a.dtype != np.int32 or not a.flags.c_contiguous:
        raise TypeError("%s must be a C-contiguous numpy int32 array" % name)
    if writable and not a.flags.writeable:
        raise ValueError("%s must be writable" % name)
    return ctypes.c_void_p(a.ctypes.data)


class BlockPool:
    """Host block pool with reference counts (kvattn_pool_*).  Tables, lengths
    and id lists are host numpy int32 arrays; tables are [rows, max_blocks]
    with -1 for no block and are updated in place where the C call does."""

    def __init__(self, num_blocks):
        h = lib().kvattn_pool_create(int(num_blocks))
        if not h:
            raise _lib.KvattnError(_lib.EINVAL, lib().kvattn_last_error().decode())
        self._h = ctypes.c_void_p(h)
        self._destroy = lib().kvattn_pool_destroy  # kept for destruction at interpreter exit

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    @property
    def num_blocks(self):
        return int(lib().kvattn_pool_num_blocks(self._h))

    def num_free(self):
        return int(lib().kvattn_pool_num_free(self._h))

    def refcount(self, block):
        return int(lib().kvattn_pool_refcount(self._h, int(block)))

    def alloc(self, n):
        ids = np.empty(max(int(n), 1), dtype=np.int32)
        check(lib().kvattn_pool_alloc(self._h, int(n), _host_i32(ids, "ids")))
        return ids[:int(n)]

    def retain(self, ids):
        check(lib().kvattn_pool_retain(self._h, ids.shape[0], _host_i32(ids, "ids")))

    def release(self, ids):
        check(lib().kvattn_pool_release(self._h, ids.shape[0], _host_i32(ids, "ids")))

    def fork(self, src_row, length, dst_row=None):
        if dst_row is None:
            dst_row = np.full(src_row.shape[0], -1, dtype=np.int32)
        check(lib().kvattn_pool_fork(self._h, _host_i32(src_row, "src_row"), _host_i32(dst_row, "dst_row", True),
                                     src_row.shape[0], int(length)))
        return dst_row

    def free_seq(self, row, length):
        check(lib().kvattn_pool_free_seq(self._h, _host_i32(row, "row", True), row.shape[0], int(length)))

    def prepare_append(self, tables, cur_lens, new_lens):
        """Updates tables [rows, max_blocks] in place; returns the
        copy-on-write pairs (src, dst) as two int32 arrays."""
        rows, mb = tables.shape
        cs = np.empty(max(rows, 1), dtype=np.int32)
        cd = np.empty(max(rows, 1), dtype=np.int32)
        n = ctypes.c_int32(0)
        check(lib().kvattn_pool_prepare_append(self._h, rows, _host_i32(tables, "tables", True), mb,
                                               _host_i32(cur_lens, "cur_lens"), _host_i32(new_lens, "new_lens"),
                                               _host_i32(cs, "copy_src", True), _host_i32(cd, "copy_dst", True),
                                               ctypes.byref(n)))
        return cs[:n.value], cd[:n.value]

    def reorder(self, perm, src_tables, src_lens):
        n = perm.shape[0]
        rows, mb = src_tables.shape
        dt = np.empty((n, mb), dtype=np.int32)
        dl = np.empty(max(n, 1), dtype=np.int32)
        check(lib().kvattn_pool_reorder(self._h, n, _host_i32(perm, "perm"), rows, _host_i32(src_tables, "src_tables"),
                                        _host_i32(src_lens, "src_lens"), mb, _host_i32(dt, "dst_tables", True),
                                        _host_i32(dl, "dst_lens", True)))
        return dt, dl[:n]
