"""Batch/beam reorder and copy-on-write block copies on the GPU against the
oracle (oracle/paging.py): bit-exact, since they move integers and bytes.
The end-to-end case forks beams off a cached prompt with the host pool,
copies the shared partial block, appends and decodes, and checks the
attention output against the oracle's decode of each beam's logical cache.

Page keys:
  [P2] "KV Cache Fully Explained" section "(4) PagedAttention"
  [P4] "Transformer Attention Masks and KV-Cache Inference" section
       "Batch and beam reorder"
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K
from kv_cache_decode_attn_amd import synth
from oracle import attention as OA
from oracle import cache as OC
from oracle import paging as P
from tests.helpers import f64, storage

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-3  # bf16 cache, fp32 accumulation: the decode parity bound


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _canary(shape, tdt, seed):
    n = int(np.prod(shape)) * torch.tensor([], dtype=tdt).element_size()
    t = torch.from_numpy(synth.rng(*seed).integers(0, 256, size=n, dtype=np.uint8)).view(tdt).reshape(shape)
    return t


# ------------------------------------------------------------ table rows ---

@pytest.mark.parametrize("with_lens", [True, False])
def test_reorder_rows_bit_exact(with_lens):
    rng = synth.rng(30, synth.T_PERM)
    rows, mb = 37, 300                          # two workgroups per row, ragged second one
    table = rng.integers(-1, 5000, size=(rows, mb)).astype(np.int32)
    lens = rng.integers(0, 16 * mb, size=rows).astype(np.int32)
    perm = rng.integers(0, rows, size=41).astype(np.int32)      # repeats: beams sharing a parent
    perm[[3, 17, 40]] = [-1, rows, 1 << 30]                      # out of range: empty rows
    want_t, want_l = P.reorder_rows(table, lens if with_lens else None, perm)
    got_t, got_l = K.reorder_rows(_dev(perm), _dev(table), _dev(lens) if with_lens else None)
    np.testing.assert_array_equal(got_t.cpu().numpy(), want_t)
    if with_lens:
        np.testing.assert_array_equal(got_l.cpu().numpy(), want_l)
    else:
        assert got_l is None


def test_reorder_rows_printed_example():
    """[P4]: rows [A0, A1, B0], permutation [2, 1, 0] -> [B0, A1, A0]."""
    table = np.array([[10, 11], [20, 21], [30, 31]], dtype=np.int32)     # A0, A1, B0
    lens = np.array([17, 18, 19], dtype=np.int32)
    t, l = K.reorder_rows(_dev(np.array([2, 1, 0], np.int32)), _dev(table), _dev(lens))
    np.testing.assert_array_equal(t.cpu().numpy(), [[30, 31], [20, 21], [10, 11]])
    np.testing.assert_array_equal(l.cpu().numpy(), [19, 18, 17])


# ------------------------------------------------------- contiguous rows ---

@pytest.mark.parametrize("dtype,d", [(K.BF16, 128), (K.F32, 64), (K.FP8_E4M3, 64), (K.FP8_E4M3, 128)])
@pytest.mark.parametrize("with_lens", [True, False])
def test_reorder_cache_bit_exact(dtype, d, with_lens):
    tdt = {K.BF16: torch.bfloat16, K.F32: torch.float32, K.FP8_E4M3: torch.uint8}[dtype]
    Hkv, cap, src_rows, n = 3, 160, 5, 7      # 160 positions x 256 B = 2.5 chunks per head row (bf16)
    sk = _canary((src_rows, Hkv, cap, d), tdt, (31, 1))
    sv = _canary((src_rows, Hkv, cap, d), tdt, (31, 2))
    dk = _canary((n, Hkv, cap, d), tdt, (31, 3))
    dv = _canary((n, Hkv, cap, d), tdt, (31, 4))
    lens = np.array([0, 1, 77, 160, 999], dtype=np.int32)          # 999 clamps to the capacity
    perm = np.array([2, 4, 2, -3, 3, 1, 0], dtype=np.int32)
    want_k, want_l = P.reorder_contiguous(storage(sk), storage(dk), perm, lens if with_lens else None)
    want_v, _ = P.reorder_contiguous(storage(sv), storage(dv), perm, lens if with_lens else None)
    scales = {}
    if dtype == K.FP8_E4M3:
        scales = dict(k_scale=torch.ones(Hkv, device=DEV), v_scale=torch.ones(Hkv, device=DEV))
    src = K.KVCache(sk.to(DEV), sv.to(DEV), K.CONTIGUOUS, dtype, **scales)
    dst = K.KVCache(dk.to(DEV), dv.to(DEV), K.CONTIGUOUS, dtype, **scales)
    out_l = torch.full((n,), -7, dtype=torch.int32, device=DEV) if with_lens else None
    K.reorder_cache(src, dst, _dev(perm), _dev(lens) if with_lens else None, out_l)
    np.testing.assert_array_equal(storage(dst.k), want_k)
    np.testing.assert_array_equal(storage(dst.v), want_v)
    if with_lens:
        np.testing.assert_array_equal(out_l.cpu().numpy(), want_l)


# ----------------------------------------------------------- block copies ---

@pytest.mark.parametrize("dtype,hkv,d", [(K.BF16, 8, 128), (K.FP8_E4M3, 1, 64), (K.F32, 2, 64)])
def test_copy_blocks_bit_exact(dtype, hkv, d):
    tdt = {K.BF16: torch.bfloat16, K.F32: torch.float32, K.FP8_E4M3: torch.uint8}[dtype]
    nblk = 40
    pk = _canary((nblk, hkv, 16, d), tdt, (32, 1))
    pv = _canary((nblk, hkv, 16, d), tdt, (32, 2))
    src = np.array([0, 5, 7, 39, 50, -1, 12], dtype=np.int32)
    dst = np.array([20, 21, 22, 23, 24, 25, -9], dtype=np.int32)    # pairs 4, 5, 6 skipped
    want_k = P.copy_blocks(storage(pk), src, dst)
    want_v = P.copy_blocks(storage(pv), src, dst)
    scales = {}
    if dtype == K.FP8_E4M3:
        scales = dict(k_scale=torch.ones(hkv, device=DEV), v_scale=torch.ones(hkv, device=DEV))
    cache = K.KVCache(pk.to(DEV), pv.to(DEV), K.PAGED, dtype, **scales)
    K.copy_blocks(cache, _dev(src), _dev(dst))
    np.testing.assert_array_equal(storage(cache.k), want_k)
    np.testing.assert_array_equal(storage(cache.v), want_v)


# ------------------------------------------- fork, copy-on-write, decode ---

def _decode_ref(q, keys, vals, lens):
    return OA.decode(f64(q), keys, vals, lens, 1.0 / math.sqrt(q.shape[-1]))


def test_beam_fork_copy_on_write_reorder_decode():
    """Three beams fork off a 37-token prompt ([P2]: shared blocks,
    copy-on-write), each appends and decodes its own token; the beams are
    then reordered with repeats ([P4]) and decode once more.  Every output
    matches the oracle's decode of that beam's logical cache, and the
    prompt's own blocks never change."""
    Hkv, Hq, d, mb, nblk = 2, 8, 128, 4, 16
    prompt = 37
    pool = K.BlockPool(nblk)
    cache = K.KVCache.paged(nblk, Hkv, d, K.BF16, fill=0.0)
    # the prompt: one row, written through kv_append
    root = np.full((1, mb), -1, dtype=np.int32)
    pool.prepare_append(root, np.zeros(1, np.int32), np.array([prompt], np.int32))
    pk = synth.normal((1, Hkv, prompt, d), (33, synth.T_K))
    pv = synth.normal((1, Hkv, prompt, d), (33, synth.T_V))
    K.kv_append(cache, pk.to(DEV), pv.to(DEV), _dev(np.zeros(1, np.int32)), block_table=_dev(root))
    root_k_before = storage(cache.k)[root[0, :3]].copy()

    # three beams share the prompt's blocks
    beams = np.stack([pool.fork(root[0], prompt) for _ in range(3)])
    assert pool.refcount(int(root[0, 2])) == 4
    lens = np.full(3, prompt, dtype=np.int32)
    cs, cd = pool.prepare_append(beams, lens, lens + 1)
    assert len(cs) == 3 and set(cs.tolist()) == {int(root[0, 2])}       # partial block copied per beam
    K.copy_blocks(cache, _dev(cs), _dev(cd))

    keys = [[f64(pk[0, g]) for g in range(Hkv)] for _ in range(3)]
    vals = [[f64(pv[0, g]) for g in range(Hkv)] for _ in range(3)]

    def step(tables, lens_before, seed):
        q = synth.normal((3, Hq, d), (seed, synth.T_Q))
        kn = synth.normal((3, Hkv, d), (seed, synth.T_KNEW))
        vn = synth.normal((3, Hkv, d), (seed, synth.T_VNEW))
        out = K.attn_decode_append(cache, q.to(DEV), kn.to(DEV), vn.to(DEV), _dev(lens_before + 1),
                                   int(lens_before.max()) + 1, block_table=_dev(tables))
        for b in range(3):
            for g in range(Hkv):
                keys[b][g] = np.concatenate([keys[b][g], f64(kn[b, g])[None]])
                vals[b][g] = np.concatenate([vals[b][g], f64(vn[b, g])[None]])
        want = _decode_ref(q, [np.stack(k) for k in keys], [np.stack(v) for v in vals], lens_before + 1)
        assert np.max(np.abs(out.cpu().numpy() - want)) < TOL

    step(beams, lens, 34)
    lens = lens + 1
    # the prompt's blocks are untouched by the beams' writes
    np.testing.assert_array_equal(storage(cache.k)[root[0, :3]], root_k_before)

    # reorder with repeats: the device gather equals the host pool's rows
    perm = np.array([2, 0, 0], dtype=np.int32)
    host_t, host_l = pool.reorder(perm, beams, lens)
    dev_t, dev_l = K.reorder_rows(_dev(perm), _dev(beams), _dev(lens))
    np.testing.assert_array_equal(dev_t.cpu().numpy(), host_t)
    np.testing.assert_array_equal(dev_l.cpu().numpy(), host_l)
    keys = [[k.copy() for k in keys[int(p)]] for p in perm]
    vals = [[v.copy() for v in vals[int(p)]] for p in perm]
    beams, lens = host_t, host_l.astype(np.int32)
    # rows 1 and 2 now share beam 0's partial block: each write copies it
    cs, cd = pool.prepare_append(beams, lens, lens + 1)
    assert len(cs) == 1
    K.copy_blocks(cache, _dev(cs), _dev(cd))
    step(beams, lens, 35)
    lens = lens + 1
    for r in range(3):
        pool.free_seq(beams[r], int(lens[r]))
    pool.free_seq(root[0], prompt)
    assert pool.num_free() == nblk


# ---------------------------------------------------------- full sizes ---

@pytest.mark.slow
def test_copy_blocks_full_size_sampled():
    """The benchmark's block-copy launch: 4096 pairs of 32 KiB Llama-3-8B
    bf16 blocks (8 KV heads x 16 positions x 128) in a 16384-block pool;
    sampled pairs compared with the oracle's copy of those blocks."""
    nblk, n, Hkv, d = 16384, 4096, 8, 128
    cache = K.KVCache.paged(nblk, Hkv, d, K.BF16)
    synth.normal_device(cache.k.shape, (40, synth.T_K), out=cache.k)
    synth.normal_device(cache.v.shape, (40, synth.T_V), out=cache.v)
    perm = synth.rng(40, synth.T_PERM).permutation(nblk).astype(np.int32)
    src, dst = perm[:n], perm[n:2 * n]
    pick = synth.rng(40, 99).choice(n, 24, replace=False)
    before_k = {i: storage(cache.k[int(src[i])]) for i in pick}
    before_v = {i: storage(cache.v[int(src[i])]) for i in pick}
    untouched = int(perm[2 * n])
    keep = storage(cache.k[untouched])
    K.copy_blocks(cache, _dev(src), _dev(dst))
    torch.cuda.synchronize()
    for i in pick:
        np.testing.assert_array_equal(storage(cache.k[int(dst[i])]), before_k[i])
        np.testing.assert_array_equal(storage(cache.v[int(dst[i])]), before_v[i])
    np.testing.assert_array_equal(storage(cache.k[untouched]), keep)


@pytest.mark.slow
def test_reorder_cache_full_size_sampled():
    """The benchmark's contiguous beam reorder: 32 rows (8 prompts x 4
    beams), 8 KV heads, capacity 4096, d = 128, bf16, lengths in
    [1024, 4096]; sampled rows compared with the oracle's gather."""
    rows, Hkv, cap, d = 32, 8, 4096, 128
    src = K.KVCache.contiguous(rows, Hkv, cap, d, K.BF16)
    dst = K.KVCache.contiguous(rows, Hkv, cap, d, K.BF16, fill=0.0)
    synth.normal_device(src.k.shape, (41, synth.T_K), out=src.k)
    synth.normal_device(src.v.shape, (41, synth.T_V), out=src.v)
    lens = synth.uniform_lengths(rows, 1024, cap, (41, synth.T_LENS))
    r = synth.rng(41, synth.T_PERM)
    perm = np.concatenate([4 * p + r.integers(0, 4, size=4) for p in range(8)]).astype(np.int32)
    out_l = torch.empty(rows, dtype=torch.int32, device=DEV)
    K.reorder_cache(src, dst, _dev(perm), _dev(lens), out_l)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_l.cpu().numpy(), lens[perm])
    for i in synth.rng(41, 98).choice(rows, 6, replace=False):
        p = int(perm[i])
        s = storage(src.k[p:p + 1])
        want, _ = P.reorder_contiguous(s, storage(dst.k[i:i + 1]).copy() * 0, [0], lens[p:p + 1])
        np.testing.assert_array_equal(storage(dst.k[i:i + 1]), want)
