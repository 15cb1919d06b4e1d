"""The allocation-free decode step (attn_decode_append_noalloc) through the
C ABI: on two calls in a row - the second with a smaller batch, fewer keys
and a different partitioning - its output and cache bytes equal those of
attn_decode_append with a caller workspace bit for bit, and both are within
the bf16 tolerance of the fp64 oracle.  Sizes past the static scratch are
refused before anything runs."""
import math

import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K
from kv_cache_decode_attn_amd import synth
from oracle import attention as OA
from tests.helpers import f64, max_abs, storage

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-3


def _problem(B, lens, seed, Hq=32, Hkv=8, d=128):
    """A paged bf16 decode step: logical K/V of every position, the caches
    filled up to the last position (which the step stores), the query."""
    lens = np.asarray(lens, np.int32)
    width = int(lens.max())
    k = synth.normal((B, Hkv, width, d), (seed, synth.T_K))
    v = synth.normal((B, Hkv, width, d), (seed, synth.T_V))
    q = synth.normal((B, Hq, d), (seed, synth.T_Q))
    nbs = [synth.blocks_for(x) for x in lens]
    table, nblk = synth.block_table(nbs, max(nbs), (seed, synth.T_PERM))
    tdev = torch.from_numpy(table).to(DEV)
    before = torch.from_numpy(lens - 1).to(DEV)
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    caches = []
    for _ in range(2):
        c = K.KVCache.paged(nblk, Hkv, d, K.BF16, DEV, fill=0.0)
        K.kv_append(c, k.to(DEV), v.to(DEV), zeros, block_table=tdev, n_valid=before)
        caches.append(c)
    idx = torch.from_numpy((lens - 1).astype(np.int64)).view(B, 1, 1, 1).expand(B, Hkv, 1, d)
    k_new = torch.gather(k, 2, idx)[:, :, 0].contiguous()
    v_new = torch.gather(v, 2, idx)[:, :, 0].contiguous()
    return dict(lens=lens, k=k, v=v, q=q, table=tdev, caches=caches, k_new=k_new, v_new=v_new, d=d, Hq=Hq)


def _check(p, part_tokens):
    B = len(p["lens"])
    seq_lens = torch.from_numpy(p["lens"]).to(DEV)
    maxlen = int(p["lens"].max())
    q, kn, vn = p["q"].to(DEV), p["k_new"].to(DEV), p["v_new"].to(DEV)
    ws = K.decode_workspace(p["caches"][0], B, p["Hq"], maxlen, part_tokens)
    ref = K.attn_decode_append(p["caches"][0], q, kn, vn, seq_lens, maxlen, block_table=p["table"], workspace=ws,
                               part_tokens=part_tokens)
    out = torch.full_like(ref, float("nan"))
    K.attn_decode_append_noalloc(p["caches"][1], q, kn, vn, seq_lens, maxlen, block_table=p["table"], out=out,
                                 part_tokens=part_tokens)
    torch.cuda.synchronize()
    got, want = out.cpu().numpy(), ref.cpu().numpy()
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(storage(p["caches"][1].k), storage(p["caches"][0].k))
    np.testing.assert_array_equal(storage(p["caches"][1].v), storage(p["caches"][0].v))
    kf, vf = f64(p["k"]), f64(p["v"])
    oracle = OA.decode(f64(p["q"]), [kf[b] for b in range(B)], [vf[b] for b in range(B)], p["lens"],
                       1.0 / math.sqrt(p["d"]))
    assert max_abs(got, oracle) <= TOL


def test_noalloc_equals_workspace_call_twice_second_smaller():
    # first call: 6 sequences up to 3000 keys over 256-key partitions (12
    # partials per head); second: 3 sequences up to 700 keys over 128-key
    # partitions, which reads back slots the first call left behind
    first = _problem(6, [3000, 1, 17, 2049, 512, 1500], seed=81)
    _check(first, 256)
    ws_first = K.decode_workspace_bytes(K.BF16, 6, 32, 8, 128, 3000, 256)
    second = _problem(3, [700, 129, 33], seed=82)
    _check(second, 128)
    assert 0 < K.decode_workspace_bytes(K.BF16, 3, 32, 8, 128, 700, 128) < ws_first <= K.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_sizes_past_the_scratch():
    p = _problem(1, [64], seed=83)
    big = 1 << 20  # 4096 partitions of 256 keys: far more partials than the scratch holds
    assert K.decode_workspace_bytes(K.BF16, 1, 32, 8, 128, big, 256) > K.NOALLOC_SCRATCH_BYTES
    with pytest.raises(K.KvattnError) as e:
        K.attn_decode_append_noalloc(p["caches"][1], p["q"].to(DEV), p["k_new"].to(DEV), p["v_new"].to(DEV),
                                     torch.from_numpy(p["lens"]).to(DEV), big, block_table=p["table"],
                                     part_tokens=256)
    assert e.value.status == K.EWORKSPACE
    assert "static scratch" in str(e.value)
