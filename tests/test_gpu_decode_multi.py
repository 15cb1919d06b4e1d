"""Several query tokens per sequence against the cache (kvattn_attn_decode_multi)
vs the fp64 oracle: the same result as a chunked prefill that attends the
cached prefix ("Transformer Attention Masks and KV-Cache Inference", sections
"Prefill and decode stages" and "Causal mask and future positions"), computed
as a split-K decode."""
import math

import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K
from kv_cache_decode_attn_amd import synth
from oracle import attention as OA
from oracle import cache as OC
from tests.helpers import f64, max_abs, storage

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-3
_TORCH = {K.F32: torch.float32, K.BF16: torch.bfloat16, K.FP8_E4M3: torch.bfloat16}
_OC = {K.F32: OC.F32, K.BF16: OC.BF16, K.FP8_E4M3: OC.FP8_E4M3}


def _case(lens, n_q, Hq, Hkv, d, dtype, layout, seed, mask=None, parts=(64,)):
    """Cache holding every sequence's lens[b] positions, the last n_q of them
    the new tokens (appended like any other); q [B, Hq, n_q, d].  Returns the
    GPU output and the oracle's."""
    lens = np.asarray(lens, np.int32)
    B = len(lens)
    total = int(lens.max())
    tdt = _TORCH[dtype]
    kx = synth.normal((B, Hkv, total, d), (seed, synth.T_K), tdt)
    vx = synth.normal((B, Hkv, total, d), (seed, synth.T_V), tdt)
    q = synth.normal((B, Hq, n_q, d), (seed, synth.T_Q), tdt)
    ks = vs = None
    if dtype == K.FP8_E4M3:
        sc = synth.fp8_scales(2 * Hkv, (seed, synth.T_SCALE)).reshape(2, Hkv)
        ks = torch.from_numpy(sc[0]).to(DEV)
        vs = torch.from_numpy(sc[1]).to(DEV)
    table = tdev = None
    if layout == K.PAGED:
        nbs = [synth.blocks_for(int(x)) for x in lens]
        table, nblk = synth.block_table(nbs, max(nbs), (seed, synth.T_PERM))
        tdev = torch.from_numpy(table).to(DEV)
        cache = K.KVCache.paged(nblk, Hkv, d, dtype, DEV, ks, vs)
    else:
        cache = K.KVCache.contiguous(B, Hkv, -(-total // 16) * 16, d, dtype, DEV, ks, vs)
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    K.kv_append(cache, kx.to(DEV), vx.to(DEV), zeros, block_table=tdev, n_valid=torch.from_numpy(lens).to(DEV))
    seq = torch.from_numpy(lens).to(DEV)
    kmask = torch.from_numpy(mask).to(DEV) if mask is not None else None
    got = [K.attn_decode_multi(cache, q.to(DEV), seq, total, block_table=tdev, key_mask=kmask,
                               part_tokens=pt).cpu().numpy() for pt in parts]
    got = got[0] if len(got) == 1 else got
    got_default = K.attn_decode_multi(cache, q.to(DEV), seq, total, block_table=tdev, key_mask=kmask)
    # oracle: the keys are the cached values as the cache holds them (fp8:
    # the oracle's own encoding, dequantised)
    kf, vf = [], []
    for b in range(B):
        if dtype == K.FP8_E4M3:
            kb = np.stack([OC.to_f64(OC.encode_rows(storage(kx)[b, g], OC.BF16, OC.FP8_E4M3, np.float32(sc[0][g])),
                                     OC.FP8_E4M3, np.float32(sc[0][g])) for g in range(Hkv)])
            vb = np.stack([OC.to_f64(OC.encode_rows(storage(vx)[b, g], OC.BF16, OC.FP8_E4M3, np.float32(sc[1][g])),
                                     OC.FP8_E4M3, np.float32(sc[1][g])) for g in range(Hkv)])
        else:
            kb, vb = f64(kx[b]), f64(vx[b])
        kf.append(kb)
        vf.append(vb)
    P = np.maximum(lens - n_q, 0)
    nq = np.minimum(lens, n_q).astype(np.int32)
    knew = np.zeros((B, Hkv, n_q, d))
    vnew = np.zeros((B, Hkv, n_q, d))
    qn = f64(q)
    qo = np.zeros_like(qn)
    for b in range(B):
        knew[b, :, :nq[b]] = kf[b][:, P[b]:lens[b]]
        vnew[b, :, :nq[b]] = vf[b][:, P[b]:lens[b]]
        # a sequence shorter than n_q holds queries n_q - len .. n_q - 1
        qo[b, :, :nq[b]] = qn[b, :, n_q - nq[b]:]
    want_o = OA.prefill(qo, knew, vnew, P, nq, 1.0 / math.sqrt(d), causal=True, key_mask=mask,
                        prefix_k=kf, prefix_v=vf, attend_prefix=True)
    want = np.zeros_like(want_o)
    for b in range(B):
        want[b, :, n_q - nq[b]:] = want_o[b, :, :nq[b]]
    return got, got_default.cpu().numpy(), want


@pytest.mark.parametrize("dtype,G,n_q", [
    (K.BF16, 4, 4),    # 16 columns per KV head, matrix-core pass
    (K.BF16, 8, 2),    # 16 columns
    (K.BF16, 2, 4),    # 8 columns, matrix-core pass
    (K.BF16, 1, 2),    # 2 columns, vector pass
    (K.FP8_E4M3, 8, 2),  # 16 columns, fp8 matrix-core pass
    (K.FP8_E4M3, 1, 2),  # fp8 vector pass
    (K.F32, 2, 2),     # f32 cache
])
@pytest.mark.parametrize("layout", [K.PAGED, K.CONTIGUOUS])
def test_decode_multi_matches_prefill_with_prefix(dtype, G, n_q, layout):
    Hkv, d = 2, 128
    lens = [1000, 70, 513, 17]
    got, got_d, want = _case(lens, n_q, G * Hkv, Hkv, d, dtype, layout, 80 + G + n_q)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL
    assert max_abs(got_d, want) <= TOL


@pytest.mark.parametrize("d", [64, 128])
def test_decode_multi_key_mask(d):
    lens = [300, 129, 40]
    mask = synth.random_mask((3, 320), 0.7, (81, synth.T_MASK))
    mask[:, 0] = 1
    got, got_d, want = _case(lens, 4, 16, 4, d, K.BF16, K.PAGED, 82, mask=mask)
    assert max_abs(got, want) <= TOL
    assert max_abs(got_d, want) <= TOL


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask_on", [False, True])
def test_decode_multi_16_columns_long_partitions(d, mask_on):
    """The 16-column bf16 pass keeps no per-key scores, so any partition size
    is allowed: 64 (many partials), 1024 (the default), 3072 and 8192 (one
    partition per sequence, with lengths past and below it)."""
    lens = [5000, 1025, 3072, 31, 4097]
    mask = None
    if mask_on:
        mask = synth.random_mask((5, 5008), 0.8, (85, synth.T_MASK))
        mask[:, 0] = 1
    got, got_d, want = _case(lens, 4, 16, 4, d, K.BF16, K.PAGED, 84, mask=mask, parts=(64, 1024, 3072, 8192))
    for g in got + [got_d]:
        assert np.isfinite(g).all()
        assert max_abs(g, want) <= TOL


def test_decode_multi_one_query_is_decode_bitwise():
    """n_q = 1 is the plain decode, bit for bit."""
    B, Hq, Hkv, d = 3, 8, 2, 128
    lens = np.array([700, 1, 300], np.int32)
    kx = synth.normal((B, Hkv, 700, d), (83, synth.T_K), torch.bfloat16)
    vx = synth.normal((B, Hkv, 700, d), (83, synth.T_V), torch.bfloat16)
    q = synth.normal((B, Hq, d), (83, synth.T_Q), torch.bfloat16).to(DEV)
    cache = K.KVCache.contiguous(B, Hkv, 704, d, K.BF16, DEV)
    K.kv_append(cache, kx.to(DEV), vx.to(DEV), torch.zeros(B, dtype=torch.int32, device=DEV),
                n_valid=torch.from_numpy(lens).to(DEV))
    seq = torch.from_numpy(lens).to(DEV)
    a = K.attn_decode(cache, q, seq, 700, part_tokens=128)
    m = K.attn_decode_multi(cache, q[:, :, None], seq, 700, part_tokens=128)
    assert torch.equal(a, m[:, :, 0])


def test_decode_multi_rejects_unsupported_groups():
    cache = K.KVCache.paged(4, 2, 64, K.BF16, DEV)
    q = torch.zeros((1, 8, 3, 64), dtype=torch.bfloat16, device=DEV)   # G 4 x 3 queries = 12 columns
    seq = torch.tensor([10], dtype=torch.int32, device=DEV)
    table = torch.zeros((1, 4), dtype=torch.int32, device=DEV)
    with pytest.raises(K.KvattnError):
        K.attn_decode_multi(cache, q, seq, 10, block_table=table)


@pytest.mark.parametrize("dtype,G,n_q,layout", [
    (K.BF16, 4, 4, K.PAGED),
    (K.BF16, 2, 2, K.CONTIGUOUS),
    (K.FP8_E4M3, 8, 2, K.PAGED),
    (K.FP8_E4M3, 1, 4, K.CONTIGUOUS),
    (K.F32, 2, 2, K.PAGED),
])
def test_decode_multi_fused_append_equals_append_then_attend(dtype, G, n_q, layout):
    """Given k_new/v_new, the call stores the n_q rows itself: the cache bytes
    and the output equal kv_append(n_q) followed by the call without them, bit
    for bit - also when the new positions straddle two partitions (64 keys
    each: lengths 66 and 130)."""
    Hkv, d = 2, 128
    Hq = G * Hkv
    lens = np.array([66, 130, 5, 700], np.int32)
    B = len(lens)
    total = int(lens.max())
    tdt = _TORCH[dtype]
    kx = synth.normal((B, Hkv, total, d), (90, synth.T_K), tdt)
    vx = synth.normal((B, Hkv, total, d), (90, synth.T_V), tdt)
    q = synth.normal((B, Hq, n_q, d), (90, synth.T_Q), tdt).to(DEV)
    ks = vs = None
    if dtype == K.FP8_E4M3:
        ks = torch.full((Hkv,), 0.7, dtype=torch.float32, device=DEV)
        vs = torch.full((Hkv,), 1.3, dtype=torch.float32, device=DEV)
    tdev = None

    def make():
        nonlocal tdev
        if layout == K.PAGED:
            nbs = [synth.blocks_for(int(x)) for x in lens]
            table, nblk = synth.block_table(nbs, max(nbs), (90, synth.T_PERM))
            tdev = torch.from_numpy(table).to(DEV)
            c = K.KVCache.paged(nblk, Hkv, d, dtype, DEV, ks, vs)
        else:
            c = K.KVCache.contiguous(B, Hkv, -(-total // 16) * 16, d, dtype, DEV, ks, vs)
        c.k.zero_()
        c.v.zero_()
        # everything but the last n_q positions of each sequence
        K.kv_append(c, kx.to(DEV), vx.to(DEV), torch.zeros(B, dtype=torch.int32, device=DEV), block_table=tdev,
                    n_valid=torch.from_numpy(lens - n_q).to(DEV))
        return c

    idx = torch.from_numpy((lens - n_q).astype(np.int64)).view(B, 1, 1, 1) + torch.arange(n_q).view(1, 1, n_q, 1)
    idx = idx.expand(B, Hkv, n_q, d)
    k1 = torch.gather(kx, 2, idx).contiguous().to(DEV)
    v1 = torch.gather(vx, 2, idx).contiguous().to(DEV)
    seq = torch.from_numpy(lens).to(DEV)
    a = make()
    got = K.attn_decode_multi(a, q, seq, total, k_new=k1, v_new=v1, block_table=tdev, part_tokens=64).cpu()
    b = make()
    K.kv_append(b, k1, v1, torch.from_numpy(lens - n_q).to(DEV), block_table=tdev)
    ref = K.attn_decode_multi(b, q, seq, total, block_table=tdev, part_tokens=64).cpu()
    assert torch.equal(got, ref)
    np.testing.assert_array_equal(storage(a.k), storage(b.k))
    np.testing.assert_array_equal(storage(a.v), storage(b.v))
