"""Prefill attention on the GPU (through the C ABI) vs the fp64 oracle."""
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


def _inputs(B, Hq, Hkv, N, d, dtype, seed, std=1.0):
    q = synth.normal((B, Hq, N, d), (seed, synth.T_Q), dtype, std=std)
    k = synth.normal((B, Hkv, N, d), (seed, synth.T_KNEW), dtype, std=std)
    v = synth.normal((B, Hkv, N, d), (seed, synth.T_VNEW), dtype, std=std)
    return q, k, v


def _oracle(q, k, v, positions, q_lens, causal=True, key_mask=None, prefix=None):
    d = q.shape[-1]
    kw = {}
    if prefix is not None:
        kw = dict(prefix_k=prefix[0], prefix_v=prefix[1], attend_prefix=True)
    return OA.prefill(f64(q), f64(k), f64(v), positions, q_lens, 1.0 / math.sqrt(d), causal=causal,
                      key_mask=key_mask, **kw)


def test_tiny_config_prefill_fp32():
    """1 layer, batch 1, 4/4 heads, d 64, fp32: causal prefill of 16 tokens."""
    q, k, v = _inputs(1, 4, 4, 16, 64, torch.float32, 20)
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV)).cpu().numpy()
    assert max_abs(got, _oracle(q, k, v, [0], [16])) <= TOL


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("G,d", [(1, 64), (4, 128), (2, 64), (8, 128)])
def test_causal_prefill_groups(dtype, G, d):
    B, Hkv, N = 2, 2, 77
    std = 1.0 if dtype == torch.float32 else 1.0 / math.sqrt(d)
    q, k, v = _inputs(B, G * Hkv, Hkv, N, d, dtype, 21 + G, std=std)
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV)).cpu().numpy()
    assert np.isfinite(got).all()
    assert max_abs(got, _oracle(q, k, v, [0, 0], [N, N])) <= TOL


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_q_lens_and_padding_mask(causal):
    """Two real length-3 sequences padded to 5 ("Transformer Attention Masks
    and KV-Cache Inference", "Implementation and verification procedure"),
    then a ragged batch with a random key mask and NaN in the padding."""
    B, Hq, Hkv, N, d = 2, 4, 2, 5, 64
    q, k, v = _inputs(B, Hq, Hkv, N, d, torch.float32, 30)
    q_lens = np.array([3, 3], np.int32)
    mask = synth.padding_mask(q_lens, N)
    k[:, :, 3:] = float("nan")
    v[:, :, 3:] = float("nan")
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), q_lens=torch.from_numpy(q_lens).to(DEV),
                         key_mask=torch.from_numpy(mask).to(DEV), causal=causal).cpu().numpy()
    assert np.isfinite(got).all()
    assert np.all(got[:, :, 3:] == 0.0)
    # real rows equal an unpadded run
    ref = K.attn_prefill(q[:, :, :3].contiguous().to(DEV), k[:, :, :3].contiguous().to(DEV),
                         v[:, :, :3].contiguous().to(DEV), causal=causal).cpu().numpy()
    assert max_abs(got[:, :, :3], ref) <= 1e-6
    assert max_abs(got, _oracle(q, k, v, [0, 0], q_lens, causal, mask)) <= TOL

    B, N = 3, 150
    q, k, v = _inputs(B, Hq, Hkv, N, d, torch.bfloat16, 31, std=1 / 8)
    q_lens = np.array([150, 1, 97], np.int32)
    mask = synth.random_mask((B, N), 0.7, (31, synth.T_MASK))
    mask[:, 0] = 1
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), q_lens=torch.from_numpy(q_lens).to(DEV),
                         key_mask=torch.from_numpy(mask).to(DEV), causal=causal).cpu().numpy()
    assert max_abs(got, _oracle(q, k, v, [0, 0, 0], q_lens, causal, mask)) <= TOL


def test_causal_matrix_through_one_hot_values():
    """V rows one-hot: output row t is the attention weight row t, so the
    printed 4x4 causal pattern shows up as exact zeros above the diagonal."""
    d, N = 64, 4
    q, k, _ = _inputs(1, 1, 1, N, d, torch.float32, 32)
    v = torch.zeros((1, 1, N, d), dtype=torch.float32)
    for s in range(N):
        v[0, 0, s, s] = 1.0
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV)).cpu().numpy()[0, 0, :, :N]
    assert np.all(got[np.triu_indices(N, 1)] == 0.0)
    assert np.all(got[np.tril_indices(N)] > 0.0)
    assert np.abs(got.sum(axis=1) - 1.0).max() <= 1e-6
    want = OA.attention_weights(f64(q)[0, 0], f64(k)[0, 0], OA.causal_allow(N), 1 / math.sqrt(d))
    assert max_abs(got, want) <= 1e-6


@pytest.mark.parametrize("layout,G,d,N,pos,cache_dtype", [
    (K.PAGED, 4, 128, 40, (0, 0), K.BF16),
    (K.CONTIGUOUS, 4, 128, 40, (0, 0), K.BF16),
    (K.PAGED, 1, 64, 300, (5, 37), K.BF16),        # two query tiles per head, shifted positions
    (K.PAGED, 8, 128, 200, (16, 3), K.BF16),       # seven query tiles
    (K.CONTIGUOUS, 2, 128, 150, (7, 0), K.BF16),
    (K.PAGED, 4, 128, 100, (3, 0), K.FP8_E4M3),    # encoded by the separate append pass
])
def test_prefill_writes_cache_bit_exact(layout, G, d, N, pos, cache_dtype):
    """The cache bytes after attn_prefill equal the oracle's append of the
    new tokens (bf16: written by the MFMA kernel's own workgroups; fp8: by
    the append kernel), and the attention output matches."""
    B, Hkv = 2, 2
    Hq = G * Hkv
    q, k, v = _inputs(B, Hq, Hkv, N, d, torch.bfloat16, 33, std=1 / math.sqrt(d))
    q_lens = np.array([N, (2 * N) // 3 + 1], np.int32)
    positions = np.array(pos, np.int32)
    ks = vs = None
    if cache_dtype == K.FP8_E4M3:
        ks = torch.from_numpy(synth.fp8_scales(Hkv, (33, synth.T_SCALE))).to(DEV)
        vs = torch.from_numpy(synth.fp8_scales(Hkv, (34, synth.T_SCALE))).to(DEV)
    if layout == K.PAGED:
        nb = [synth.blocks_for(p + N) for p in positions]
        table, nblk = synth.block_table(nb, max(nb), (33, synth.T_PERM), num_blocks=sum(nb) + 3)
        cache = K.KVCache.paged(nblk, Hkv, d, cache_dtype, DEV, ks, vs, fill=0.5 if ks is None else 7)
        tdev = torch.from_numpy(table).to(DEV)
    else:
        table, tdev = None, None
        cap = 16 * synth.blocks_for(int(positions.max()) + N)
        cache = K.KVCache.contiguous(B, Hkv, cap, d, cache_dtype, DEV, ks, vs, fill=0.5)
    before_k, before_v = storage(cache.k), storage(cache.v)
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), cache=cache, q_lens=torch.from_numpy(q_lens).to(DEV),
                         positions=torch.from_numpy(positions).to(DEV), block_table=tdev).cpu().numpy()
    want_k, want_v = OC.predict_append(before_k, before_v, storage(k), storage(v), positions, N, layout == K.PAGED,
                                       table, in_dtype=K.BF16, cache_dtype=cache_dtype,
                                       k_scale=None if ks is None else ks.cpu().numpy(),
                                       v_scale=None if vs is None else vs.cpu().numpy(), n_valid=q_lens)
    np.testing.assert_array_equal(storage(cache.k), want_k)
    np.testing.assert_array_equal(storage(cache.v), want_v)
    assert max_abs(got, _oracle(q, k, v, positions, q_lens)) <= TOL


@pytest.mark.parametrize("cache_dtype", [K.BF16, K.FP8_E4M3])
def test_chunked_prefill_attends_cached_prefix(cache_dtype):
    """A second chunk at positions P.. attends the cached prefix plus itself,
    equal to the matching rows of a one-shot prefill."""
    B, Hq, Hkv, d, N = 2, 8, 2, 128, 96
    P = np.array([40, 17], np.int32)
    n2 = N - P
    q, k, v = _inputs(B, Hq, Hkv, N, d, torch.bfloat16, 34, std=1 / math.sqrt(d))
    table, nblk = synth.block_table([6, 6], 6, (34, synth.T_PERM))
    ks = vs = None
    if cache_dtype == K.FP8_E4M3:
        ks = torch.full((Hkv,), 0.02, dtype=torch.float32, device=DEV)
        vs = torch.full((Hkv,), 0.03, dtype=torch.float32, device=DEV)
    cache = K.KVCache.paged(nblk, Hkv, d, cache_dtype, DEV, ks, vs)
    cache.k.zero_()
    cache.v.zero_()
    tdev = torch.from_numpy(table).to(DEV)
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    K.kv_append(cache, k.to(DEV), v.to(DEV), zeros, block_table=tdev, n_valid=torch.from_numpy(P).to(DEV))
    # second chunk: new tokens P .. N-1 (ragged), padded to the longest
    n_max = int(n2.max())
    q2 = torch.zeros((B, Hq, n_max, d), dtype=torch.bfloat16)
    k2 = torch.zeros((B, Hkv, n_max, d), dtype=torch.bfloat16)
    v2 = torch.zeros((B, Hkv, n_max, d), dtype=torch.bfloat16)
    for b in range(B):
        q2[b, :, :n2[b]] = q[b, :, P[b]:]
        k2[b, :, :n2[b]] = k[b, :, P[b]:]
        v2[b, :, :n2[b]] = v[b, :, P[b]:]
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=torch.from_numpy(P).to(DEV),
                         q_lens=torch.from_numpy(n2).to(DEV), block_table=tdev, attend_prefix=True).cpu().numpy()
    if cache_dtype == K.BF16:
        full = _oracle(q, k, v, [0, 0], [N, N])
        for b in range(B):
            assert max_abs(got[b, :, :n2[b]], full[b, :, P[b]:]) <= TOL
            assert np.all(got[b, :, n2[b]:] == 0.0)
    else:
        # prefix read back from the fp8 cache: the oracle dequantises its own codes
        pk = [np.stack([OC.to_f64(OC.encode_rows(storage(k)[b, g, :P[b]], OC.BF16, OC.FP8_E4M3, np.float32(0.02)),
                                  OC.FP8_E4M3, np.float32(0.02)) for g in range(Hkv)]) for b in range(B)]
        pv = [np.stack([OC.to_f64(OC.encode_rows(storage(v)[b, g, :P[b]], OC.BF16, OC.FP8_E4M3, np.float32(0.03)),
                                  OC.FP8_E4M3, np.float32(0.03)) for g in range(Hkv)]) for b in range(B)]
        want = _oracle(q2, k2, v2, P, n2, prefix=(pk, pv))
        assert max_abs(got, want) <= TOL


def test_decode_equals_last_row_of_prefill():
    """Cached decode == the last row of a full recompute ("Transformer
    Attention Masks and KV-Cache Inference", "Implementation and verification
    procedure"), both on the GPU."""
    Hq, Hkv, d, N = 8, 2, 128, 200
    q, k, v = _inputs(1, Hq, Hkv, N, d, torch.bfloat16, 35, std=1 / math.sqrt(d))
    full = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV)).cpu().numpy()
    table, nblk = synth.block_table([13], 13, (35, synth.T_PERM))
    cache = K.KVCache.paged(nblk, Hkv, d, K.BF16, DEV, fill=0.0)
    tdev = torch.from_numpy(table).to(DEV)
    K.kv_append(cache, k.to(DEV), v.to(DEV), torch.zeros(1, dtype=torch.int32, device=DEV), block_table=tdev)
    dec = K.attn_decode(cache, q[:, :, -1].contiguous().to(DEV), torch.tensor([N], dtype=torch.int32, device=DEV), N,
                        block_table=tdev, part_tokens=64).cpu().numpy()
    assert max_abs(dec, full[:, :, -1]) <= TOL


@pytest.mark.parametrize("G,d,causal", [(4, 128, True), (1, 128, True), (8, 64, True), (2, 128, False)])
def test_mfma_prefill_many_tiles_ragged(G, d, causal):
    """bf16 MFMA path over several 32-key tiles and query tiles with a
    ragged tail (N not a multiple of any tile) and ragged q_lens."""
    B, Hkv, N = 2, 2, 333
    q, k, v = _inputs(B, G * Hkv, Hkv, N, d, torch.bfloat16, 40 + G, std=1 / math.sqrt(d))
    q_lens = np.array([333, 190], np.int32)
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), q_lens=torch.from_numpy(q_lens).to(DEV),
                         causal=causal).cpu().numpy()
    assert np.isfinite(got).all()
    assert np.all(got[1, :, 190:] == 0.0)
    assert max_abs(got, _oracle(q, k, v, [0, 0], q_lens, causal)) <= TOL


def test_mfma_prefill_unit_scale_inputs_and_key_mask():
    """N(0,1) inputs (larger scores) with a random key mask and NaN in the
    masked K/V rows."""
    B, Hq, Hkv, N, d = 1, 8, 2, 200, 128
    q, k, v = _inputs(B, Hq, Hkv, N, d, torch.bfloat16, 46, std=0.5)
    mask = synth.random_mask((B, N), 0.5, (46, synth.T_MASK))
    mask[:, 0] = 1
    m = torch.from_numpy(mask == 0)
    k[m[:, None, :, None].expand_as(k)] = float("nan")
    v[m[:, None, :, None].expand_as(v)] = float("nan")
    for causal in (True, False):
        got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), key_mask=torch.from_numpy(mask).to(DEV),
                             causal=causal).cpu().numpy()
        assert np.isfinite(got).all()
        assert max_abs(got, _oracle(q, k, v, [0], [N], causal, mask)) <= TOL


def test_mfma_prefill_constant_values_give_ones():
    """Row sums are taken over the same rounded weights as the output, so
    V == 1 gives exactly-normalised rows."""
    B, Hq, Hkv, N, d = 1, 4, 1, 257, 128
    q, k, _ = _inputs(B, Hq, Hkv, N, d, torch.bfloat16, 47)
    v = torch.ones((B, Hkv, N, d), dtype=torch.bfloat16)
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV)).cpu().numpy()
    assert np.abs(got - 1.0).max() <= 1e-6


@pytest.mark.parametrize("causal", [False, True])
def test_mfma_prefill_each_masked_key_gets_zero_weight(causal):
    """V rows one-hot, so output row t is query t's weight vector.  Masking
    single keys at every accumulator position of the two 32-key tiles must
    give those keys weight exactly 0 and leave every row summing to 1."""
    N, d = 64, 128
    q = synth.normal((1, 1, N, d), (48, synth.T_Q), std=0.1)
    k = synth.normal((1, 1, N, d), (48, synth.T_KNEW), std=0.1)
    v = torch.zeros((1, 1, N, d), dtype=torch.bfloat16)
    for s in range(N):
        v[0, 0, s, s] = 1.0
    for masked in ([0], [1], [3], [4], [8], [12], [16], [27], [31], [32], [33], [63], [0, 5, 40, 41]):
        mask = np.ones((1, N), np.uint8)
        mask[0, masked] = 0
        got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), key_mask=torch.from_numpy(mask).to(DEV),
                             causal=causal).cpu().numpy()[0, 0, :, :N]
        for c in masked:
            assert np.all(got[:, c] == 0.0), masked
        rows = [t for t in range(N) if mask[0, :t + 1 if causal else N].any()]
        assert np.abs(got[rows].sum(axis=1) - 1.0).max() <= 1e-6, masked


def _prefix_case(B, Hq, Hkv, d, P, n2, layout, seed, poison=None, cache_dtype=K.BF16, scales=None):
    """A cache holding positions 0 .. P[b]-1 of each sequence (appended from
    seeded bf16 rows; `poison` marks prefix positions whose K/V are set to NaN
    first), and a padded chunk of n2[b] new tokens.  An fp8 cache takes the
    per-head (k_scale, v_scale) of `scales`, and the oracle's prefix is then
    its own decoding of its own E4M3FN encoding of those rows."""
    P = np.asarray(P, np.int32)
    n2 = np.asarray(n2, np.int32)
    n_max = int(n2.max())
    total = int((P + n2).max())
    std = 1.0 if cache_dtype == K.FP8_E4M3 else 1 / math.sqrt(d)
    kp = synth.normal((B, Hkv, total, d), (seed, synth.T_K), torch.bfloat16, std=std)
    vp = synth.normal((B, Hkv, total, d), (seed, synth.T_V), torch.bfloat16, std=std)
    ks = vs = None
    if cache_dtype == K.FP8_E4M3:
        ks = torch.tensor(scales[0], dtype=torch.float32, device=DEV)
        vs = torch.tensor(scales[1], dtype=torch.float32, device=DEV)
    if poison is not None:
        for b, s in zip(*np.nonzero(poison[:, :total])):
            kp[b, :, s] = float("nan")
            vp[b, :, s] = float("nan")
    q2, k2, v2 = _inputs(B, Hq, Hkv, n_max, d, torch.bfloat16, seed + 1, std=1 / math.sqrt(d))
    for b in range(B):
        q2[b, :, n2[b]:] = 0
        k2[b, :, n2[b]:] = 0
        v2[b, :, n2[b]:] = 0
    table = tdev = None
    if layout == K.PAGED:
        nbs = [synth.blocks_for(int(P[b] + n2[b])) for b in range(B)]
        table, nblk = synth.block_table(nbs, max(nbs), (seed, synth.T_PERM))
        cache = K.KVCache.paged(nblk, Hkv, d, cache_dtype, DEV, ks, vs)
        tdev = torch.from_numpy(table).to(DEV)
    else:
        cap = -(-total // 16) * 16
        cache = K.KVCache.contiguous(B, Hkv, cap, d, cache_dtype, DEV, ks, vs)
    cache.k.zero_()
    cache.v.zero_()
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    K.kv_append(cache, kp.to(DEV), vp.to(DEV), zeros, block_table=tdev, n_valid=torch.from_numpy(P).to(DEV))
    if cache_dtype == K.FP8_E4M3:
        def deq(x, b, sc):
            with np.errstate(divide="ignore"):   # a zero scale encodes every value as +-448
                return np.stack([OC.to_f64(OC.encode_rows(storage(x)[b, g, :P[b]], OC.BF16, OC.FP8_E4M3,
                                                          np.float32(sc[g])), OC.FP8_E4M3, np.float32(sc[g]))
                                 for g in range(Hkv)])
        prefix = ([deq(kp, b, scales[0]) for b in range(B)], [deq(vp, b, scales[1]) for b in range(B)])
    else:
        prefix = ([f64(kp[b, :, :P[b]]) for b in range(B)], [f64(vp[b, :, :P[b]]) for b in range(B)])
    return cache, table, tdev, q2, k2, v2, P, n2, prefix


@pytest.mark.parametrize("G,d", [(4, 128), (8, 64), (1, 128), (2, 64)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("layout", [K.PAGED, K.CONTIGUOUS])
def test_mfma_chunked_prefill_attends_cached_prefix(G, d, causal, layout):
    """bf16 chunk against a bf16 cached prefix on the matrix-core kernel:
    prefixes that are not whole tiles (77 and 130 positions), ragged chunks,
    causal and not; the chunk's rows are also stored in the cache."""
    B, Hkv = 2, 2
    Hq = G * Hkv
    cache, table, tdev, q2, k2, v2, P, n2, prefix = _prefix_case(B, Hq, Hkv, d, [77, 130], [100, 37], layout,
                                                                   60 + G + d)
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=torch.from_numpy(P).to(DEV),
                         q_lens=torch.from_numpy(n2).to(DEV), block_table=tdev, causal=causal,
                         attend_prefix=True).cpu().numpy()
    want = _oracle(q2, k2, v2, P, n2, causal=causal, prefix=prefix)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL
    for b in range(B):
        assert np.all(got[b, :, n2[b]:] == 0.0)
    # the chunk's K rows were stored at positions P[b] + i
    kc = storage(cache.k)
    k2s = storage(k2)
    for b in range(B):
        for i in (0, int(n2[b]) - 1):
            p = int(P[b]) + i
            if layout == K.PAGED:
                row = kc[table[b][p // 16], :, p % 16]
            else:
                row = kc[b, :, p]
            np.testing.assert_array_equal(row, k2s[b, :, i])


def test_mfma_chunked_prefill_long_prefix_many_tiles():
    """A 1,000-position prefix and a 300-token chunk (GQA 4, d 128): most
    tiles take the unmasked step; equals the matching rows of a one-shot
    prefill of all 1,300 tokens."""
    B, Hq, Hkv, d = 1, 8, 2, 128
    N, P0 = 1300, 1000
    q, k, v = _inputs(B, Hq, Hkv, N, d, torch.bfloat16, 70, std=1 / math.sqrt(d))
    nb = synth.blocks_for(N)
    table, nblk = synth.block_table([nb], nb, (70, synth.T_PERM))
    tdev = torch.from_numpy(table).to(DEV)
    cache = K.KVCache.paged(nblk, Hkv, d, K.BF16, DEV)
    P = torch.tensor([P0], dtype=torch.int32, device=DEV)
    K.kv_append(cache, k.to(DEV), v.to(DEV), torch.zeros(1, dtype=torch.int32, device=DEV), block_table=tdev,
                n_valid=P)
    got = K.attn_prefill(q[:, :, P0:].contiguous().to(DEV), k[:, :, P0:].contiguous().to(DEV),
                         v[:, :, P0:].contiguous().to(DEV), cache=cache, positions=P, block_table=tdev,
                         attend_prefix=True).cpu().numpy()
    full = _oracle(q, k, v, [0], [N])
    assert max_abs(got[0], full[0, :, P0:]) <= TOL



@pytest.mark.parametrize("P0,d", [(131072, 64), (140007, 64), (140007, 128)])
def test_mfma_chunked_prefill_prefix_of_many_blocks(P0, d):
    """Paged prefixes of 8,192 blocks (131,072 positions) and of 8,751
    blocks: the kernel keeps up to 8,192 of a prefix's block ids in LDS and
    otherwise reads them from the table in global memory; both give the
    oracle's rows (GQA 2, a 40-token causal chunk).  Attention over
    the prefix does not depend on the order of its keys, and one row among
    10^5 barely moves an average, so 24 "needle" keys spread over the prefix
    (the last block included) are made to dominate every query's weights: a
    needle's block read from its neighbour changes the result by 5e-3 or
    more (the oracle with that mistake), while rounding the weights to bf16
    can move it by at most 2^-9 of the needles' largest V element (< 2e-3)."""
    Hq, Hkv, n = 2, 1, 40
    total = P0 + n
    kp = synth.normal((1, Hkv, total, d), (75, synth.T_K), torch.bfloat16, std=1 / math.sqrt(d))
    vp = synth.normal((1, Hkv, total, d), (75, synth.T_V), torch.bfloat16, std=1 / math.sqrt(d))
    u = synth.normal((d,), (76, synth.T_Q), torch.float32)
    u = u / u.norm()
    needles = np.linspace(5, P0 - 1, 24).astype(np.int64)
    for j, pos in enumerate(needles):
        kp[0, :, pos] = ((40.0 + 0.25 * j) * u).to(torch.bfloat16)   # scores ~20 against 4u
        vp[0, :, pos] = synth.normal((d,), (77 + j, synth.T_V), torch.bfloat16, std=0.25)
    q2 = (synth.normal((1, Hq, n, d), (78, synth.T_Q), torch.float32, std=0.1) + 4.0 * u).to(torch.bfloat16)
    k2 = kp[:, :, P0:].contiguous()
    v2 = vp[:, :, P0:].contiguous()
    nb = synth.blocks_for(total)
    table, nblk = synth.block_table([nb], nb, (75, synth.T_PERM))
    tdev = torch.from_numpy(table).to(DEV)
    cache = K.KVCache.paged(nblk, Hkv, d, K.BF16, DEV)
    P = torch.tensor([P0], dtype=torch.int32, device=DEV)
    K.kv_append(cache, kp.to(DEV), vp.to(DEV), torch.zeros(1, dtype=torch.int32, device=DEV), block_table=tdev,
                n_valid=P)
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=P, block_table=tdev,
                         attend_prefix=True).cpu().numpy()
    want = _oracle(q2, k2, v2, [P0], [n], prefix=([f64(kp[0, :, :P0])], [f64(vp[0, :, :P0])]))
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL


@pytest.mark.parametrize("P0", [65536, 70007])
def test_mfma_fp8_prefix_of_many_blocks(P0):
    """An fp8 paged prefix of 4,096 blocks (65,536 positions, as many block
    ids as the fp8-prefix kernel keeps in LDS) and of 4,376 blocks (ids read
    from the table in global memory), with 24 dominant needle keys as in the
    bf16 case above, against the oracle's decoding of its own E4M3FN encoding
    of the same rows (GQA 2, d 128, a 40-token causal chunk at bf16)."""
    Hq, Hkv, d, n = 2, 1, 128, 40
    ks, vs = 0.05, 0.005   # needle K codes up to ~300, needle V codes up to ~180
    total = P0 + n
    kp = synth.normal((1, Hkv, total, d), (85, synth.T_K), torch.bfloat16, std=1 / math.sqrt(d))
    vp = synth.normal((1, Hkv, total, d), (85, synth.T_V), torch.bfloat16, std=1 / math.sqrt(d))
    u = synth.normal((d,), (86, synth.T_Q), torch.float32)
    u = u / u.norm()
    needles = np.linspace(5, P0 - 1, 24).astype(np.int64)
    for j, pos in enumerate(needles):
        kp[0, :, pos] = ((40.0 + 0.25 * j) * u).to(torch.bfloat16)
        vp[0, :, pos] = synth.normal((d,), (87 + j, synth.T_V), torch.bfloat16, std=0.25)
    q2 = (synth.normal((1, Hq, n, d), (88, synth.T_Q), torch.float32, std=0.1) + 4.0 * u).to(torch.bfloat16)
    k2 = kp[:, :, P0:].contiguous()
    v2 = vp[:, :, P0:].contiguous()
    nb = synth.blocks_for(total)
    table, nblk = synth.block_table([nb], nb, (85, synth.T_PERM))
    tdev = torch.from_numpy(table).to(DEV)
    cache = K.KVCache.paged(nblk, Hkv, d, K.FP8_E4M3, DEV, torch.tensor([ks], device=DEV),
                            torch.tensor([vs], device=DEV))
    P = torch.tensor([P0], dtype=torch.int32, device=DEV)
    K.kv_append(cache, kp.to(DEV), vp.to(DEV), torch.zeros(1, dtype=torch.int32, device=DEV), block_table=tdev,
                n_valid=P)
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=P, block_table=tdev,
                         attend_prefix=True).cpu().numpy()

    def deq(x, sc):
        codes = OC.encode_rows(storage(x)[0, 0, :P0], OC.BF16, OC.FP8_E4M3, np.float32(sc))
        return OC.to_f64(codes, OC.FP8_E4M3, np.float32(sc))[None]
    want = _oracle(q2, k2, v2, [P0], [n], prefix=([deq(kp, ks)], [deq(vp, vs)]))
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL

def test_mfma_prefix_key_mask_nan_poisoned_and_verify_shape():
    """Key mask over absolute positions with NaN in the masked cached rows
    (weights exactly 0, outputs finite), and a 4-token chunk (the shape of
    checking drafted tokens) after 500 cached positions."""
    B, Hq, Hkv, d = 2, 16, 2, 128
    P, n2 = [200, 500], [64, 4]
    mask = synth.random_mask((B, 520), 0.7, (71, synth.T_MASK))
    mask[:, 0] = 1
    poison = (mask == 0)
    poison[:, 200:] = False   # only cached rows are poisoned
    cache, table, tdev, q2, k2, v2, P, n2, prefix = _prefix_case(B, Hq, Hkv, d, P, n2, K.PAGED, 72, poison=poison)
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=torch.from_numpy(P).to(DEV),
                         q_lens=torch.from_numpy(n2).to(DEV), block_table=tdev,
                         key_mask=torch.from_numpy(mask).to(DEV), attend_prefix=True).cpu().numpy()
    assert np.isfinite(got).all()
    # the oracle sees the masked positions as masked, whatever they hold
    clean = ([np.nan_to_num(x, nan=0.0) for x in prefix[0]], [np.nan_to_num(x, nan=0.0) for x in prefix[1]])
    want = _oracle(q2, k2, v2, P, n2, key_mask=mask, prefix=clean)
    assert max_abs(got, want) <= TOL


def test_mfma_prefix_invalid_block_ids_are_masked():
    """Prefix positions whose block id is out of range or negative are masked
    keys (as for decode); every tile then takes the masked step."""
    B, Hq, Hkv, d = 1, 8, 2, 64
    cache, table, tdev, q2, k2, v2, P, n2, prefix = _prefix_case(B, Hq, Hkv, d, [96], [70], K.PAGED, 73)
    bad = tdev.clone()
    bad[0, 1] = 10 ** 6   # positions 16..31
    bad[0, 4] = -1        # positions 64..79
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=torch.from_numpy(P).to(DEV),
                         block_table=bad, attend_prefix=True).cpu().numpy()
    mask = np.ones((1, 96 + 70), np.uint8)
    mask[0, 16:32] = 0
    mask[0, 64:80] = 0
    want = _oracle(q2, k2, v2, P, n2, key_mask=mask, prefix=prefix)
    assert max_abs(got, want) <= TOL


FP8_SCALES = ([0.011, 0.023], [0.017, 0.009])   # per KV head (k_scale, v_scale): codes up to ~400


@pytest.mark.parametrize("G,d", [(4, 128), (8, 64), (1, 128), (2, 64)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("layout", [K.PAGED, K.CONTIGUOUS])
@pytest.mark.parametrize("P,n2", [([77, 130], [100, 37]), ([64, 0], [70, 33])])
def test_mfma_fp8_prefix_chunk(G, d, causal, layout, P, n2):
    """bf16 chunk against an fp8 (E4M3FN) cached prefix on the matrix-core
    kernel: the cached rows are dequantised with per-head K and V scales
    ("KV Cache Fully Explained", section "(1) FP8 quantization"); prefixes
    that end inside a 32-key tile (77, 130), on a tile edge (64) and empty
    (0); ragged chunks, causal and not, paged and contiguous."""
    B, Hkv = 2, 2
    Hq = G * Hkv
    cache, table, tdev, q2, k2, v2, P, n2, prefix = _prefix_case(
        B, Hq, Hkv, d, P, n2, layout, 80 + G + d, cache_dtype=K.FP8_E4M3, scales=FP8_SCALES)
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=torch.from_numpy(P).to(DEV),
                         q_lens=torch.from_numpy(n2).to(DEV), block_table=tdev, causal=causal,
                         attend_prefix=True).cpu().numpy()
    want = _oracle(q2, k2, v2, P, n2, causal=causal, prefix=prefix)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL
    for b in range(B):
        assert np.all(got[b, :, n2[b]:] == 0.0)


@pytest.mark.parametrize("scales", [([-0.011, 0.023], [0.017, -0.009]), ([0.011, 0.023], [0.0, 0.009])])
def test_mfma_fp8_prefix_key_mask_and_scale_signs(scales):
    """fp8 prefix with a key mask over absolute positions, a negative K scale
    (not foldable into the score scale: every tile takes the masked step), a
    negative V scale and a zero V scale."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    P, n2 = [150, 45], [64, 90]
    mask = synth.random_mask((B, 240), 0.7, (82, synth.T_MASK))
    mask[:, 0] = 1
    cache, table, tdev, q2, k2, v2, P, n2, prefix = _prefix_case(
        B, Hq, Hkv, d, P, n2, K.PAGED, 83, cache_dtype=K.FP8_E4M3, scales=scales)
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=torch.from_numpy(P).to(DEV),
                         q_lens=torch.from_numpy(n2).to(DEV), block_table=tdev,
                         key_mask=torch.from_numpy(mask).to(DEV), attend_prefix=True).cpu().numpy()
    want = _oracle(q2, k2, v2, P, n2, key_mask=mask, prefix=prefix)
    assert np.isfinite(got).all()
    assert max_abs(got, want) <= TOL


def test_mfma_fp8_prefix_long_many_tiles():
    """A 1,000-position fp8 prefix (not a whole number of tiles) and a
    300-token chunk (GQA 4, d 128): most tiles take the unmasked step."""
    B, Hq, Hkv, d = 1, 8, 2, 128
    cache, table, tdev, q2, k2, v2, P, n2, prefix = _prefix_case(
        B, Hq, Hkv, d, [1000], [300], K.PAGED, 84, cache_dtype=K.FP8_E4M3, scales=FP8_SCALES)
    got = K.attn_prefill(q2.to(DEV), k2.to(DEV), v2.to(DEV), cache=cache, positions=torch.from_numpy(P).to(DEV),
                         block_table=tdev, attend_prefix=True).cpu().numpy()
    want = _oracle(q2, k2, v2, P, n2, prefix=prefix)
    assert max_abs(got, want) <= TOL


@pytest.mark.parametrize("cache_dtype", [K.BF16, K.FP8_E4M3])
def test_prefill_graph_replay_matches_eager(cache_dtype):
    """A chunked prefill against a cached prefix captured in a HIP graph (for
    fp8 the graph holds the append kernel and the attention kernel): every
    replay, with other eager prefills in between, equals the eager call bit
    for bit, and the cache holds the same bytes."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    scales = FP8_SCALES if cache_dtype == K.FP8_E4M3 else None
    case = _prefix_case(B, Hq, Hkv, d, [77, 130], [100, 37], K.PAGED, 90, cache_dtype=cache_dtype, scales=scales)
    cache, table, tdev, q2, k2, v2, P, n2, prefix = case
    q2, k2, v2 = q2.to(DEV), k2.to(DEV), v2.to(DEV)
    pos = torch.from_numpy(P).to(DEV)
    ql = torch.from_numpy(n2).to(DEV)
    want = K.attn_prefill(q2, k2, v2, cache=cache, positions=pos, q_lens=ql, block_table=tdev,
                          attend_prefix=True).clone()
    cache_bytes = (cache.k.clone(), cache.v.clone())
    out = torch.empty_like(want)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        K.attn_prefill(q2, k2, v2, cache=cache, positions=pos, q_lens=ql, block_table=tdev, attend_prefix=True,
                       out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.attn_prefill(q2, k2, v2, cache=cache, positions=pos, q_lens=ql, block_table=tdev, attend_prefix=True,
                       out=out)
    other = torch.randn_like(q2)
    for r in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), r
        K.attn_prefill(other, k2, v2, causal=False)   # eager work between replays
        torch.cuda.synchronize()
    assert torch.equal(cache.k, cache_bytes[0]) and torch.equal(cache.v, cache_bytes[1])


@pytest.mark.parametrize("Hq,d", [(8, 128), (4, 64), (1, 128)])
def test_prefill_mqa_single_kv_head(Hq, d):
    """MQA prefill: one KV head for every query head, causal, ragged q_lens."""
    B, N = 2, 150
    q, k, v = _inputs(B, Hq, 1, N, d, torch.bfloat16, 95 + Hq, std=1 / math.sqrt(d))
    q_lens = np.array([150, 61], np.int32)
    got = K.attn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), q_lens=torch.from_numpy(q_lens).to(DEV)).cpu().numpy()
    assert max_abs(got, _oracle(q, k, v, [0, 0], q_lens)) <= TOL
