"""kv_append on the GPU vs the oracle's predicted cache bytes: bit-exact."""
import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K
from kv_cache_decode_attn_amd import synth
from oracle import cache as OC
from tests.helpers import storage

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _canary_pool(shape, torch_dtype, seed):
    """A pool pre-filled with random bytes so untouched slots are recognisable."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=torch_dtype).element_size()
    b = synth.rng(*seed).integers(0, 256, size=n, dtype=np.uint8)
    t = torch.from_numpy(b).view(torch_dtype).reshape(shape)
    if torch_dtype != torch.uint8:  # keep canaries finite so comparisons stay bitwise
        t = torch.nan_to_num(t.float(), nan=1.0, posinf=2.0, neginf=-2.0).to(torch_dtype)
    return t


@pytest.mark.parametrize("dtype", [K.BF16, K.F32])
@pytest.mark.parametrize("d", [64, 128])
def test_append_paged_bit_exact(dtype, d):
    tdt = torch.bfloat16 if dtype == K.BF16 else torch.float32
    B, Hkv, n, nblk, mb = 3, 2, 9, 20, 5
    positions = np.array([0, 15, 40], np.int32)
    table, _ = synth.block_table([4, 4, 4], mb, (1, synth.T_PERM), num_blocks=nblk)
    pool_k = _canary_pool((nblk, Hkv, 16, d), tdt, (1, 20))
    pool_v = _canary_pool((nblk, Hkv, 16, d), tdt, (1, 21))
    kn = synth.normal((B, Hkv, n, d), (1, synth.T_KNEW), tdt)
    vn = synth.normal((B, Hkv, n, d), (1, synth.T_VNEW), tdt)
    want_k, want_v = OC.predict_append(storage(pool_k), storage(pool_v), storage(kn), storage(vn), positions, n, True,
                                       table, in_dtype=dtype, cache_dtype=dtype)
    cache = K.KVCache(pool_k.to(DEV), pool_v.to(DEV), K.PAGED, dtype)
    K.kv_append(cache, kn.to(DEV), vn.to(DEV), torch.from_numpy(positions).to(DEV),
                block_table=torch.from_numpy(table).to(DEV))
    np.testing.assert_array_equal(storage(cache.k), want_k)
    np.testing.assert_array_equal(storage(cache.v), want_v)


def test_append_contiguous_n_valid_and_capacity_edge():
    B, Hkv, d, cap, n = 2, 4, 128, 32, 6
    positions = np.array([3, 28], np.int32)     # sequence 1 runs past capacity 32
    n_valid = np.array([4, 6], np.int32)
    ck = _canary_pool((B, Hkv, cap, d), torch.bfloat16, (2, 20))
    cv = _canary_pool((B, Hkv, cap, d), torch.bfloat16, (2, 21))
    kn = synth.normal((B, Hkv, n, d), (2, synth.T_KNEW))
    vn = synth.normal((B, Hkv, n, d), (2, synth.T_VNEW))
    # positions >= capacity are skipped: only 4 tokens of sequence 1 fit
    want_k, want_v = OC.predict_append(storage(ck), storage(cv), storage(kn), storage(vn), positions, n, False,
                                       n_valid=np.array([4, 4]))
    cache = K.KVCache(ck.to(DEV), cv.to(DEV), K.CONTIGUOUS, K.BF16)
    K.kv_append(cache, kn.to(DEV), vn.to(DEV), torch.from_numpy(positions).to(DEV),
                n_valid=torch.from_numpy(n_valid).to(DEV))
    np.testing.assert_array_equal(storage(cache.k), want_k)
    np.testing.assert_array_equal(storage(cache.v), want_v)


def test_append_skips_out_of_range_blocks():
    B, Hkv, d, nblk = 2, 1, 64, 4
    table = np.array([[0, 99], [1, -5]], np.int32)  # second block of each sequence is invalid
    pk = _canary_pool((nblk, Hkv, 16, d), torch.bfloat16, (3, 20))
    pv = _canary_pool((nblk, Hkv, 16, d), torch.bfloat16, (3, 21))
    kn = synth.normal((B, Hkv, 4, d), (3, synth.T_KNEW))
    vn = synth.normal((B, Hkv, 4, d), (3, synth.T_VNEW))
    positions = np.array([14, 13], np.int32)  # tokens at 16.. fall in the invalid blocks
    want_k, want_v = OC.predict_append(storage(pk), storage(pv), storage(kn), storage(vn), positions, 4, True, table,
                                       n_valid=np.array([2, 3]))
    cache = K.KVCache(pk.to(DEV), pv.to(DEV), K.PAGED, K.BF16)
    K.kv_append(cache, kn.to(DEV), vn.to(DEV), torch.from_numpy(positions).to(DEV),
                block_table=torch.from_numpy(table).to(DEV))
    np.testing.assert_array_equal(storage(cache.k), want_k)
    np.testing.assert_array_equal(storage(cache.v), want_v)


@pytest.mark.parametrize("in_dtype", [K.BF16, K.F32])
def test_append_fp8_encode_bit_exact(in_dtype):
    tdt = torch.bfloat16 if in_dtype == K.BF16 else torch.float32
    B, Hkv, d, n, nblk = 2, 8, 128, 20, 8
    table, _ = synth.block_table([3, 3], 4, (4, synth.T_PERM), num_blocks=nblk)
    positions = np.array([5, 16], np.int32)
    scales_k = synth.fp8_scales(Hkv, (4, synth.T_SCALE, 0))
    scales_v = synth.fp8_scales(Hkv, (4, synth.T_SCALE, 1))
    kn = synth.normal((B, Hkv, n, d), (4, synth.T_KNEW), tdt, std=3.0)
    vn = synth.normal((B, Hkv, n, d), (4, synth.T_VNEW), tdt, std=3.0)
    # special values: saturation, subnormal range, ties, signed zero, NaN, inf
    special = torch.tensor([1e4, -1e4, 447.0, 449.0, 470.0, 2.0 ** -10, 3 * 2.0 ** -10, -0.0, 0.0, 1.0625,
                            float("nan"), float("inf"), -float("inf"), 2.0 ** -7, -2.0 ** -8, 5e-4], dtype=torch.float32)
    kn[0, 0, 0, :special.numel()] = special.to(tdt) * float(scales_k[0])
    pk = torch.zeros((nblk, Hkv, 16, d), dtype=torch.uint8)
    pv = torch.zeros((nblk, Hkv, 16, d), dtype=torch.uint8)
    want_k, want_v = OC.predict_append(storage(pk), storage(pv), storage(kn), storage(vn), positions, n, True, table,
                                       in_dtype=in_dtype, cache_dtype=OC.FP8_E4M3, k_scale=scales_k,
                                       v_scale=scales_v)
    cache = K.KVCache(pk.to(DEV), pv.to(DEV), K.PAGED, K.FP8_E4M3, torch.from_numpy(scales_k).to(DEV),
                      torch.from_numpy(scales_v).to(DEV))
    K.kv_append(cache, kn.to(DEV), vn.to(DEV), torch.from_numpy(positions).to(DEV),
                block_table=torch.from_numpy(table).to(DEV))
    np.testing.assert_array_equal(storage(cache.k), want_k)
    np.testing.assert_array_equal(storage(cache.v), want_v)


def test_validate_reports_contract_violations():
    B, Hkv, d = 3, 1, 64
    cache = K.KVCache.paged(6, Hkv, d, K.BF16, device=DEV, fill=0.0)
    table = torch.tensor([[0, 1], [2, 77], [3, 4]], dtype=torch.int32, device=DEV)
    lens = torch.tensor([20, 20, 40], dtype=torch.int32, device=DEV)
    err = K.validate(cache, lens, 64, block_table=table)
    assert err & K.VALIDATE_BLOCK_RANGE          # block 77 is outside the pool
    assert err & K.VALIDATE_LEN_RANGE            # 40 > 2 blocks * 16
    ok_lens = torch.tensor([20, 10, 30], dtype=torch.int32, device=DEV)
    assert K.validate(cache, ok_lens, 64, block_table=table) == 0
    pos = torch.tensor([20, 10, 29], dtype=torch.int32, device=DEV)
    assert K.validate(cache, ok_lens, 64, positions=pos, block_table=table) == K.VALIDATE_POSITION
