"""The fused decode step (kvattn_attn_decode_append) on the GPU.

It must equal kv_append(positions = seq_lens - 1) followed by attn_decode bit
for bit - output and cache bytes - and the oracle's append prediction and
attention on the same inputs."""
import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K
from oracle import cache as OC
from tests.helpers import max_abs, storage
from tests.test_gpu_decode import DEV, TOL, Case

pytestmark = pytest.mark.gpu


class StepCase(Case):
    """A Case whose cache holds every token but the last; the last token's
    K/V rows are the step's k_new / v_new."""

    def _build_cache(self, seed):
        super()._build_cache(seed)
        # undo the last token's append: restore the stale bytes there
        B, Hkv, d = self.B, self.Hkv, self.d
        stale = 0x7F if self.dtype == K.FP8_E4M3 else float("nan")
        for b in range(B):
            if self.lens[b] <= 0:
                continue
            p = int(self.lens[b]) - 1
            if self.layout == K.PAGED:
                blk = int(self.table[b, p // 16])
                self.cache.k[blk, :, p % 16] = stale
                self.cache.v[blk, :, p % 16] = stale
            else:
                self.cache.k[b, :, p] = stale
                self.cache.v[b, :, p] = stale
        last = torch.from_numpy(np.maximum(self.lens - 1, 0)).to(torch.int64)
        idx = last.view(B, 1, 1, 1).expand(B, Hkv, 1, d)
        self.k1 = torch.gather(self.k, 2, idx)[:, :, 0].contiguous()
        self.v1 = torch.gather(self.v, 2, idx)[:, :, 0].contiguous()

    def clone_cache(self):
        c = self.cache
        return K.KVCache(c.k.clone(), c.v.clone(), c.layout, c.dtype, c.k_scale, c.v_scale)

    def step_fused(self, cache, part, in_dtype=None):
        maskd = torch.from_numpy(self.mask).to(DEV) if self.mask is not None else None
        k1, v1 = self.k1, self.v1
        if in_dtype is not None:
            k1, v1 = k1.to(in_dtype), v1.to(in_dtype)
        return K.attn_decode_append(cache, self.q.to(DEV), k1.to(DEV), v1.to(DEV), torch.from_numpy(self.lens).to(DEV),
                                    self.maxlen, block_table=self.table, key_mask=maskd, part_tokens=part)

    def step_unfused(self, cache, part, in_dtype=None):
        maskd = torch.from_numpy(self.mask).to(DEV) if self.mask is not None else None
        k1, v1 = self.k1, self.v1
        if in_dtype is not None:
            k1, v1 = k1.to(in_dtype), v1.to(in_dtype)
        pos = torch.from_numpy(np.maximum(self.lens - 1, 0)).to(DEV)
        one = torch.from_numpy((self.lens > 0).astype(np.int32)).to(DEV)
        K.kv_append(cache, k1[:, :, None].contiguous().to(DEV), v1[:, :, None].contiguous().to(DEV), pos,
                    block_table=self.table, n_valid=one)
        return K.attn_decode(cache, self.q.to(DEV), torch.from_numpy(self.lens).to(DEV), self.maxlen,
                             block_table=self.table, key_mask=maskd, part_tokens=part)

    def predicted_cache(self, before_k, before_v, in_dtype=None):
        """The oracle's append prediction applied to the cache storage before
        the step (before_k / before_v: raw storage arrays)."""
        k1, v1 = self.k1, self.v1
        if in_dtype is not None:
            k1, v1 = k1.to(in_dtype), v1.to(in_dtype)
        icode = OC.F32 if k1.dtype == torch.float32 else OC.BF16
        ks = vs = None
        if self.scales is not None:
            ks, vs = self.scales
        table = self.table.cpu().numpy() if self.table is not None else None
        return OC.predict_append(before_k, before_v, storage(k1)[:, :, None], storage(v1)[:, :, None],
                                 np.maximum(self.lens - 1, 0), 1, self.layout == K.PAGED, block_table=table,
                                 in_dtype=icode, cache_dtype=self.dtype, k_scale=ks, v_scale=vs,
                                 n_valid=(self.lens > 0).astype(np.int32))


CASES = [
    # dtype, layout, Hq, Hkv, d, lens, mask, input dtype
    ("bf16-paged-g4", K.BF16, K.PAGED, 16, 4, 128, [1, 15, 16, 17, 300, 513, 64], False, None),
    ("bf16-contig-g1-mask", K.BF16, K.CONTIGUOUS, 4, 4, 64, [5, 129, 260], True, None),
    ("f32-contig-g2", K.F32, K.CONTIGUOUS, 8, 4, 128, [40, 1, 200], False, None),
    ("fp8-paged-g8-mfma", K.FP8_E4M3, K.PAGED, 16, 2, 128, [1, 16, 17, 513, 1000], False, None),
    ("fp8-paged-g2-f32in", K.FP8_E4M3, K.PAGED, 4, 2, 64, [33, 64, 65], False, torch.float32),
    ("fp8-contig-g4-mask", K.FP8_E4M3, K.CONTIGUOUS, 8, 2, 64, [31, 129, 300], True, None),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("part", [64, 0])
def test_fused_step_equals_append_then_decode_and_oracle(case, part):
    name, dtype, layout, Hq, Hkv, d, lens, use_mask, in_dtype = case
    mask = None
    if use_mask:
        from kv_cache_decode_attn_amd import synth
        mask = synth.random_mask((len(lens), max(lens) + 16), 0.7, (31, synth.T_MASK))
        mask[:, 0] = 1
    c = StepCase(len(lens), Hq, Hkv, d, lens, dtype=dtype, layout=layout, seed=30 + len(name), mask=mask,
                 poison_masked=False)
    a = c.clone_cache()
    b = c.clone_cache()
    before_k, before_v = storage(c.cache.k), storage(c.cache.v)
    got = c.step_fused(a, part, in_dtype).cpu()
    ref = c.step_unfused(b, part, in_dtype).cpu()
    # bit for bit the two-call step
    assert torch.equal(got, ref)
    np.testing.assert_array_equal(storage(a.k), storage(b.k))
    np.testing.assert_array_equal(storage(a.v), storage(b.v))
    # the cache bytes are the oracle's append prediction, bit for bit
    pk, pv = c.predicted_cache(before_k, before_v, in_dtype)
    np.testing.assert_array_equal(storage(a.k), pk)
    np.testing.assert_array_equal(storage(a.v), pv)
    # the output is the oracle's attention over the appended cache
    want = c.oracle(quantised=(dtype == K.FP8_E4M3))
    assert np.isfinite(got.numpy()).all()
    assert max_abs(got.numpy(), want) <= TOL


def test_fused_step_empty_sequence_writes_nothing():
    """seq_lens[b] = 0: no key, no append; the output row is 0."""
    c = StepCase(3, 8, 2, 128, [70, 0, 20], seed=41)
    a = c.clone_cache()
    before_k = storage(c.cache.k)
    got = c.step_fused(a, 64).cpu().numpy()
    assert np.all(got[1] == 0.0)
    after_k = storage(a.k)
    # only the blocks of the two appended slots changed
    changed = np.nonzero((after_k != before_k).reshape(after_k.shape[0], -1).any(axis=1))[0].tolist()
    tab = c.table.cpu().numpy()
    assert sorted(changed) == sorted({int(tab[0, 69 // 16]), int(tab[2, 19 // 16])})


def test_fused_step_repeated_decode_loop():
    """Several steps in a row, each appending its token and attending it, equal
    the two-call loop bit for bit."""
    c = StepCase(4, 32, 8, 128, [100, 300, 17, 60], seed=42)
    a, b = c.clone_cache(), c.clone_cache()
    lens0 = c.lens.copy()
    for step in range(4):
        c.lens = lens0 + step
        c.maxlen = int(c.lens.max())
        src = torch.randn((c.B, c.Hkv, 1, c.d), generator=torch.Generator().manual_seed(100 + step)).to(torch.bfloat16)
        c.k1 = src[:, :, 0].contiguous()
        c.v1 = (-src[:, :, 0]).contiguous()
        x = c.step_fused(a, 64).cpu()
        y = c.step_unfused(b, 64).cpu()
        assert torch.equal(x, y), step
    np.testing.assert_array_equal(storage(a.k), storage(b.k))
    np.testing.assert_array_equal(storage(a.v), storage(b.v))
