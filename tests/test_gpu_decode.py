"""Decode attention on the GPU (through the C ABI) vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K
from kv_cache_decode_attn_amd import synth
from oracle import attention as OA
from oracle import cache as OC
from oracle import codec
from tests.helpers import f64, max_abs, storage

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = 2e-3       # bf16 / fp32 cache, fp32 accumulate
TOL_FP8 = 3e-2   # fp8 cache vs the unquantised values


class Case:
    """A decode problem: logical K/V per sequence, a cache filled through
    kv_append (the last token appended on its own, as in a decode step), and
    the query.  Stale cache slots hold NaN so that reading one would show."""

    def __init__(self, B, Hq, Hkv, d, lens, dtype=K.BF16, layout=K.PAGED, seed=0, mask=None, std=1.0,
                 poison_masked=True):
        self.B, self.Hq, self.Hkv, self.d = B, Hq, Hkv, d
        self.lens = np.asarray(lens, np.int32)
        self.maxlen = int(self.lens.max()) if len(lens) else 0
        self.dtype, self.layout = dtype, layout
        width = max(self.maxlen, 1)
        src_dt = torch.float32 if dtype == K.F32 else torch.bfloat16
        self.k = synth.normal((B, Hkv, width, d), (seed, synth.T_K), src_dt, std=std)
        self.v = synth.normal((B, Hkv, width, d), (seed, synth.T_V), src_dt, std=std)
        self.q = synth.normal((B, Hq, d), (seed, synth.T_Q), src_dt)
        self.mask = mask
        if mask is not None and poison_masked:
            m = torch.from_numpy(mask[:, :width] == 0)
            self.k[m[:, None, :, None].expand_as(self.k)] = float("nan")
            self.v[m[:, None, :, None].expand_as(self.v)] = float("nan")
        self.scales = None
        if dtype == K.FP8_E4M3:
            self.scales = (synth.fp8_scales(Hkv, (seed, synth.T_SCALE, 0)), synth.fp8_scales(Hkv, (seed, synth.T_SCALE, 1)))
        self._build_cache(seed)

    def _build_cache(self, seed):
        B, Hkv, d = self.B, self.Hkv, self.d
        ks = vs = None
        if self.scales is not None:
            ks = torch.from_numpy(self.scales[0]).to(DEV)
            vs = torch.from_numpy(self.scales[1]).to(DEV)
        fill = float("nan") if self.dtype != K.FP8_E4M3 else None
        self.table = None
        if self.layout == K.PAGED:
            nbs = [synth.blocks_for(x) for x in self.lens]
            self.max_blocks = max(max(nbs), 1)
            spare = 3  # unused blocks in the pool
            table, nblk = synth.block_table(nbs, self.max_blocks, (seed, synth.T_PERM), num_blocks=sum(nbs) + spare)
            self.table = torch.from_numpy(table).to(DEV)
            self.cache = K.KVCache.paged(nblk, Hkv, d, self.dtype, DEV, ks, vs, fill=fill)
        else:
            cap = max(16, ((self.maxlen + 15) // 16) * 16 + 16)
            self.cache = K.KVCache.contiguous(B, Hkv, cap, d, self.dtype, DEV, ks, vs, fill=fill)
        if self.dtype == K.FP8_E4M3:
            self.cache.k.fill_(0x7F)  # NaN codes in stale slots
            self.cache.v.fill_(0x7F)
        # all but the last token of each sequence, then the last one alone
        kd, vd = self.k.to(DEV), self.v.to(DEV)
        zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
        before = torch.from_numpy(np.maximum(self.lens - 1, 0)).to(DEV)
        K.kv_append(self.cache, kd, vd, zeros, block_table=self.table, n_valid=before)
        last = torch.from_numpy(np.maximum(self.lens - 1, 0)).to(torch.int64)
        idx = last.view(B, 1, 1, 1).expand(B, Hkv, 1, d).to(DEV)
        k1 = torch.gather(kd, 2, idx).contiguous()
        v1 = torch.gather(vd, 2, idx).contiguous()
        one = torch.from_numpy((self.lens > 0).astype(np.int32)).to(DEV)
        K.kv_append(self.cache, k1, v1, before, block_table=self.table, n_valid=one)

    def run(self, part_tokens=0, q=None):
        maskd = torch.from_numpy(self.mask).to(DEV) if self.mask is not None else None
        return K.attn_decode(self.cache, (q if q is not None else self.q).to(DEV),
                             torch.from_numpy(self.lens).to(DEV), self.maxlen, block_table=self.table,
                             key_mask=maskd, part_tokens=part_tokens)

    def oracle(self, quantised=False):
        kf, vf = f64(self.k), f64(self.v)
        if quantised:  # the oracle's own fp8 codec on the same inputs
            kq = np.stack([OC.encode_rows(storage(self.k)[:, g], OC.BF16, OC.FP8_E4M3, self.scales[0][g])
                           for g in range(self.Hkv)], axis=1)
            vq = np.stack([OC.encode_rows(storage(self.v)[:, g], OC.BF16, OC.FP8_E4M3, self.scales[1][g])
                           for g in range(self.Hkv)], axis=1)
            kf = np.stack([codec.e4m3_decode(kq[:, g]) * np.float64(self.scales[0][g]) for g in range(self.Hkv)], 1)
            vf = np.stack([codec.e4m3_decode(vq[:, g]) * np.float64(self.scales[1][g]) for g in range(self.Hkv)], 1)
        keys = [kf[b] for b in range(self.B)]
        vals = [vf[b] for b in range(self.B)]
        return OA.decode(f64(self.q), keys, vals, self.lens, 1.0 / math.sqrt(self.d), key_mask=self.mask)


def test_tiny_config_decode_fp32_mha():
    """1 layer, batch 1, 4/4 heads, d 64, fp32, 128 cached + 1 appended key."""
    c = Case(1, 4, 4, 64, [129], dtype=K.F32, layout=K.CONTIGUOUS)
    got = c.run().cpu().numpy()
    assert max_abs(got, c.oracle()) <= TOL


EDGE_LENS = [1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 300, 511, 512, 513]


@pytest.mark.parametrize("layout", [K.PAGED, K.CONTIGUOUS])
@pytest.mark.parametrize("part", [64, 128, 0])
def test_bf16_gqa_edge_lengths(layout, part):
    c = Case(len(EDGE_LENS), 16, 4, 128, EDGE_LENS, layout=layout, seed=1)
    got = c.run(part).cpu().numpy()
    assert np.isfinite(got).all()
    assert max_abs(got, c.oracle()) <= TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_group_sizes(G, d):
    lens = [5, 77, 200, 33]
    c = Case(4, 2 * G, 2, d, lens, seed=2 + G)
    assert max_abs(c.run(64).cpu().numpy(), c.oracle()) <= TOL


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_cache(d):
    c = Case(3, 8, 2, d, [40, 129, 1], dtype=K.F32, seed=4)
    assert max_abs(c.run(64).cpu().numpy(), c.oracle()) <= TOL


@pytest.mark.parametrize("Hq,Hkv,d", [(8, 2, 128), (16, 2, 64), (4, 4, 64)])
def test_key_mask_with_nan_poisoned_padding(Hq, Hkv, d):
    """Masked keys carry NaN K/V: weights exactly 0, outputs finite
    ("Transformer Attention Masks and KV-Cache Inference", "Padding mask and
    batch length").  Group 4 and 8 (matrix-core pass, K staged through LDS
    with 256- and 128-byte rows) and group 1 (vector pass)."""
    lens = [100, 37, 260]
    mask = synth.random_mask((3, 272), 0.6, (5, synth.T_MASK))
    mask[:, 0] = 1
    c = Case(3, Hq, Hkv, d, lens, seed=5, mask=mask)
    for part in (64, 0):
        got = c.run(part).cpu().numpy()
        assert np.isfinite(got).all()
        assert max_abs(got, c.oracle()) <= TOL


def test_fully_masked_sequence_and_empty_sequence_output_zero():
    mask = np.ones((3, 80), np.uint8)
    mask[1, :] = 0
    c = Case(3, 4, 4, 64, [70, 70, 0], seed=6, mask=mask)
    got = c.run(64).cpu().numpy()
    assert np.all(got[1] == 0.0) and np.all(got[2] == 0.0)
    assert max_abs(got, c.oracle()) <= TOL


def test_constant_values_give_ones():
    """Softmax rows sum to 1: with V == 1 every output is 1."""
    c = Case(2, 8, 2, 128, [700, 45], seed=7)
    c.v.fill_(1.0)
    c._build_cache(7)
    got = c.run(128).cpu().numpy()
    assert np.abs(got - 1.0).max() <= 1e-6


def test_partition_sweep_agrees():
    c = Case(2, 8, 2, 128, [1500, 999], seed=8)
    ref = c.oracle()
    outs = [c.run(p).cpu().numpy() for p in (64, 128, 256, 512, 1024, 2048)]
    for o in outs:
        assert max_abs(o, ref) <= TOL
        assert max_abs(o, outs[0]) <= 1e-5


def test_paged_equals_contiguous_bitwise_and_deterministic():
    a = Case(3, 8, 2, 128, [333, 1, 600], layout=K.PAGED, seed=9)
    b = Case(3, 8, 2, 128, [333, 1, 600], layout=K.CONTIGUOUS, seed=9)
    for part in (64, 256):
        x1 = a.run(part).cpu()
        x2 = a.run(part).cpu()
        y = b.run(part).cpu()
        assert torch.equal(x1, x2)
        assert torch.equal(x1, y)


def test_gqa_equals_mha_with_repeated_heads():
    """Query head h reads KV head h // G ("KV Cache Fully Explained", "(2) GQA")."""
    lens = [90, 150]
    g = Case(2, 8, 2, 64, lens, seed=10)
    m = Case(2, 8, 8, 64, lens, seed=10)
    m.k = g.k.repeat_interleave(4, dim=1).contiguous()
    m.v = g.v.repeat_interleave(4, dim=1).contiguous()
    m.q = g.q.clone()
    m._build_cache(10)
    assert max_abs(g.run(64).cpu().numpy(), m.run(64).cpu().numpy()) <= 1e-5


def test_one_key_returns_its_value():
    c = Case(2, 4, 1, 128, [1, 1], seed=11)
    got = c.run().cpu().numpy()
    want = f64(c.v)[:, 0, 0]
    for h in range(4):
        assert max_abs(got[:, h], want) <= 1e-6


@pytest.mark.parametrize("Hq,d", [(4, 64), (8, 128), (16, 64)])
def test_invalid_block_ids_read_as_masked(Hq, d):
    """Out-of-range and negative block ids: those blocks read as masked
    (group 2: vector pass; groups 4 and 8: matrix-core pass)."""
    c = Case(2, Hq, 2, d, [64, 64], seed=12)
    bad = c.table.clone()
    bad[0, 1] = 10 ** 6   # positions 16..31 of sequence 0 unreadable
    bad[1, 3] = -1        # positions 48..63 of sequence 1
    got = K.attn_decode(c.cache, c.q.to(DEV), torch.from_numpy(c.lens).to(DEV), c.maxlen, block_table=bad,
                        part_tokens=64).cpu().numpy()
    mask = np.ones((2, 64), np.uint8)
    mask[0, 16:32] = 0
    mask[1, 48:64] = 0
    c.mask = mask
    assert max_abs(got, c.oracle()) <= TOL


@pytest.mark.parametrize("G,d", [(8, 128), (4, 64), (1, 128), (2, 64)])
def test_fp8_cache_vs_dequantised_oracle(G, d):
    """Kernel error alone: the oracle quantises the same inputs with its own
    E4M3FN codec and attends the dequantised values."""
    lens = [513, 64, 1000, 1]
    c = Case(4, 2 * G, 2, d, lens, dtype=K.FP8_E4M3, seed=13 + G)
    got = c.run(128).cpu().numpy()
    assert np.isfinite(got).all()
    assert max_abs(got, c.oracle(quantised=True)) <= TOL


def test_fp8_cache_vs_unquantised_oracle_at_long_context():
    """fp8 bar (3e-2) against the unquantised values, at the shape it is
    stated for: 64/8 heads, d 128, N(0,1) K/V, scales in [0.5, 2], long
    context (a 4096-key slice of the 131,073-key workload here).  The gap to
    the unquantised result is E4M3's own rounding, which shrinks as the
    softmax spreads over more keys; the kernel's part is the test above."""
    c = Case(2, 64, 8, 128, [4097, 2500], dtype=K.FP8_E4M3, seed=19)
    got = c.run(512).cpu().numpy()
    assert max_abs(got, c.oracle(quantised=True)) <= TOL
    assert max_abs(got, c.oracle(quantised=False)) <= TOL_FP8


def test_fp8_decode_table_through_attention():
    """Every E4M3FN code read back through a single-key attention: with one
    allowed key the output is that key's value row, dequantised exactly."""
    d = 128
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0  # the two NaN codes
    scales = np.array([1.0], np.float32)
    ks = torch.from_numpy(scales).to(DEV)
    cache = K.KVCache.paged(2, 1, d, K.FP8_E4M3, DEV, ks, ks)
    cache.k.zero_()
    cache.v.zero_()
    cache.v[0, 0, 0, :] = torch.from_numpy(codes[:128]).to(DEV)
    cache.v[1, 0, 0, :] = torch.from_numpy(codes[128:]).to(DEV)
    table = torch.tensor([[0], [1]], dtype=torch.int32, device=DEV)
    q = torch.zeros((2, 1, d), dtype=torch.bfloat16, device=DEV)
    got = K.attn_decode(cache, q, torch.tensor([1, 1], dtype=torch.int32, device=DEV), 1,
                        block_table=table).cpu().numpy()
    want = codec.e4m3_decode(codes).reshape(2, 128)
    np.testing.assert_array_equal(got[:, 0, :], want)


@pytest.mark.parametrize("G,d", [(8, 128), (4, 128), (8, 64), (4, 64)])
def test_fp8_gqa_key_mask_nan_codes_and_edge_lengths(G, d):
    """fp8 cache, GQA 4/8 (the matrix-core partition pass): a random key mask
    whose masked positions hold NaN codes, stale NaN codes in the tail slots,
    and lengths around the 16-token block and partition edges."""
    lens = [1, 15, 16, 17, 64, 129, 300]
    mask = synth.random_mask((len(lens), 304), 0.6, (21, synth.T_MASK))
    mask[:, 0] = 1
    c = Case(len(lens), 2 * G, 2, d, lens, dtype=K.FP8_E4M3, seed=21 + G + d, mask=mask)
    for part in (64, 128, 0):
        got = c.run(part).cpu().numpy()
        assert np.isfinite(got).all()
        assert max_abs(got, c.oracle(quantised=True)) <= TOL


def test_workspace_contents_on_entry_do_not_matter():
    """Workspace contents on entry are ignored: a workspace full of garbage
    (or of another call's partials) gives the same bits."""
    c = Case(3, 16, 4, 128, [900, 77, 1500], seed=50)
    lens = torch.from_numpy(c.lens).to(DEV)
    q = c.q.to(DEV)
    ws = K.decode_workspace(c.cache, 3, 16, c.maxlen, 64)
    ws.zero_()
    first = K.attn_decode(c.cache, q, lens, c.maxlen, block_table=c.table, workspace=ws, part_tokens=64).cpu()
    assert max_abs(first.numpy(), c.oracle()) <= TOL
    g = torch.Generator().manual_seed(7)
    for fill in ("random", "ones", "reuse"):
        if fill == "random":
            ws.copy_(torch.randint(-2 ** 31, 2 ** 31 - 1, ws.shape, generator=g, dtype=torch.int32).view(torch.float32))
        elif fill == "ones":
            ws.view(torch.int32).fill_(-1)
        again = K.attn_decode(c.cache, q, lens, c.maxlen, block_table=c.table, workspace=ws, part_tokens=64).cpu()
        assert torch.equal(again, first), fill


def test_merge_of_many_partitions():
    """938 partitions of one sequence (G = 8): the merge's long partition
    loop; same tolerance as ever, and a 59-partition split agrees."""
    c = Case(1, 8, 1, 64, [60001], seed=51)
    got = c.run(64).cpu().numpy()   # 938 partitions x 8 heads
    assert max_abs(got, c.oracle()) <= TOL
    ref = c.run(1024).cpu().numpy()  # 59 partitions: staged
    assert max_abs(got, ref) <= 1e-5


def test_graph_replay_matches_eager():
    """The decode and the fused decode step captured in a HIP graph: every
    replay (with eager work in between) equals the eager call bit for bit."""
    from tests.test_gpu_decode_append import StepCase
    c = StepCase(4, 32, 8, 128, [1000, 33, 700, 2048], seed=52)
    lens = torch.from_numpy(c.lens).to(DEV)
    q = c.q.to(DEV)
    k1, v1 = c.k1.to(DEV), c.v1.to(DEV)
    out = torch.empty((4, 32, 128), dtype=torch.float32, device=DEV)
    ws = K.decode_workspace(c.cache, 4, 32, c.maxlen, 64)  # also fits the part-128 calls
    eager_cache = c.clone_cache()
    want = K.attn_decode_append(eager_cache, q, k1, v1, lens, c.maxlen, block_table=c.table, workspace=ws,
                                part_tokens=128).clone()
    graph_cache = c.clone_cache()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        K.attn_decode_append(graph_cache, q, k1, v1, lens, c.maxlen, block_table=c.table, out=out, workspace=ws,
                             part_tokens=128)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        K.attn_decode_append(graph_cache, q, k1, v1, lens, c.maxlen, block_table=c.table, out=out, workspace=ws,
                             part_tokens=128)
    for r in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want), r
        # eager work on the same workspace between replays
        K.attn_decode(eager_cache, q, lens, c.maxlen, block_table=c.table, workspace=ws, part_tokens=64)
        torch.cuda.synchronize()
    np.testing.assert_array_equal(storage(graph_cache.k), storage(eager_cache.k))


def test_decode_maximum_batch_single_partition():
    """The largest batch the call takes (65,535 sequences, the grid's z
    extent), lengths 1..16 in one partition each (no merge launch), bf16
    contiguous cache, GQA 4: 1,024 sampled sequences (incl. the first and the
    last) against the oracle; every one-key sequence returns its V row
    exactly (one weight of exactly 1); every output lies within the range of
    its sequence's V rows (a convex combination; the margin is the parity
    tolerance: the weights the kernel applies carry about 16 bits, so their
    sum differs from the normaliser by about 2^-16)."""
    B, Hq, Hkv, d, cap = 65535, 8, 2, 64, 16
    G = Hq // Hkv
    gen = torch.Generator().manual_seed(60)
    k = torch.randn((B, Hkv, cap, d), generator=gen).to(torch.bfloat16)
    v = torch.randn((B, Hkv, cap, d), generator=gen).to(torch.bfloat16)
    q = torch.randn((B, Hq, d), generator=gen).to(torch.bfloat16)
    lens = (1 + np.arange(B) % 16).astype(np.int32)
    cache = K.KVCache.contiguous(B, Hkv, cap, d, K.BF16, DEV)
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    K.kv_append(cache, k.to(DEV), v.to(DEV), zeros, n_valid=torch.from_numpy(lens).to(DEV))
    out = K.attn_decode(cache, q.to(DEV), torch.from_numpy(lens).to(DEV), cap).cpu().numpy()
    assert np.isfinite(out).all()
    vf = v.float().numpy()
    one = lens == 1
    np.testing.assert_array_equal(out[one], np.repeat(vf[one, :, 0], G, axis=1))
    live = np.arange(cap)[None, :] < lens[:, None]                       # [B, cap]
    vmask = np.where(live[:, None, :, None], vf, np.nan)                  # [B, Hkv, cap, d]
    lo = np.repeat(np.nanmin(vmask, axis=2), G, axis=1)
    hi = np.repeat(np.nanmax(vmask, axis=2), G, axis=1)
    assert (out >= lo - TOL).all() and (out <= hi + TOL).all()
    picks = sorted({0, B - 1} | set(np.random.default_rng(61).choice(B, size=1022, replace=False).tolist()))
    kf, vd, qf = f64(k), f64(v), f64(q)
    scale = 1.0 / math.sqrt(d)
    for b in picks:
        want = OA.decode(qf[b:b + 1], [kf[b]], [vd[b]], [int(lens[b])], scale)
        assert max_abs(out[b:b + 1], want) <= TOL, b


@pytest.mark.parametrize("dtype,Hq", [(K.BF16, 1), (K.BF16, 2), (K.BF16, 8), (K.BF16, 16), (K.FP8_E4M3, 8),
                                      (K.F32, 4)])
def test_mqa_single_kv_head(dtype, Hq):
    """MQA: one KV head shared by every query head (the vector pass for 1 and
    2 heads and f32, the matrix-core passes for 8 and 16), against the oracle."""
    lens = [1, 64, 300, 513]
    c = Case(4, Hq, 1, 128, lens, dtype=dtype, seed=70 + Hq)
    got = c.run(128).cpu().numpy()
    if dtype == K.FP8_E4M3:
        assert max_abs(got, c.oracle(quantised=True)) <= TOL
    else:
        assert max_abs(got, c.oracle()) <= TOL
