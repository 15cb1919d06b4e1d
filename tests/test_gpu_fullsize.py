"""Full-size parity: the workloads bench.py times, built by bench.py's own
classes and run in the launch configuration it times (default partition
sizes, fused append), checked against the fp64 oracle on sampled outputs
that the oracle computes one by one ("Transformer Attention Masks and
KV-Cache Inference", section "Implementation and verification procedure":
decode with the cache equals the last row of a full recompute; "KV Cache,
Flash Attention and Inference Optimization", section "Flash Attention").

Each case samples the sequences or query rows at the edges of the workload
(shortest, longest, first and last rows) plus seeded random ones; integer
work (the appended rows, the prefill's cache write) is compared bit for bit
over the whole workload."""
import math

import numpy as np
import pytest
import torch

import kv_cache_decode_attn_amd as K
from oracle import attention as OA
from oracle import cache as OC
from tests.helpers import f64, max_abs, storage

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
TOL = 2e-3
TOL_FP8 = 3e-2


def _bench():
    import bench  # imported here: it needs the GPU library
    return bench


def _paged_rows(cache_t, table, b, positions):
    """Rows [len(positions), Hkv, d] of sequence b at the given positions of a
    paged pool [num_blocks, Hkv, 16, d], read through the block table."""
    pos = torch.as_tensor(positions, dtype=torch.long, device=cache_t.device)
    blk = table[b].long()[pos // 16]
    return cache_t[blk, :, pos % 16]


def _pick(lens, extra, seed):
    lens = np.asarray(lens)
    rng = np.random.default_rng(seed)
    picks = {int(np.argmin(lens)), int(np.argmax(lens))}
    picks.update(int(x) for x in rng.choice(len(lens), size=extra, replace=False))
    return sorted(picks)


def test_llama3_8b_decode_step_full_size():
    """Batch 32, 32/8 heads, d 128, bf16 paged cache, lengths U[1, 8192]: one
    fused append + decode step as timed; sampled sequences against the
    oracle's decode of the logical cache, every appended row bit for bit."""
    bench = _bench()
    w = bench.PagedDecode(replicas=1)
    w.step(0)
    torch.cuda.synchronize()
    c = w.caches[0]
    got = w.out.cpu().numpy()
    # the appended token of every sequence sits at position ctx - 1
    for b in range(w.B):
        p = int(w.ctx[b]) - 1
        k_row = _paged_rows(c.k, w.table, b, [p])[0]
        v_row = _paged_rows(c.v, w.table, b, [p])[0]
        assert torch.equal(k_row, w.k_new3[b]) and torch.equal(v_row, w.v_new3[b]), b
    scale = 1.0 / math.sqrt(w.D)
    for b in _pick(w.ctx, 3, 101):
        n = int(w.ctx[b])
        keys = [f64(w.src_k[b, :, :n])]
        vals = [f64(w.src_v[b, :, :n])]
        want = OA.decode(f64(w.q[b:b + 1]), keys, vals, [n], scale)
        assert max_abs(got[b:b + 1], want) <= TOL, (b, n)


def test_llama3_8b_verify_four_tokens_full_size():
    """The same workload with 4 drafted tokens per sequence stored and
    attended in one attn_decode_multi call: sampled sequences against the
    oracle's prefill with the cached prefix, the new rows bit for bit."""
    bench = _bench()
    w = bench.PagedVerify(replicas=1)
    w.step(0)
    torch.cuda.synchronize()
    c = w.caches[0]
    got = w.out.cpu().numpy()
    n_q = w.nq
    for b in range(w.B):
        ps = list(range(int(w.cached[b]), int(w.cached[b]) + n_q))
        assert torch.equal(_paged_rows(c.k, w.table, b, ps).transpose(0, 1), w.k_new[b]), b
        assert torch.equal(_paged_rows(c.v, w.table, b, ps).transpose(0, 1), w.v_new[b]), b
    scale = 1.0 / math.sqrt(w.D)
    # the cached prefix: the seeded source rows the workload appended (bf16
    # into a bf16 cache is a copy), regenerated from the generator
    from kv_cache_decode_attn_amd import synth
    width = int(w.ctx.max())
    src_k = synth.normal_device((w.B, w.Hkv, width, w.D), (9, synth.T_K))
    src_v = synth.normal_device((w.B, w.Hkv, width, w.D), (9, synth.T_V))
    for b in _pick(w.ctx, 3, 102):
        P = int(w.cached[b])
        want = OA.prefill(f64(w.q[b:b + 1]), f64(w.k_new[b:b + 1]), f64(w.v_new[b:b + 1]), np.array([P]),
                          np.array([n_q], np.int32), scale, causal=True, prefix_k=[f64(src_k[b, :, :P])],
                          prefix_v=[f64(src_v[b, :, :P])], attend_prefix=True)
        assert max_abs(got[b:b + 1], want) <= TOL, (b, P)


def test_padded_mha_decode_layer_full_size():
    """Batch 8, 32/32 heads, d 128, bf16 contiguous cache of 4,096 positions,
    real lengths U[512, 4096] with the padding mask: one layer's fused call as
    timed; every sequence and head against the oracle with the same mask."""
    bench = _bench()
    w = bench.PaddedDecode()
    c = w.caches[0]
    picks = list(range(w.B))
    keys = {b: f64(c.k[b]) for b in picks}   # the seeded cache contents, before the call
    vals = {b: f64(c.v[b]) for b in picks}
    out = K.attn_decode_append(c, w.q[0], w.k_new[0], w.v_new[0], w.seq_lens, w.cap, key_mask=w.mask,
                               workspace=w.ws, part_tokens=w.part).cpu().numpy()
    mask = w.mask.cpu().numpy()
    scale = 1.0 / math.sqrt(w.D)
    for b in picks:
        n = int(w.real[b])
        want = OA.decode(f64(w.q[0][b:b + 1]), [keys[b]], [vals[b]], [n], scale, key_mask=mask[b:b + 1])
        assert max_abs(out[b:b + 1], want) <= TOL, (b, n)


def test_llama3_70b_fp8_long_context_layer_full_size():
    """Batch 1, 64/8 heads, d 128, fp8 paged cache of 131,073 keys with
    per-head scales in [0.5, 2]: one layer's fused call in the timed
    partitioning (4,160 keys, one workgroup per compute unit).  All 64 query
    heads against the oracle on the values it quantises itself (2e-3) and on
    the unquantised values (3e-2)."""
    bench = _bench()
    from kv_cache_decode_attn_amd import synth
    w = bench.LongContextFp8Decode(layers=1)
    w.step(0)
    torch.cuda.synchronize()
    got = w.out[0].cpu().numpy()
    G = w.Hq // w.Hkv
    scale = 1.0 / math.sqrt(w.D)
    src_k = synth.normal_device((1, w.Hkv, w.ctx, w.D), (5, synth.T_K, 0))[0]
    src_v = synth.normal_device((1, w.Hkv, w.ctx, w.D), (5, synth.T_V, 0))[0]
    for g in range(w.Hkv):
        sk, sv = src_k[g], src_v[g]
        q = f64(w.q[0])[:, g * G:(g + 1) * G]
        mine = got[:, g * G:(g + 1) * G]
        want_u = OA.decode(q, [f64(sk)[None]], [f64(sv)[None]], [w.ctx], scale)
        assert max_abs(mine, want_u) <= TOL_FP8, g
        ks, vs = [np.float32(x) for x in w.scales[0, :, g].cpu().numpy()]
        kq = OC.to_f64(OC.encode_rows(storage(sk), OC.BF16, OC.FP8_E4M3, ks), OC.FP8_E4M3, ks)
        vq = OC.to_f64(OC.encode_rows(storage(sv), OC.BF16, OC.FP8_E4M3, vs), OC.FP8_E4M3, vs)
        want_q = OA.decode(q, [kq[None]], [vq[None]], [w.ctx], scale)
        assert max_abs(mine, want_q) <= TOL, g


def test_causal_prefill_8192_full_size():
    """Batch 1, 32/8 heads, 8,192 causal tokens, bf16, writing the paged
    cache: the timed call; sampled query rows of every head against the
    oracle (each row attends keys 0..t), and the whole cache write bit for
    bit through the block table."""
    bench = _bench()
    w = bench.CausalPrefill()
    w.step(0)
    torch.cuda.synchronize()
    rows = sorted({0, 1, 15, 16, 31, 32, 4095, 8190, 8191} |
                  set(int(x) for x in np.random.default_rng(104).choice(w.N, size=6, replace=False)))
    got = w.out[0][:, rows].cpu().numpy()
    kf, vf = f64(w.k[0]), f64(w.v[0])
    qf = f64(w.q[0][:, rows])
    G = w.Hq // w.Hkv
    scale = 1.0 / math.sqrt(w.D)
    allow = np.arange(w.N)[None, :] <= np.asarray(rows)[:, None]
    for h in range(w.Hq):
        want = OA.sdpa(qf[h], kf[h // G], vf[h // G], allow, scale)
        assert max_abs(got[h], want) <= TOL, h
    all_pos = list(range(w.N))
    assert torch.equal(_paged_rows(w.cache.k, w.table, 0, all_pos).transpose(0, 1), w.k[0])
    assert torch.equal(_paged_rows(w.cache.v, w.table, 0, all_pos).transpose(0, 1), w.v[0])


def test_chunked_prefill_6144_cached_2048_new_full_size():
    """A 2,048-token chunk of a 32/8-head layer at positions 6,144..8,191
    attending the 6,144 cached positions and, causally, itself (the timed
    attn_prefill with attend_prefix): sampled rows of every head against the
    oracle, and the chunk's cache write bit for bit."""
    bench = _bench()
    from kv_cache_decode_attn_amd import synth
    w = bench.ChunkedPrefill()
    w.step(0)
    torch.cuda.synchronize()
    std = 1.0 / math.sqrt(w.D)
    kp = synth.normal_device((1, w.Hkv, w.P, w.D), (8, synth.T_K), std=std)   # the appended prefix
    vp = synth.normal_device((1, w.Hkv, w.P, w.D), (8, synth.T_V), std=std)
    kf = np.concatenate([f64(kp[0]), f64(w.k[0])], axis=1)
    vf = np.concatenate([f64(vp[0]), f64(w.v[0])], axis=1)
    rows = sorted({0, 1, 31, 32, 1023, 2046, 2047} |
                  set(int(x) for x in np.random.default_rng(105).choice(w.n, size=5, replace=False)))
    got = w.out[0][:, rows].cpu().numpy()
    qf = f64(w.q[0][:, rows])
    G = w.Hq // w.Hkv
    scale = 1.0 / math.sqrt(w.D)
    allow = np.arange(w.P + w.n)[None, :] <= (w.P + np.asarray(rows))[:, None]
    for h in range(w.Hq):
        want = OA.sdpa(qf[h], kf[h // G], vf[h // G], allow, scale)
        assert max_abs(got[h], want) <= TOL, h
    new_pos = list(range(w.P, w.P + w.n))
    assert torch.equal(_paged_rows(w.cache.k, w.table, 0, new_pos).transpose(0, 1), w.k[0])
    assert torch.equal(_paged_rows(w.cache.v, w.table, 0, new_pos).transpose(0, 1), w.v[0])
    prefix_pos = list(range(w.P))
    assert torch.equal(_paged_rows(w.cache.k, w.table, 0, prefix_pos).transpose(0, 1), kp[0])


def test_chunked_prefill_fp8_cache_full_size():
    """The same 2,048-token chunk against an fp8 (E4M3FN) cache of the 6,144
    positions (the timed chunkprefill_fp8 call): sampled rows of every head
    against the oracle with the cached rows dequantised by the oracle's own
    codec, and the chunk's codes in the cache bit for bit against the
    oracle's encoder."""
    bench = _bench()
    from kv_cache_decode_attn_amd import synth
    w = bench.ChunkedPrefill(kv_dtype=K.FP8_E4M3)
    w.step(0)
    torch.cuda.synchronize()
    std = 1.0 / math.sqrt(w.D)
    kp = synth.normal_device((1, w.Hkv, w.P, w.D), (8, synth.T_K), std=std)   # the appended prefix
    vp = synth.normal_device((1, w.Hkv, w.P, w.D), (8, synth.T_V), std=std)
    ks = w.cache.k_scale.cpu().numpy()
    vs = w.cache.v_scale.cpu().numpy()

    def deq(x, sc):
        return np.stack([OC.to_f64(OC.encode_rows(storage(x[0])[g], OC.BF16, OC.FP8_E4M3, sc[g]), OC.FP8_E4M3, sc[g])
                         for g in range(w.Hkv)])
    kf = np.concatenate([deq(kp, ks), f64(w.k[0])], axis=1)
    vf = np.concatenate([deq(vp, vs), f64(w.v[0])], axis=1)
    rows = sorted({0, 1, 31, 32, 1023, 2046, 2047} |
                  set(int(x) for x in np.random.default_rng(106).choice(w.n, size=5, replace=False)))
    got = w.out[0][:, rows].cpu().numpy()
    qf = f64(w.q[0][:, rows])
    G = w.Hq // w.Hkv
    scale = 1.0 / math.sqrt(w.D)
    allow = np.arange(w.P + w.n)[None, :] <= (w.P + np.asarray(rows))[:, None]
    for h in range(w.Hq):
        want = OA.sdpa(qf[h], kf[h // G], vf[h // G], allow, scale)
        assert max_abs(got[h], want) <= TOL, h
    new_pos = [0, 1, 15, 16, 1000, 2047]
    got_k = _paged_rows(w.cache.k, w.table, 0, [w.P + i for i in new_pos]).cpu().numpy()  # [n, Hkv, D] codes
    got_v = _paged_rows(w.cache.v, w.table, 0, [w.P + i for i in new_pos]).cpu().numpy()
    for j, i in enumerate(new_pos):
        for g in range(w.Hkv):
            np.testing.assert_array_equal(got_k[j, g], OC.encode_rows(storage(w.k[0, g, i]), OC.BF16, OC.FP8_E4M3,
                                                                     ks[g]))
            np.testing.assert_array_equal(got_v[j, g], OC.encode_rows(storage(w.v[0, g, i]), OC.BF16, OC.FP8_E4M3,
                                                                     vs[g]))
