"""Benchmark of the KV-cache attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads ...]

Prints ONE JSON line.  The headline workload (`value`) is the Llama-3-8B-
shaped paged GQA decode step: batch 32, 32 query / 8 KV heads, head_dim 128,
bf16 cache in 16-token blocks behind a permuted block table, cached lengths
uniform in [1, 8192]; a step appends one token per sequence and attends it,
in one library call (attn_decode_append: the split-K partition pass, which
also stores the new token, then the merge pass).  `value` is algorithmic
HBM bytes per step / step time, in GB/s.  The same step as two calls
(kv_append, then attn_decode) is timed too and reported beside it.

Other workloads run in the same invocation and are reported under
"workloads": the padded 32-layer MHA decode (batch 8, 4096-position
contiguous cache, key padding mask), the 80-layer fp8 long-context decode
(batch 1, 64/8 heads, 131,073 keys per layer), the check of 4 drafted
tokens per sequence on the Llama-3-8B decode workload (append, then all 4
attended together), the causal 8192-token prefill that writes the paged
cache, a 2048-token chunked prefill against
6144 cached positions, a copy-on-write fan-out of 4096 paged blocks and a
contiguous beam reorder (32 rows of 4096 positions).

Timing: W untimed warm-up steps, then K steps bracketed by synchronize +
HIP events on the stream the library launches on (torch's current stream).
Each decode step reads a different replica of the cache (round-robin) so the
256 MB Infinity Cache cannot serve the previous step's bytes.  A second pass
of K steps with HIP events around every call gives the call's own duration
for the roofline (kept out of the first pass: event records between kernels
cost a few microseconds each).  The CPU baseline is the fp64 oracle on the host, timed on the
same inputs (single thread).
"""
import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import kv_cache_decode_attn_amd as K  # noqa: E402
from kv_cache_decode_attn_amd import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, TFLOP/s (256 CU x 4096 flop/clk x 2.4 GHz)
METRIC = "decode-attn HBM GB/s (% of peak) & seqs/s; prefill TFLOP/s (% MFMA peak)"
DEV = "cuda"


DECODE_SOURCES = ("kv_cache_decode_attn_amd/csrc/decode.hip", "kv_cache_decode_attn_amd/csrc/common.h")
LAUNCH_HEADER = "kv_cache_decode_attn_amd/csrc/launch.h"


def _decode_struct(text):
    """The DecodeLaunch declaration of launch.h: the only part of that
    header the decode kernels compile against."""
    i = text.index("struct DecodeLaunch {")
    return text[i:text.index("};", i) + 2]


def decode_source_sha(read=None):
    """Hash of the sources the decode kernels are built from."""
    if read is None:
        def read(rel):
            with open(os.path.join(ROOT, rel), "rb") as f:
                return f.read()
    h = hashlib.sha256()
    for rel in DECODE_SOURCES:
        h.update(read(rel))
    h.update(_decode_struct(read(LAUNCH_HEADER).decode()).encode())
    return h.hexdigest()


def decode_traffic():
    """HBM bytes per attn_decode call measured with rocprofv3 counters
    (profiles/decode_traffic.json), or None when that measurement was taken
    on different decode kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", "decode_traffic.json")) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_sha256") != decode_source_sha():
        return None
    return d.get("bytes_per_call")


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "min_ms": float(a.min()), "p90_ms": float(np.percentile(a, 90)),
            "mean_ms": float(a.mean())}


# ------------------------------------------------------------------ decode ---

class PagedDecode:
    """Llama-3-8B-shaped paged GQA decode step (one layer)."""

    name = "llama3-8b-paged-gqa-decode"

    def __init__(self, replicas=4, wid=2, fused=True, batch=32, min_cached=1):
        self.fused = fused
        self.B, self.Hq, self.Hkv, self.D = batch, 32, 8, 128
        self.cached = synth.uniform_lengths(self.B, min_cached, 8192, (wid, synth.T_LENS))
        self.ctx = (self.cached + 1).astype(np.int32)          # keys incl. the appended token
        self.maxlen = int(self.ctx.max()) if self.B else 0
        self.max_seq_len = 8193
        nbs = [synth.blocks_for(c) for c in self.ctx]
        self.max_blocks = 513
        table, self.nblk = synth.block_table(nbs, self.max_blocks, (wid, synth.T_PERM))
        self.table = torch.from_numpy(table).to(DEV)
        # logical K/V of every position, the query, and the new token's K/V
        width = self.maxlen
        self.src_k = synth.normal_device((self.B, self.Hkv, width, self.D), (wid, synth.T_K))
        self.src_v = synth.normal_device((self.B, self.Hkv, width, self.D), (wid, synth.T_V))
        self.q = synth.normal_device((self.B, self.Hq, self.D), (wid, synth.T_Q))
        idx = torch.from_numpy(self.cached.astype(np.int64)).to(DEV).view(self.B, 1, 1, 1).expand(
            self.B, self.Hkv, 1, self.D)
        self.k_new = torch.gather(self.src_k, 2, idx).contiguous()
        self.v_new = torch.gather(self.src_v, 2, idx).contiguous()
        self.k_new3 = self.k_new[:, :, 0].contiguous()   # [B, Hkv, D] rows of the fused call
        self.v_new3 = self.v_new[:, :, 0].contiguous()
        self.positions = torch.from_numpy(self.cached).to(DEV)
        self.seq_lens = torch.from_numpy(self.ctx).to(DEV)
        zeros = torch.zeros(self.B, dtype=torch.int32, device=DEV)
        self.caches = []
        for _ in range(replicas):
            c = K.KVCache.paged(self.nblk, self.Hkv, self.D, K.BF16, DEV)
            K.kv_append(c, self.src_k, self.src_v, zeros, block_table=self.table, n_valid=self.positions)
            self.caches.append(c)
        self.out = torch.empty((self.B, self.Hq, self.D), dtype=torch.float32, device=DEV)
        self.part = K.decode_default_part_tokens(K.BF16, self.B, self.Hq, self.Hkv, self.max_seq_len)
        self.ws = K.decode_workspace(self.caches[0], self.B, self.Hq, self.max_seq_len, self.part)
        torch.cuda.synchronize()

    def kv_bytes(self):
        return 2 * self.Hkv * self.D * 2 * int(self.ctx.sum())

    def decode_bytes(self):
        """Algorithmic bytes of one attn_decode call: K/V of every attended
        key, the query, the fp32 output, the block-table entries and lengths."""
        blocks = sum(synth.blocks_for(c) for c in self.ctx)
        return self.kv_bytes() + self.B * self.Hq * self.D * 2 + self.B * self.Hq * self.D * 4 + 4 * blocks + 4 * self.B

    def append_bytes(self):
        return 2 * (2 * self.B * self.Hkv * self.D * 2) + 4 * self.B + 4 * self.B

    def step_bytes(self):
        return self.decode_bytes() + self.append_bytes()

    def step(self, i, ev=None):
        c = self.caches[i % len(self.caches)]
        if ev:
            ev[0].record()
        if self.fused:
            K.attn_decode_append(c, self.q, self.k_new3, self.v_new3, self.seq_lens, self.max_seq_len,
                                 block_table=self.table, out=self.out, workspace=self.ws, part_tokens=self.part)
            if ev:
                ev[1].record()
            return
        K.kv_append(c, self.k_new, self.v_new, self.positions, block_table=self.table)
        if ev:
            ev[1].record()
        K.attn_decode(c, self.q, self.seq_lens, self.max_seq_len, block_table=self.table, out=self.out,
                      workspace=self.ws, part_tokens=self.part)
        if ev:
            ev[2].record()

    def launch_names(self):
        """Names of the calls the per-launch events of step() bracket."""
        return ("attn_decode_append",) if self.fused else ("kv_append", "attn_decode")

    def config(self):
        return {"workload": self.name, "batch": self.B, "q_heads": self.Hq, "kv_heads": self.Hkv,
                "head_dim": self.D, "kv_dtype": "bf16", "block_tokens": 16, "keys_total": int(self.ctx.sum()),
                "cached_len": "U[1,8192] + 1 appended", "part_tokens": self.part, "cache_replicas": len(self.caches)}

    def cpu_baseline(self, max_seqs=None, min_seconds=10.0):
        """The oracle on the same bytes, single thread: bf16 -> fp64 decode of
        the cache plus the attention, timed; returns (result dict, max abs err)."""
        from threadpoolctl import threadpool_limits

        from oracle import attention as OA
        from oracle import cache as OC

        seqs = list(range(self.B if max_seqs is None else min(max_seqs, self.B)))
        kh = [self.src_k[b, :, :self.ctx[b]].cpu().view(torch.int16).numpy().view(np.uint16) for b in seqs]
        vh = [self.src_v[b, :, :self.ctx[b]].cpu().view(torch.int16).numpy().view(np.uint16) for b in seqs]
        qh = self.q[seqs].cpu().view(torch.int16).numpy().view(np.uint16)
        # the whole decode (bf16 decode of the cache + attention) repeated
        # until about min_seconds of single-thread CPU time has run
        reps = 0
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            while True:
                keys = [OC.to_f64(x, OC.BF16) for x in kh]
                vals = [OC.to_f64(x, OC.BF16) for x in vh]
                want = OA.decode(OC.to_f64(qh, OC.BF16), keys, vals, self.ctx[seqs], 1.0 / math.sqrt(self.D))
                reps += 1
                dt = time.perf_counter() - t0
                if dt >= min_seconds:
                    break
        # the GPU output of the last timed step covers the same sequences
        got = self.out[seqs].cpu().numpy()
        err = float(np.abs(got - want).max())
        nbytes = 2 * self.Hkv * self.D * 2 * int(self.ctx[seqs].sum())
        res = {"value": reps * nbytes / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": "%d of %d sequences (%d keys, %.0f MB of K/V) x %d repetitions, fp64 numpy, 1 thread, "
                         "%.1f s; %s" % (len(seqs), self.B, int(self.ctx[seqs].sum()), nbytes / 1e6, reps, dt,
                                         platform.processor() or platform.machine()),
               "seqs_per_s": reps * len(seqs) / dt}
        return res, err


class PaddedDecode:
    """Padded-batch MHA decode over 32 layers with a key padding mask."""

    name = "padded-mha-decode-32-layers"

    def __init__(self, wid=3):
        self.L, self.B, self.H, self.D, self.cap = 32, 8, 32, 128, 4096
        self.real = synth.uniform_lengths(self.B, 512, 4096, (wid, synth.T_LENS))
        self.mask = torch.from_numpy(synth.padding_mask(self.real, self.cap)).to(DEV)
        self.seq_lens = torch.from_numpy(self.real).to(DEV)
        self.positions = torch.from_numpy(self.real - 1).to(DEV)
        self.caches, self.k_new, self.v_new, self.q = [], [], [], []
        idx = torch.from_numpy((self.real - 1).astype(np.int64)).to(DEV).view(self.B, 1, 1, 1).expand(
            self.B, self.H, 1, self.D)
        for layer in range(self.L):
            c = K.KVCache.contiguous(self.B, self.H, self.cap, self.D, K.BF16, DEV)
            synth.normal_device(c.k.shape, (wid, synth.T_K, layer), out=c.k)
            synth.normal_device(c.v.shape, (wid, synth.T_V, layer), out=c.v)
            self.caches.append(c)
            # the new token is the one at real_b - 1 (re-written in place each step)
            self.k_new.append(torch.gather(c.k, 2, idx)[:, :, 0].contiguous())
            self.v_new.append(torch.gather(c.v, 2, idx)[:, :, 0].contiguous())
            self.q.append(synth.normal_device((self.B, self.H, self.D), (wid, synth.T_Q, layer)))
        self.out = torch.empty((self.L, self.B, self.H, self.D), dtype=torch.float32, device=DEV)
        self.part = K.decode_default_part_tokens(K.BF16, self.B, self.H, self.H, self.cap)
        self.ws = K.decode_workspace(self.caches[0], self.B, self.H, self.cap, self.part)
        torch.cuda.synchronize()

    def step_bytes(self):
        per_layer = (2 * self.H * self.D * 2 * int(self.real.sum()) + self.B * self.H * self.D * (2 + 4)
                     + 2 * 2 * self.B * self.H * self.D * 2 + int(self.real.sum()) + 8 * self.B)
        return self.L * per_layer

    def step(self, i, ev=None):
        for layer in range(self.L):
            K.attn_decode_append(self.caches[layer], self.q[layer], self.k_new[layer], self.v_new[layer],
                                 self.seq_lens, self.cap, key_mask=self.mask, out=self.out[layer], workspace=self.ws,
                                 part_tokens=self.part)

    def config(self):
        return {"workload": self.name, "layers": self.L, "batch": self.B, "q_heads": self.H, "kv_heads": self.H,
                "head_dim": self.D, "kv_dtype": "bf16", "capacity": self.cap, "real_len": "U[512,4096]",
                "part_tokens": self.part}


class LongContextFp8Decode:
    """Llama-3-70B-shaped fp8 long-context decode over 80 layers, batch 1."""

    name = "llama3-70b-fp8-longctx-decode-80-layers"

    def __init__(self, wid=5, layers=80):
        self.L, self.B, self.Hq, self.Hkv, self.D = layers, 1, 64, 8, 128
        self.cached = 131072
        self.ctx = self.cached + 1
        nb = synth.blocks_for(self.ctx)
        self.caches, self.k_new, self.v_new, self.q, self.tables = [], [], [], [], []
        scales = synth.fp8_scales(self.L * self.Hkv * 2, (wid, synth.T_SCALE)).reshape(self.L, 2, self.Hkv)
        self.scales = torch.from_numpy(scales).to(DEV)
        zeros = torch.zeros(1, dtype=torch.int32, device=DEV)
        pos = torch.tensor([self.cached], dtype=torch.int32, device=DEV)
        self.positions, self.seq_lens = pos, torch.tensor([self.ctx], dtype=torch.int32, device=DEV)
        for layer in range(self.L):
            table, nblk = synth.block_table([nb], nb, (wid, synth.T_PERM, layer))
            tdev = torch.from_numpy(table).to(DEV)
            c = K.KVCache.paged(nblk, self.Hkv, self.D, K.FP8_E4M3, DEV, self.scales[layer, 0].contiguous(),
                                self.scales[layer, 1].contiguous())
            sk = synth.normal_device((1, self.Hkv, self.ctx, self.D), (wid, synth.T_K, layer))
            sv = synth.normal_device((1, self.Hkv, self.ctx, self.D), (wid, synth.T_V, layer))
            K.kv_append(c, sk, sv, zeros, block_table=tdev, n_valid=pos)
            self.k_new.append(sk[:, :, self.cached].contiguous())
            self.v_new.append(sv[:, :, self.cached].contiguous())
            del sk, sv
            self.caches.append(c)
            self.tables.append(tdev)
            self.q.append(synth.normal_device((1, self.Hq, self.D), (wid, synth.T_Q, layer)))
        self.out = torch.empty((self.L, 1, self.Hq, self.D), dtype=torch.float32, device=DEV)
        self.part = K.decode_default_part_tokens(K.FP8_E4M3, 1, self.Hq, self.Hkv, self.ctx)
        self.ws = K.decode_workspace(self.caches[0], 1, self.Hq, self.ctx, self.part)
        torch.cuda.synchronize()

    def step_bytes(self):
        per_layer = (2 * self.Hkv * self.D * self.ctx + self.Hq * self.D * (2 + 4) + 2 * self.Hkv * self.D * (2 + 1)
                     + 4 * synth.blocks_for(self.ctx) + 16)
        return self.L * per_layer

    def step(self, i, ev=None):
        for layer in range(self.L):
            K.attn_decode_append(self.caches[layer], self.q[layer], self.k_new[layer], self.v_new[layer],
                                 self.seq_lens, self.ctx, block_table=self.tables[layer], out=self.out[layer],
                                 workspace=self.ws, part_tokens=self.part)

    def config(self):
        return {"workload": self.name, "layers": self.L, "batch": 1, "q_heads": self.Hq, "kv_heads": self.Hkv,
                "head_dim": self.D, "kv_dtype": "fp8_e4m3", "keys": self.ctx, "part_tokens": self.part}


class CausalPrefill:
    """Causal 8192-token prefill, GQA 32/8, d 128, bf16, writing the paged cache."""

    name = "causal-prefill-8192-gqa"

    def __init__(self, wid=4):
        self.B, self.Hq, self.Hkv, self.N, self.D = 1, 32, 8, 8192, 128
        std = 1.0 / math.sqrt(self.D)
        self.q = synth.normal_device((1, self.Hq, self.N, self.D), (wid, synth.T_Q), std=std)
        self.k = synth.normal_device((1, self.Hkv, self.N, self.D), (wid, synth.T_KNEW), std=std)
        self.v = synth.normal_device((1, self.Hkv, self.N, self.D), (wid, synth.T_VNEW), std=std)
        nb = self.N // 16
        table, nblk = synth.block_table([nb], nb, (wid, synth.T_PERM))
        self.table = torch.from_numpy(table).to(DEV)
        self.cache = K.KVCache.paged(nblk, self.Hkv, self.D, K.BF16, DEV)
        self.positions = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.out = torch.empty((1, self.Hq, self.N, self.D), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()

    def flops(self):
        return 2 * self.D * self.Hq * self.N * (self.N + 1)  # QK^T and PV over the causal triangle

    def step(self, i, ev=None):
        K.attn_prefill(self.q, self.k, self.v, cache=self.cache, positions=self.positions, block_table=self.table,
                       out=self.out)

    def config(self):
        return {"workload": self.name, "batch": 1, "q_heads": self.Hq, "kv_heads": self.Hkv, "seq": self.N,
                "head_dim": self.D, "dtype": "bf16", "causal": True, "writes_paged_cache": True}


class ChunkedPrefill:
    """Chunked prefill against a paged bf16 cache: a 2,048-token chunk of a
    Llama-3-8B-shaped layer (32/8 heads, d 128) at positions 6,144..8,191 that
    attends the 6,144 cached positions and, causally, itself, and stores its
    rows in the cache (attn_prefill with attend_prefix)."""

    name = "chunked-prefill-6144-cached-2048-new-gqa"

    def __init__(self, wid=8, P=6144, n=2048):
        self.Hq, self.Hkv, self.D, self.P, self.n = 32, 8, 128, P, n
        std = 1.0 / math.sqrt(self.D)
        nb = synth.blocks_for(P + n)
        table, nblk = synth.block_table([nb], nb, (wid, synth.T_PERM))
        self.table = torch.from_numpy(table).to(DEV)
        self.cache = K.KVCache.paged(nblk, self.Hkv, self.D, K.BF16, DEV)
        kp = synth.normal_device((1, self.Hkv, P, self.D), (wid, synth.T_K), std=std)
        vp = synth.normal_device((1, self.Hkv, P, self.D), (wid, synth.T_V), std=std)
        K.kv_append(self.cache, kp, vp, torch.zeros(1, dtype=torch.int32, device=DEV), block_table=self.table)
        del kp, vp
        self.q = synth.normal_device((1, self.Hq, n, self.D), (wid, synth.T_Q), std=std)
        self.k = synth.normal_device((1, self.Hkv, n, self.D), (wid, synth.T_KNEW), std=std)
        self.v = synth.normal_device((1, self.Hkv, n, self.D), (wid, synth.T_VNEW), std=std)
        self.positions = torch.tensor([P], dtype=torch.int32, device=DEV)
        self.out = torch.empty((1, self.Hq, n, self.D), dtype=torch.float32, device=DEV)
        torch.cuda.synchronize()

    def flops(self):
        # QK^T and PV over the attended (query, key) pairs: every cached key,
        # and the causal triangle of the chunk incl. its diagonal
        pairs = self.n * self.P + self.n * (self.n + 1) // 2
        return 4 * self.D * self.Hq * pairs

    def step(self, i, ev=None):
        K.attn_prefill(self.q, self.k, self.v, cache=self.cache, positions=self.positions, block_table=self.table,
                       attend_prefix=True, out=self.out)

    def config(self):
        return {"workload": self.name, "batch": 1, "q_heads": self.Hq, "kv_heads": self.Hkv, "cached": self.P,
                "new": self.n, "head_dim": self.D, "dtype": "bf16", "causal": True, "writes_paged_cache": True}


class PagedVerify:
    """Checking drafted tokens: the Llama-3-8B-shaped paged decode workload
    (batch 32, 32/8 heads, d 128, bf16, cached lengths U[1, 8192]) with 4 new
    tokens per sequence stored in the cache and attended together, causal
    among themselves, in one attn_decode_multi call (16 query columns per KV
    head; each partition's workgroup stores the new rows in its key range)."""

    name = "llama3-8b-paged-gqa-verify-4-tokens"

    def __init__(self, replicas=4, wid=9, n_q=4):
        self.B, self.Hq, self.Hkv, self.D, self.nq = 32, 32, 8, 128, n_q
        self.cached = synth.uniform_lengths(self.B, 1, 8192, (wid, synth.T_LENS))
        self.ctx = (self.cached + n_q).astype(np.int32)
        self.max_seq_len = 8192 + n_q
        nbs = [synth.blocks_for(c) for c in self.ctx]
        self.max_blocks = synth.blocks_for(self.max_seq_len)
        table, self.nblk = synth.block_table(nbs, self.max_blocks, (wid, synth.T_PERM))
        self.table = torch.from_numpy(table).to(DEV)
        width = int(self.ctx.max())
        src_k = synth.normal_device((self.B, self.Hkv, width, self.D), (wid, synth.T_K))
        src_v = synth.normal_device((self.B, self.Hkv, width, self.D), (wid, synth.T_V))
        self.q = synth.normal_device((self.B, self.Hq, n_q, self.D), (wid, synth.T_Q))
        idx = torch.from_numpy(self.cached.astype(np.int64)).to(DEV).view(self.B, 1, 1, 1) + \
            torch.arange(n_q, device=DEV).view(1, 1, n_q, 1)
        idx = idx.expand(self.B, self.Hkv, n_q, self.D)
        self.k_new = torch.gather(src_k, 2, idx).contiguous()
        self.v_new = torch.gather(src_v, 2, idx).contiguous()
        self.positions = torch.from_numpy(self.cached).to(DEV)
        self.seq_lens = torch.from_numpy(self.ctx).to(DEV)
        zeros = torch.zeros(self.B, dtype=torch.int32, device=DEV)
        self.caches = []
        for _ in range(replicas):
            c = K.KVCache.paged(self.nblk, self.Hkv, self.D, K.BF16, DEV)
            K.kv_append(c, src_k, src_v, zeros, block_table=self.table, n_valid=self.positions)
            self.caches.append(c)
        del src_k, src_v
        self.out = torch.empty((self.B, self.Hq, n_q, self.D), dtype=torch.float32, device=DEV)
        self.part = K.decode_default_part_tokens(K.BF16, self.B, self.Hq * n_q, self.Hkv, self.max_seq_len)
        self.ws = K.decode_workspace(self.caches[0], self.B, self.Hq * n_q, self.max_seq_len, self.part)
        torch.cuda.synchronize()

    def step_bytes(self):
        """K/V of every attended key (4096 B per key over the 8 KV heads), q,
        the fp32 output, the block table and lengths, and the appended rows
        (read and written)."""
        blocks = sum(synth.blocks_for(c) for c in self.ctx)
        kv = 2 * self.Hkv * self.D * 2 * int(self.ctx.sum())
        new = 2 * 2 * self.B * self.Hkv * self.nq * self.D * 2
        return kv + self.B * self.Hq * self.nq * self.D * (2 + 4) + 4 * blocks + 8 * self.B + new

    def step(self, i, ev=None):
        c = self.caches[i % len(self.caches)]
        K.attn_decode_multi(c, self.q, self.seq_lens, self.max_seq_len, k_new=self.k_new, v_new=self.v_new,
                            block_table=self.table, out=self.out, workspace=self.ws, part_tokens=self.part)

    def config(self):
        return {"workload": self.name, "batch": self.B, "q_heads": self.Hq, "kv_heads": self.Hkv, "new_tokens": self.nq,
                "head_dim": self.D, "kv_dtype": "bf16", "block_tokens": 16, "keys_total": int(self.ctx.sum()),
                "cached_len": "U[1,8192] + 4 appended", "part_tokens": self.part}


class CowBlockCopy:
    """Copy-on-write fan-out: 4096 whole-block copies in a Llama-3-8B-shaped
    bf16 paged pool (8 KV heads x 16 positions x 128 = 32 KiB per block per
    pool), K and V, one kvattn_copy_blocks launch per step."""

    name = "cow-block-copy-4096-llama3-8b"

    def __init__(self, wid=6, replicas=4):
        self.nblk, self.n, self.Hkv, self.D = 16384, 4096, 8, 128
        self.caches, self.src, self.dst = [], [], []
        for r in range(replicas):
            c = K.KVCache.paged(self.nblk, self.Hkv, self.D, K.BF16, DEV)
            synth.normal_device(c.k.shape, (wid, synth.T_K, r), out=c.k)
            synth.normal_device(c.v.shape, (wid, synth.T_V, r), out=c.v)
            perm = synth.rng(wid, synth.T_PERM, r).permutation(self.nblk).astype(np.int32)
            self.caches.append(c)
            self.src.append(torch.from_numpy(perm[:self.n].copy()).to(DEV))
            self.dst.append(torch.from_numpy(perm[self.n:2 * self.n].copy()).to(DEV))
        torch.cuda.synchronize()

    def step_bytes(self):
        block = self.Hkv * 16 * self.D * 2
        return 2 * 2 * self.n * block + 8 * self.n  # K and V, read + write, plus the id pairs

    def step(self, i, ev=None):
        r = i % len(self.caches)
        K.copy_blocks(self.caches[r], self.src[r], self.dst[r])

    def config(self):
        return {"workload": self.name, "pairs": self.n, "pool_blocks": self.nblk, "kv_heads": self.Hkv,
                "head_dim": self.D, "kv_dtype": "bf16", "block_bytes_per_pool": self.Hkv * 16 * self.D * 2}


class BeamReorder:
    """Beam reorder of a contiguous Llama-3-8B-shaped bf16 cache layer: 32
    rows (8 prompts x 4 beams, each beam's parent drawn from its prompt's
    beams), 8 KV heads, capacity 4096, d 128, lengths U[1024, 4096]; one
    kvattn_reorder_cache launch per step copies each row's stored
    positions."""

    name = "beam-reorder-contiguous-32x4096-llama3-8b"

    def __init__(self, wid=7, replicas=3):
        self.rows, self.Hkv, self.cap, self.D = 32, 8, 4096, 128
        self.lens_np = synth.uniform_lengths(self.rows, 1024, self.cap, (wid, synth.T_LENS))
        r = synth.rng(wid, synth.T_PERM)
        self.perm_np = np.concatenate([4 * p + r.integers(0, 4, size=4) for p in range(8)]).astype(np.int32)
        self.lens = torch.from_numpy(self.lens_np).to(DEV)
        self.perm = torch.from_numpy(self.perm_np).to(DEV)
        self.out_lens = torch.empty(self.rows, dtype=torch.int32, device=DEV)
        self.pairs = []
        for k in range(replicas):
            s = K.KVCache.contiguous(self.rows, self.Hkv, self.cap, self.D, K.BF16, DEV)
            d = K.KVCache.contiguous(self.rows, self.Hkv, self.cap, self.D, K.BF16, DEV)
            synth.normal_device(s.k.shape, (wid, synth.T_K, k), out=s.k)
            synth.normal_device(s.v.shape, (wid, synth.T_V, k), out=s.v)
            self.pairs.append((s, d))
        torch.cuda.synchronize()

    def step_bytes(self):
        moved = int(np.minimum(self.lens_np[self.perm_np], self.cap).sum())
        return 2 * 2 * moved * self.Hkv * self.D * 2 + 4 * 3 * self.rows  # K and V, read + write; perm, lengths

    def step(self, i, ev=None):
        s, d = self.pairs[i % len(self.pairs)]
        K.reorder_cache(s, d, self.perm, self.lens, self.out_lens)

    def config(self):
        return {"workload": self.name, "rows": self.rows, "kv_heads": self.Hkv, "capacity": self.cap,
                "head_dim": self.D, "kv_dtype": "bf16", "lengths": "U[1024,4096]", "beams_per_prompt": 4}


def time_steps(w, steps, warmup, per_launch=False):
    for i in range(warmup):
        w.step(i)
    torch.cuda.synchronize()
    evs = [_events(3) for _ in range(steps)] if per_launch else [None] * steps
    start, end = _events(2)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        w.step(warmup + i, evs[i])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    launch = None
    if per_launch:
        launch = {n: _stats([e[k].elapsed_time(e[k + 1]) for e in evs]) for k, n in enumerate(w.launch_names())}
    return total_ms / steps, launch


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads",
                    default="decode8b,padded32,longctx70b,verify8b,prefill8k,chunkprefill,cowcopy,beamreorder",
                    help="comma list: decode8b (headline), padded32, longctx70b, verify8b, prefill8k, chunkprefill, "
                         "cowcopy, beamreorder")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=None, help="sequences of the headline workload the oracle runs")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library is a single-GPU kernel library and this build runs on a "
              "one-GPU box (how the path would shard is described in the design notes).", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    names = [x for x in args.workloads.split(",") if x]

    w = PagedDecode()
    # the same step as two calls (kv_append, attn_decode), for reference
    w.fused = False
    ms2, _ = time_steps(w, args.steps, args.warmup)
    _, launch2 = time_steps(w, args.steps, args.warmup, per_launch=True)
    w.fused = True
    # `value`: K steps with nothing else in the timed region; then a second
    # pass with HIP events around every call for the call's own duration
    # (the event records themselves add a few microseconds per step)
    ms, _ = time_steps(w, args.steps, args.warmup)
    _, launch = time_steps(w, args.steps, args.warmup, per_launch=True)
    step_bytes = w.step_bytes()
    call_ms = launch["attn_decode_append"]["mean_ms"]
    achieved = step_bytes / (call_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": step_bytes / (ms * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 K/V/Q, seeded lengths and block permutation)",
        "config": w.config(),
        "frac_of_hbm_peak": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "seqs_per_s": w.B / (ms * 1e-3),
        "step_bytes": step_bytes,
        "per_launch": launch,
        "two_call_step": {"ms_per_step": ms2, "GB/s": step_bytes / (ms2 * 1e-3) / 1e9, "per_launch": launch2,
                          "attn_decode_GB/s": w.decode_bytes() / (launch2["attn_decode"]["mean_ms"] * 1e-3) / 1e9},
        "roofline": {"bound": "hbm",
                     "kernel": "attn_decode_append (decode_partition_bf16_mfma with the fused append, "
                               "then decode_merge)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "bytes_per_launch": step_bytes, "traffic": decode_traffic()},
    }
    if not args.no_cpu_baseline:
        base, err = w.cpu_baseline(args.cpu_seqs)
        line["cpu_baseline"] = base
        line["parity_max_abs_err_vs_oracle"] = err
    del w
    torch.cuda.empty_cache()

    extra = {}
    if "padded32" in names:
        p = PaddedDecode()
        ms3, _ = time_steps(p, max(5, args.steps // 2), args.warmup)
        gbs = p.step_bytes() / (ms3 * 1e-3) / 1e9
        extra["padded32"] = {"config": p.config(), "ms_per_step": ms3, "GB/s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
                             "seqs_per_s": p.B / (ms3 * 1e-3), "step_bytes": p.step_bytes()}
        del p
        torch.cuda.empty_cache()
    if "longctx70b" in names:
        lw = LongContextFp8Decode()
        ms5, _ = time_steps(lw, max(5, args.steps // 2), args.warmup)
        gbs = lw.step_bytes() / (ms5 * 1e-3) / 1e9
        extra["longctx70b"] = {"config": lw.config(), "ms_per_step": ms5, "GB/s": gbs,
                               "frac_of_hbm_peak": gbs / HBM_PEAK_GBS, "seqs_per_s": 1 / (ms5 * 1e-3),
                               "step_bytes": lw.step_bytes()}
        del lw
        torch.cuda.empty_cache()
    if "verify8b" in names:
        vw = PagedVerify()
        msv, _ = time_steps(vw, max(10, args.steps), args.warmup)
        gbs = vw.step_bytes() / (msv * 1e-3) / 1e9
        extra["verify8b"] = {"config": vw.config(), "ms_per_step": msv, "GB/s": gbs,
                             "frac_of_hbm_peak": gbs / HBM_PEAK_GBS, "seqs_per_s": vw.B / (msv * 1e-3),
                             "step_bytes": vw.step_bytes()}
        del vw
        torch.cuda.empty_cache()
    if "prefill8k" in names:
        pf = CausalPrefill()
        # the first few dozen calls run below the steady-state rate (clocks ramp under sustained
        # matrix-core load): 50 untimed calls (~30 ms) first, then at least 20 timed
        msp, _ = time_steps(pf, max(20, args.steps), max(50, args.warmup))
        tf = pf.flops() / (msp * 1e-3) / 1e12
        extra["prefill8k"] = {"config": pf.config(), "ms_per_step": msp, "TFLOP/s": tf,
                              "frac_of_bf16_mfma_peak": tf / BF16_PEAK_TFLOPS, "flops": pf.flops(),
                              "roofline": {"bound": "mfma",
                                           "kernel": "attn_prefill (prefill_mfma_kernel, which also writes the cache)",
                                           "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                           "frac": tf / BF16_PEAK_TFLOPS, "traffic": None}}
        del pf
        torch.cuda.empty_cache()
    if "chunkprefill" in names:
        cp = ChunkedPrefill()
        msc, _ = time_steps(cp, max(20, args.steps), max(50, args.warmup))
        tf = cp.flops() / (msc * 1e-3) / 1e12
        extra["chunkprefill"] = {"config": cp.config(), "ms_per_step": msc, "TFLOP/s": tf,
                                 "frac_of_bf16_mfma_peak": tf / BF16_PEAK_TFLOPS, "flops": cp.flops(),
                                 "roofline": {"bound": "mfma", "kernel": "attn_prefill (prefill_mfma_kernel, "
                                              "cached prefix gathered through the block table)",
                                              "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                              "frac": tf / BF16_PEAK_TFLOPS, "traffic": None}}
        del cp
        torch.cuda.empty_cache()
    for key, cls_ in (("cowcopy", CowBlockCopy), ("beamreorder", BeamReorder)):
        if key not in names:
            continue
        cw = cls_()
        msc, _ = time_steps(cw, max(10, args.steps), args.warmup)
        gbs = cw.step_bytes() / (msc * 1e-3) / 1e9
        extra[key] = {"config": cw.config(), "ms_per_launch": msc, "GB/s": gbs, "bytes_per_launch": cw.step_bytes(),
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": gbs / HBM_PEAK_GBS, "traffic": None}}
        del cw
        torch.cuda.empty_cache()
    if extra:
        line["workloads"] = extra
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
