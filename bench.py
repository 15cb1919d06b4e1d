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
"workloads": the tiny fp32 sequence (16-token prefill into the cache, then a
decode step over 129 keys; latency), the padded 32-layer MHA decode (batch
8, 4096-position contiguous cache, key padding mask), the 80-layer fp8
long-context decode (batch 1, 64/8 heads, 131,073 keys per layer), the check
of 4 drafted tokens per sequence on the Llama-3-8B decode workload, the
causal 8192-token prefill that writes the paged cache, a 2048-token chunked
prefill against 6144 cached positions, a copy-on-write fan-out of 4096 paged
blocks and a contiguous beam reorder (32 rows of 4096 positions).  A plain
streaming read and copy (torch kernels) are timed as HBM context.

Timing: W untimed warm-up steps, then K steps bracketed by synchronize +
HIP events on the stream the library launches on (torch's current stream).
Each decode step reads a different replica of the cache (round-robin) so the
256 MB Infinity Cache cannot serve the previous step's bytes.  A second pass
of K steps with HIP events around every call is reported for information.
The CPU baseline is the fp64 oracle timed on the host's cores (a pool of
processes, one BLAS thread each) on the same input bytes, for the headline
step and a stated sample of the padded, fp8 and prefill workloads; each also
gives the max abs error of the GPU output against the oracle.
"""
import argparse
import hashlib
import json
import math
import os
import platform
import re
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


# Sources each workload's timed kernels are built from: files (the build
# script included: it holds the compiler flags; and the host side of the
# library, which picks the launch shapes, such as the default partition
# size), and the launch-argument structs of launch.h they compile against.
CSRC = "kv_cache_decode_attn_amd/csrc/"
BUILD_PY = "kv_cache_decode_attn_amd/build.py"
API_CPP = CSRC + "kvattn_api.cpp"
KERNEL_SOURCES = {
    "decode": (CSRC + "decode.hip", CSRC + "common.h", API_CPP, BUILD_PY, "DecodeLaunch"),
    "prefill": (CSRC + "prefill_mfma.hip", CSRC + "common.h", API_CPP, BUILD_PY, "PrefillLaunch"),
}
WORKLOAD_KERNELS = {"decode8b": "decode", "padded32": "decode", "longctx70b": "decode", "verify8b": "decode",
                    "prefill8k": "prefill", "chunkprefill": "prefill", "chunkprefill_fp8": "prefill"}


def _launch_struct(text, name):
    i = text.index("struct %s {" % name)
    return text[i:text.index("};", i) + 2]


_C_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def _code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed: a
    change to the comments does not change the kernels."""
    return " ".join(_C_COMMENT.sub(" ", text).split())


def source_sha(kind, read=None):
    """Hash of the sources the `kind` kernels ("decode", "prefill") are built
    and launched from: the code of the kernel files and of the library's host
    side (comments and layout ignored), the build script, and the launch
    struct they compile against."""
    if read is None:
        def read(rel):
            with open(os.path.join(ROOT, rel), "rb") as f:
                return f.read()
    h = hashlib.sha256()
    for item in KERNEL_SOURCES[kind]:
        if item.endswith((".hip", ".h", ".cpp")):
            h.update(_code_only(read(item).decode()).encode())
        elif item.endswith(".py"):
            h.update(read(item))
        else:
            h.update(_code_only(_launch_struct(read(CSRC + "launch.h").decode(), item)).encode())
    return h.hexdigest()


def _stored(workload):
    """The workload's entry of profiles/traffic.json (rocprofv3 figures of
    its dominant call), or None when they were measured on different kernel
    sources or are missing."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            d = json.load(f)["workloads"][workload]
    except (OSError, ValueError, KeyError):
        return None
    if d.get("source_sha256") != source_sha(WORKLOAD_KERNELS[workload]):
        return None
    return d


def traffic(workload):
    """HBM bytes per launch of the workload's dominant call measured with
    rocprofv3 FETCH_SIZE / WRITE_SIZE counters and scaled by the copy-kernel
    calibration (profiles/traffic.json), or None (see _stored)."""
    d = _stored(workload)
    return None if d is None else d.get("bytes_per_launch")


def kernel_times(workload, work, peak, unit):
    """The same call at the rocprofv3 kernel-trace averages of its kernels
    (partition pass and merge, or the prefill kernel), stored beside the
    traffic figures: {"kernel_avg_us", "us_per_call", "achieved", "frac"}
    for `work` algorithmic bytes (GB/s) or FLOPs (TFLOP/s) per call, or None
    (see _stored)."""
    d = _stored(workload)
    if d is None or not d.get("kernel_avg_us"):
        return None
    us = float(sum(d["kernel_avg_us"].values()))
    scale = 1e9 if unit == "GB/s" else 1e12
    achieved = work / (us * 1e-6) / scale
    return {"kernel_avg_us": d["kernel_avg_us"], "us_per_call": us, "achieved": achieved, "frac": achieved / peak,
            "unit": unit, "source": "rocprofv3 kernel trace, profiles/kernels_per_workload.md"}


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _stats(ms):
    a = np.asarray(ms, dtype=np.float64)
    return {"median_ms": float(np.median(a)), "min_ms": float(a.min()), "p90_ms": float(np.percentile(a, 90)),
            "mean_ms": float(a.mean())}


def _bits(t):
    """Raw storage words of a device tensor on the host (uint16 for bf16)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def cpu_workers():
    """Host processes the oracle runs on: the cores this process may use,
    at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def run_oracle(arrays, fn, units, min_seconds=3.0, prep=None):
    """Times the oracle work units `units` (oracle.pool function `fn`) on a
    pool of cpu_workers() host processes that map `arrays` from shared
    memory; the whole set is repeated until min_seconds of wall time have
    run.  `prep` = (fn, units) runs once first, untimed (input preparation).
    Returns (workers, repetitions, seconds, results of the last pass)."""
    from oracle.pool import OraclePool, SharedInputs

    workers = cpu_workers()
    with SharedInputs(arrays) as shm, OraclePool(workers, shm.specs) as pool:
        if prep is not None:
            pool.run(*prep)
        reps, total = 0, 0.0
        while True:
            dt, res = pool.run(fn, units)
            reps += 1
            total += dt
            if total >= min_seconds:
                break
    return workers, reps, total, res


def cpu_record(value, unit, workers, what, reps, seconds):
    return {"value": value, "unit": unit, "cores": workers, "kind": "oracle",
            "sample": "%s; x%d repetitions in %.1f s; fp64 numpy oracle over a pool of %d host processes "
                      "(one BLAS thread each) on %s" % (what, reps, seconds, workers, cpu_model())}


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

    def cpu_baseline(self, min_seconds=5.0):
        """The oracle on the same bytes: per (sequence, KV head), the bf16 ->
        fp64 decode of the cache and the attention of the group's G query
        heads; all 32 sequences.  Returns (record, max abs err of the GPU
        output of the last timed step vs the oracle)."""
        G = self.Hq // self.Hkv
        arrays = {"k": _bits(self.src_k), "v": _bits(self.src_v), "q": _bits(self.q)}
        units = [("", b, g, G, int(self.ctx[b]), 1.0 / math.sqrt(self.D), K.BF16, None)
                 for b in range(self.B) for g in range(self.Hkv)]
        workers, reps, dt, res = run_oracle(arrays, "decode_unit", units, min_seconds)
        want = np.zeros((self.B, self.Hq, self.D))
        for (_, b, g, G_, _, _, _, _), o in res:
            want[b, g * G:(g + 1) * G] = o
        err = float(np.abs(self.out.cpu().numpy() - want).max())
        gbs = reps * self.kv_bytes() / dt / 1e9
        rec = cpu_record(gbs, "GB/s", workers, "the whole step: 32 sequences x 8 KV heads, %d keys, %.0f MB of K/V"
                         % (int(self.ctx.sum()), self.kv_bytes() / 1e6), reps, dt)
        rec["seqs_per_s"] = reps * self.B / dt
        return rec, err


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

    def layer_bytes(self):
        return self.step_bytes() // self.L

    def cpu_baseline(self, layers=(0, 8, 16, 24), min_seconds=3.0, wid=3):
        """The oracle on a stated subset of layers (every sequence and head of
        each): the layer's K/V regenerated from their seeds (the bytes the
        cache was filled with), then per (sequence, KV head) the bf16 -> fp64
        decode and the masked attention over the 4096 cache positions.
        Returns (record, max abs err of the GPU outputs of those layers)."""
        arrays = {"mask": self.mask.cpu().numpy()}
        for l in layers:
            arrays["L%d_k" % l] = _bits(synth.normal_device(self.caches[l].k.shape, (wid, synth.T_K, l)))
            arrays["L%d_v" % l] = _bits(synth.normal_device(self.caches[l].v.shape, (wid, synth.T_V, l)))
            arrays["L%d_q" % l] = _bits(self.q[l])
        units = [("L%d_" % l, b, g, 1, self.cap, 1.0 / math.sqrt(self.D), K.BF16, "mask")
                 for l in layers for b in range(self.B) for g in range(self.H)]
        workers, reps, dt, res = run_oracle(arrays, "decode_unit", units, min_seconds)
        got = self.out.cpu().numpy()
        err = 0.0
        for (prefix, b, g, _, _, _, _, _), o in res:
            l = int(prefix[1:-1])
            err = max(err, float(np.abs(got[l, b, g] - o[0]).max()))
        gbs = reps * len(layers) * self.layer_bytes() / dt / 1e9
        rec = cpu_record(gbs, "GB/s", workers, "layers %s of 32 (every sequence and head; key mask over 4096 "
                         "positions)" % (list(layers),), reps, dt)
        rec["ms_per_step_extrapolated_to_32_layers"] = self.step_bytes() / (gbs * 1e9) * 1e3
        return rec, err

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

    def cpu_baseline(self, layers=(0, 40), min_seconds=1.0, wid=5):
        """The oracle on a stated subset of layers: the layer's bf16 K/V
        regenerated from their seeds, quantised by the oracle's own E4M3FN
        encoder with the layer's scales (input preparation, untimed), then per
        KV head the fp8 -> fp64 decode of 131,073 keys and the attention of
        its 8 query heads.  Returns (record, max abs err of the GPU outputs of
        those layers vs that quantised oracle)."""
        Hkv, ctx, D = self.Hkv, self.ctx, self.D
        arrays, prep = {}, []
        scales = self.scales.cpu().numpy()
        for l in layers:
            arrays["L%d_srck" % l] = _bits(synth.normal_device((1, Hkv, ctx, D), (wid, synth.T_K, l)))[0]
            arrays["L%d_srcv" % l] = _bits(synth.normal_device((1, Hkv, ctx, D), (wid, synth.T_V, l)))[0]
            arrays["L%d_k" % l] = np.zeros((Hkv, ctx, D), np.uint8)
            arrays["L%d_v" % l] = np.zeros((Hkv, ctx, D), np.uint8)
            arrays["L%d_ks" % l] = scales[l, 0].copy()
            arrays["L%d_vs" % l] = scales[l, 1].copy()
            arrays["L%d_q" % l] = _bits(self.q[l])
            for g in range(Hkv):
                prep.append(("L%d_srck" % l, "L%d_k" % l, g, float(scales[l, 0, g])))
                prep.append(("L%d_srcv" % l, "L%d_v" % l, g, float(scales[l, 1, g])))
        G = self.Hq // Hkv
        units = [("L%d_" % l, 0, g, G, ctx, 1.0 / math.sqrt(D), K.FP8_E4M3, None) for l in layers for g in range(Hkv)]
        workers, reps, dt, res = run_oracle(arrays, "decode_unit", units, min_seconds, prep=("quantize_unit", prep))
        got = self.out.cpu().numpy()
        err = 0.0
        for (prefix, _, g, _, _, _, _, _), o in res:
            l = int(prefix[1:-1])
            err = max(err, float(np.abs(got[l, 0, g * G:(g + 1) * G] - o).max()))
        gbs = reps * len(layers) * (self.step_bytes() // self.L) / dt / 1e9
        rec = cpu_record(gbs, "GB/s", workers, "layers %s of 80 (8 KV heads x 131,073 fp8 keys each)"
                         % (list(layers),), reps, dt)
        rec["ms_per_step_extrapolated_to_80_layers"] = self.step_bytes() / (gbs * 1e9) * 1e3
        return rec, err

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

    def cpu_baseline(self, rows=16, starts=(0, 1024, 2048, 3072, 4096, 5120, 6144, 7168, 8176), min_seconds=2.0):
        """The oracle on a stated sample of query rows: for every query head,
        `rows` consecutive rows at each start position, computed as
        oracle.attention.prefill of those rows with the keys before them as
        the attended prefix (the rows of the one-shot causal prefill); FLOPs
        4 d (t + 1) per row t.  Returns (record, max abs err of the GPU
        output rows vs the oracle)."""
        arrays = {"q": _bits(self.q)[0], "k": _bits(self.k)[0], "v": _bits(self.v)[0]}
        G = self.Hq // self.Hkv
        units = [(h, h // G, t0, rows, 1.0 / math.sqrt(self.D)) for h in range(self.Hq) for t0 in starts]
        workers, reps, dt, res = run_oracle(arrays, "prefill_rows_unit", units, min_seconds)
        got = self.out.cpu().numpy()
        err = 0.0
        for (h, _, t0, n, _), o in res:
            err = max(err, float(np.abs(got[0, h, t0:t0 + n] - o).max()))
        flops = sum(4 * self.D * (t + 1) for t0 in starts for t in range(t0, t0 + rows)) * self.Hq
        tf = reps * flops / dt / 1e12
        rec = cpu_record(tf, "TFLOP/s", workers, "%d rows at each of positions %s for all %d query heads (%.2f GFLOP)"
                         % (rows, list(starts), self.Hq, flops / 1e9), reps, dt)
        rec["ms_per_step_extrapolated"] = self.flops() / (tf * 1e12) * 1e3
        return rec, err

    def config(self):
        return {"workload": self.name, "batch": 1, "q_heads": self.Hq, "kv_heads": self.Hkv, "seq": self.N,
                "head_dim": self.D, "dtype": "bf16", "causal": True, "writes_paged_cache": True}


class ChunkedPrefill:
    """Chunked prefill against a paged cache: a 2,048-token chunk of a
    Llama-3-8B-shaped layer (32/8 heads, d 128) at positions 6,144..8,191 that
    attends the 6,144 cached positions and, causally, itself, and stores its
    rows in the cache (attn_prefill with attend_prefix).  The cache is bf16,
    or fp8 E4M3FN with per-head scales of about max|x| / 448 (the chunk's
    rows are then quantised into the cache before the attention)."""

    name = "chunked-prefill-6144-cached-2048-new-gqa"

    def __init__(self, wid=8, P=6144, n=2048, kv_dtype=K.BF16):
        self.Hq, self.Hkv, self.D, self.P, self.n = 32, 8, 128, P, n
        self.kv_dtype = kv_dtype
        std = 1.0 / math.sqrt(self.D)
        nb = synth.blocks_for(P + n)
        table, nblk = synth.block_table([nb], nb, (wid, synth.T_PERM))
        self.table = torch.from_numpy(table).to(DEV)
        ks = vs = None
        if kv_dtype == K.FP8_E4M3:
            self.name = "chunked-prefill-6144-cached-fp8-2048-new-gqa"
            sc = synth.fp8_scales(2 * self.Hkv, (wid, synth.T_SCALE), lo=0.5e-3, hi=1.0e-3)
            ks = torch.from_numpy(sc[:self.Hkv].copy()).to(DEV)
            vs = torch.from_numpy(sc[self.Hkv:].copy()).to(DEV)
        self.cache = K.KVCache.paged(nblk, self.Hkv, self.D, kv_dtype, DEV, ks, vs)
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
                "new": self.n, "head_dim": self.D, "dtype": "bf16",
                "kv_dtype": "fp8_e4m3" if self.kv_dtype == K.FP8_E4M3 else "bf16", "causal": True,
                "writes_paged_cache": True}


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


class TinySequence:
    """The tiny workload: 1 layer, batch 1, 4 query / 4 KV heads, head_dim
    64, fp32, contiguous cache of 256 positions.  A causal prefill of 16
    tokens fills the cache (attn_prefill with the cache write), positions
    16..127 are appended, and the decode step stores token 128 and attends
    the 129 keys (attn_decode_append).  Launch-bound: reported as latency
    per call."""

    name = "tiny-fp32-prefill16-decode129"

    def __init__(self, wid=1):
        self.H, self.D, self.cap, self.n_pre, self.cached = 4, 64, 256, 16, 128
        n = self.cached + 1
        self.q = synth.normal((1, self.H, n, self.D), (wid, synth.T_Q), torch.float32).to(DEV)
        self.k = synth.normal((1, self.H, n, self.D), (wid, synth.T_K), torch.float32).to(DEV)
        self.v = synth.normal((1, self.H, n, self.D), (wid, synth.T_V), torch.float32).to(DEV)
        self.cache = K.KVCache.contiguous(1, self.H, self.cap, self.D, K.F32, DEV)
        self.zero = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.qp = self.q[:, :, :self.n_pre].contiguous()
        self.kp = self.k[:, :, :self.n_pre].contiguous()
        self.vp = self.v[:, :, :self.n_pre].contiguous()
        self.out_pre = torch.empty((1, self.H, self.n_pre, self.D), dtype=torch.float32, device=DEV)
        # the prefill once, then positions 16..127
        K.attn_prefill(self.qp, self.kp, self.vp, cache=self.cache, positions=self.zero, out=self.out_pre)
        K.kv_append(self.cache, self.k[:, :, self.n_pre:self.cached].contiguous(),
                    self.v[:, :, self.n_pre:self.cached].contiguous(),
                    torch.full((1,), self.n_pre, dtype=torch.int32, device=DEV))
        self.qd = self.q[:, :, self.cached].contiguous()
        self.kd = self.k[:, :, self.cached].contiguous()
        self.vd = self.v[:, :, self.cached].contiguous()
        self.seq_lens = torch.full((1,), self.cached + 1, dtype=torch.int32, device=DEV)
        self.out = torch.empty((1, self.H, self.D), dtype=torch.float32, device=DEV)
        self.ws = K.decode_workspace(self.cache, 1, self.H, self.cap)
        self.phase = "decode"
        torch.cuda.synchronize()

    def step(self, i, ev=None):
        if self.phase == "prefill":  # re-writes positions 0..15 with the same rows
            K.attn_prefill(self.qp, self.kp, self.vp, cache=self.cache, positions=self.zero, out=self.out_pre)
        else:  # re-writes position 128 with the same row
            K.attn_decode_append(self.cache, self.qd, self.kd, self.vd, self.seq_lens, self.cap, out=self.out,
                                 workspace=self.ws)

    def parity(self):
        """Max abs error of the decode output and of the prefill output vs the
        oracle (fp64 on the same fp32 inputs)."""
        from oracle import attention as OA

        q, k, v = (t.cpu().numpy().astype(np.float64) for t in (self.q, self.k, self.v))
        scale = 1.0 / math.sqrt(self.D)
        dec = OA.decode(q[:, :, self.cached], [k[0]], [v[0]], [self.cached + 1], scale)
        pre = OA.prefill(q[:, :, :self.n_pre], k[:, :, :self.n_pre], v[:, :, :self.n_pre], [0], [self.n_pre], scale)
        return (float(np.abs(self.out.cpu().numpy() - dec).max()),
                float(np.abs(self.out_pre.cpu().numpy() - pre).max()))

    def config(self):
        return {"workload": self.name, "layers": 1, "batch": 1, "q_heads": self.H, "kv_heads": self.H,
                "head_dim": self.D, "dtype": "f32", "capacity": self.cap, "prefill_tokens": self.n_pre,
                "decode_keys": self.cached + 1}


class StreamRead:
    """Context for the HBM rooflines: one pass over 4 GiB with the library's
    streaming-read helper (kvattn_stream_read: 16-byte non-temporal loads,
    whole 1 KB per wave instruction), the same read as torch.sum, and a
    plain copy (2 GiB to 2 GiB, torch copy_) on this GPU.  Not a workload of
    the library; the bars stay relative to 8 TB/s."""

    name = "plain-stream-read-and-copy"

    def __init__(self):
        self.x = torch.ones(1 << 30, dtype=torch.float32, device=DEV)
        self.a = torch.ones(1 << 29, dtype=torch.float32, device=DEV)
        self.b = torch.empty_like(self.a)
        self.sink = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.phase = "read"
        torch.cuda.synchronize()

    def step(self, i, ev=None):
        if self.phase == "stream_read":
            K.stream_read(self.x, self.sink)
        elif self.phase == "read":
            torch.sum(self.x)
        else:
            self.b.copy_(self.a)

    def bytes(self):
        return self.x.numel() * 4 if self.phase in ("read", "stream_read") else 2 * self.a.numel() * 4


def warm_clocks(w, seconds=0.5):
    """Runs the workload's step untimed for about `seconds` of wall time: the
    GPU's clocks ramp for a while after idle host work (the oracle timing,
    input set-up), and a few warm-up steps of a 1-5 ms step do not cover it."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        w.step(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


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


LEGS = ("tiny", "padded32", "longctx70b", "verify8b", "prefill8k", "chunkprefill", "chunkprefill_fp8", "cowcopy",
        "beamreorder", "stream")


def run_leg(name, args, cpu):
    """Times one workload besides the headline; returns its record."""
    if name == "tiny":
        t = TinySequence()
        rec = {"config": t.config()}
        for phase, reps in (("prefill", 200), ("decode", 200)):
            t.phase = phase
            warm_clocks(t, 0.1)
            msx, _ = time_steps(t, reps, 20)
            rec["%s_us_per_call" % phase] = msx * 1e3
        rec["sequence_us"] = rec["prefill_us_per_call"] + rec["decode_us_per_call"]
        rec["note"] = "launch-bound: latency only (the 112 positions appended in between are set-up, not timed)"
        if cpu:
            rec["parity_max_abs_err_vs_oracle"], rec["prefill_parity_max_abs_err_vs_oracle"] = t.parity()
        return rec
    if name == "padded32":
        p = PaddedDecode()
        warm_clocks(p)
        ms3, _ = time_steps(p, max(5, args.steps // 2), args.warmup)
        gbs = p.step_bytes() / (ms3 * 1e-3) / 1e9
        rec = {"config": p.config(), "ms_per_step": ms3, "GB/s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
               "seqs_per_s": p.B / (ms3 * 1e-3), "step_bytes": p.step_bytes(),
               "roofline": {"bound": "hbm", "kernel": "attn_decode_append per layer (decode_partition vector pass "
                            "with the key mask and fused append, then decode_merge)",
                            "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                            "bytes_per_launch": p.layer_bytes(), "traffic": traffic("padded32"),
                            "rocprof": kernel_times("padded32", p.layer_bytes(), HBM_PEAK_GBS, "GB/s")}}
        if cpu:
            rec["cpu_baseline"], rec["parity_max_abs_err_vs_oracle"] = p.cpu_baseline()
        return rec
    if name == "longctx70b":
        lw = LongContextFp8Decode()
        warm_clocks(lw)
        ms5, _ = time_steps(lw, max(5, args.steps // 2), args.warmup)
        gbs = lw.step_bytes() / (ms5 * 1e-3) / 1e9
        rec = {"config": lw.config(), "ms_per_step": ms5, "GB/s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
               "seqs_per_s": 1 / (ms5 * 1e-3), "step_bytes": lw.step_bytes(),
               "roofline": {"bound": "hbm", "kernel": "attn_decode_append per layer (decode_partition_fp8_mfma "
                            "with the fused append, then decode_merge)",
                            "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                            "bytes_per_launch": lw.step_bytes() // lw.L, "traffic": traffic("longctx70b"),
                            "rocprof": kernel_times("longctx70b", lw.step_bytes() // lw.L, HBM_PEAK_GBS, "GB/s")}}
        if cpu:
            rec["cpu_baseline"], rec["parity_max_abs_err_vs_quantised_oracle"] = lw.cpu_baseline()
        return rec
    if name == "verify8b":
        vw = PagedVerify()
        warm_clocks(vw)
        msv, _ = time_steps(vw, max(10, args.steps), args.warmup)
        gbs = vw.step_bytes() / (msv * 1e-3) / 1e9
        return {"config": vw.config(), "ms_per_step": msv, "GB/s": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
                "seqs_per_s": vw.B / (msv * 1e-3), "step_bytes": vw.step_bytes(),
                "roofline": {"bound": "hbm", "kernel": "attn_decode_append with 4 queries per sequence "
                             "(decode_partition_bf16_online with the fused append, then decode_merge)",
                             "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                             "bytes_per_launch": vw.step_bytes(), "traffic": traffic("verify8b"),
                             "rocprof": kernel_times("verify8b", vw.step_bytes(), HBM_PEAK_GBS, "GB/s")}}
    if name == "prefill8k":
        pf = CausalPrefill()
        # the first calls run below the steady-state rate (clocks ramp under sustained
        # matrix-core load): a second of untimed calls first, then at least 20 timed
        warm_clocks(pf, 1.0)
        msp, _ = time_steps(pf, max(20, args.steps), args.warmup)
        tf = pf.flops() / (msp * 1e-3) / 1e12
        rec = {"config": pf.config(), "ms_per_step": msp, "TFLOP/s": tf, "frac_of_bf16_mfma_peak": tf / BF16_PEAK_TFLOPS,
               "flops": pf.flops(),
               "roofline": {"bound": "mfma", "kernel": "attn_prefill (prefill_mfma_kernel, which also writes the cache)",
                            "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                            "traffic": traffic("prefill8k"),
                            "rocprof": kernel_times("prefill8k", pf.flops(), BF16_PEAK_TFLOPS, "TFLOP/s")}}
        if cpu:
            rec["cpu_baseline"], rec["parity_max_abs_err_vs_oracle"] = pf.cpu_baseline()
        return rec
    if name in ("chunkprefill", "chunkprefill_fp8"):
        cp = ChunkedPrefill(kv_dtype=K.FP8_E4M3 if name == "chunkprefill_fp8" else K.BF16)
        warm_clocks(cp, 1.0)
        msc, _ = time_steps(cp, max(20, args.steps), args.warmup)
        tf = cp.flops() / (msc * 1e-3) / 1e12
        return {"config": cp.config(), "ms_per_step": msc, "TFLOP/s": tf, "frac_of_bf16_mfma_peak": tf / BF16_PEAK_TFLOPS,
                "flops": cp.flops(),
                "roofline": {"bound": "mfma", "kernel": "attn_prefill (prefill_mfma_kernel, cached prefix gathered "
                             "through the block table" + (
                                 "; fp8 codes expanded to bf16 in LDS, after kv_append_kernel quantises the chunk "
                                 "into the cache)" if cp.kv_dtype == K.FP8_E4M3 else ")"),
                             "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": tf / BF16_PEAK_TFLOPS, "traffic": traffic(name)}}
    if name in ("cowcopy", "beamreorder"):
        cw = CowBlockCopy() if name == "cowcopy" else BeamReorder()
        warm_clocks(cw)
        msc, _ = time_steps(cw, max(10, args.steps), args.warmup)
        gbs = cw.step_bytes() / (msc * 1e-3) / 1e9
        return {"config": cw.config(), "ms_per_launch": msc, "GB/s": gbs, "bytes_per_launch": cw.step_bytes(),
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": gbs / HBM_PEAK_GBS, "traffic": None}}
    if name == "stream":
        sr = StreamRead()
        rec = {}
        for phase in ("stream_read", "read", "copy"):
            sr.phase = phase
            warm_clocks(sr, 0.3)
            msx, _ = time_steps(sr, 10, 3)
            rec["%s_GB/s" % phase] = sr.bytes() / (msx * 1e-3) / 1e9
        rec["kernels"] = ("stream_read: kvattn_stream_read over 4 GiB (one pass, 16-byte non-temporal loads); "
                          "read: torch.sum over the same 4 GiB fp32; copy: torch copy_ of 2 GiB fp32 (4 GiB moved)")
        return rec
    raise ValueError("unknown workload %r" % name)


def leg_in_child(name, args):
    """Runs one leg in a fresh process (`bench.py --leg NAME`): each workload
    then starts from an empty device allocator, as a serving process that
    sizes its cache at start-up does, instead of inheriting the address
    space the previous legs fragmented (that history alone moved the fp8
    long-context step by 5%)."""
    import subprocess

    cmd = [sys.executable, os.path.abspath(__file__), "--leg", name, "--steps", str(args.steps),
           "--warmup", str(args.warmup)] + (["--no-cpu-baseline"] if args.no_cpu_baseline else [])
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    if r.returncode != 0 or not lines:
        sys.stderr.write(r.stderr[-4000:])
        return {"error": "leg %s exited with status %d" % (name, r.returncode)}
    return json.loads(lines[-1])


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workloads", default=",".join(LEGS),
                    help="comma list of workloads timed besides the headline (decode8b, always run), each in a "
                         "process of its own: " + ", ".join(LEGS))
    ap.add_argument("--leg", default=None, help="run only this workload, in this process, and print its record")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip every oracle timing and parity sample")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: the library is a single-GPU kernel library and this build runs on a "
              "one-GPU box (how the path would shard is described in the design notes).", file=sys.stderr)
        return 2
    cpu = not args.no_cpu_baseline
    if args.leg:
        torch.cuda.set_device(0)
        print(json.dumps(run_leg(args.leg, args, cpu)))
        return 0
    names = [x for x in args.workloads.split(",") if x]
    torch.cuda.set_device(0)
    w = PagedDecode()
    warm_clocks(w)
    # the same step as two calls (kv_append, attn_decode), for reference
    w.fused = False
    ms2, _ = time_steps(w, args.steps, args.warmup)
    _, launch2 = time_steps(w, args.steps, args.warmup, per_launch=True)
    w.fused = True
    # `value`: K steps with nothing else in the timed region (HIP events on
    # the launch stream around the whole region); then a second pass with HIP
    # events around every call, reported for information (the event records
    # themselves add a few microseconds per call)
    ms, _ = time_steps(w, args.steps, args.warmup)
    _, launch = time_steps(w, args.steps, args.warmup, per_launch=True)
    step_bytes = w.step_bytes()
    achieved = step_bytes / (ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": achieved,
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
        "frac_of_hbm_peak": achieved / HBM_PEAK_GBS,
        "seqs_per_s": w.B / (ms * 1e-3),
        "step_bytes": step_bytes,
        "per_launch": launch,
        "two_call_step": {"ms_per_step": ms2, "GB/s": step_bytes / (ms2 * 1e-3) / 1e9, "per_launch": launch2,
                          "attn_decode_GB/s": w.decode_bytes() / (launch2["attn_decode"]["mean_ms"] * 1e-3) / 1e9},
        # the dominant launch pair is the whole timed step (one attn_decode_append call:
        # the partition pass, then the merge); achieved = algorithmic bytes / mean step time
        "roofline": {"bound": "hbm",
                     "kernel": "attn_decode_append (decode_partition_bf16_mfma with the fused append, "
                               "then decode_merge)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "bytes_per_launch": step_bytes, "traffic": traffic("decode8b"),
                     "rocprof": kernel_times("decode8b", step_bytes, HBM_PEAK_GBS, "GB/s")},
    }
    if cpu:
        base, err = w.cpu_baseline()
        line["cpu_baseline"] = base
        line["parity_max_abs_err_vs_oracle"] = err
    del w
    torch.cuda.empty_cache()

    extra = {name: leg_in_child(name, args) for name in names if name != "stream"}
    if "stream" in names:
        line["hbm_context"] = leg_in_child("stream", args)
    if extra:
        line["workloads"] = extra
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
