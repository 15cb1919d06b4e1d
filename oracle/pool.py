"""Run oracle functions over a pool of host processes, to time the oracle on
the host's cores (the CPU baseline the benchmark reports).

TEST INFRASTRUCTURE ONLY, like the rest of this package.  The pool adds no
arithmetic of its own: each work unit is one call of an unmodified oracle
function (attention.decode or attention.prefill on one sequence and one KV
head's query group, or on a chunk of query rows) on inputs read from shared
memory.  Workers are fresh interpreters (the "spawn" start method): they
import numpy and this package only, and each runs its BLAS on one thread.

    with SharedInputs({"k": k_bits, ...}) as shm:
        with OraclePool(workers, shm.specs) as pool:
            seconds, results = pool.run("decode_unit", units)
"""
import multiprocessing as mp
import time
from multiprocessing import shared_memory

import numpy as np

from . import attention as A
from . import cache as C

_ARRAYS = {}
_HANDLES = []


class SharedInputs:
    """numpy arrays copied once into shared memory; `specs` lets a worker
    map them again by name."""

    def __init__(self, arrays):
        self._blocks = []
        self.specs = {}
        try:
            for name, a in arrays.items():
                a = np.ascontiguousarray(a)
                blk = shared_memory.SharedMemory(create=True, size=max(a.nbytes, 1))
                self._blocks.append(blk)
                np.ndarray(a.shape, a.dtype, buffer=blk.buf)[...] = a
                self.specs[name] = (blk.name, a.shape, a.dtype.str)
        except BaseException:
            self.close()
            raise

    def close(self):
        for blk in self._blocks:
            blk.close()
            blk.unlink()
        self._blocks = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _init(specs):
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)
    for name, (shm_name, shape, dtype) in specs.items():
        h = shared_memory.SharedMemory(name=shm_name)
        _HANDLES.append(h)
        _ARRAYS[name] = np.ndarray(shape, np.dtype(dtype), buffer=h.buf)


def _ready(_):
    return len(_ARRAYS)


class OraclePool:
    """`workers` spawned processes with the shared inputs mapped."""

    def __init__(self, workers, specs):
        self.workers = int(workers)
        self._pool = mp.get_context("spawn").Pool(self.workers, initializer=_init, initargs=(specs,))
        # every worker started and mapped before anything is timed
        self._pool.map(_ready, range(4 * self.workers), chunksize=1)

    def run(self, fn_name, units):
        """Runs fn_name(unit) for every unit; returns (wall seconds, results)."""
        fn = globals()[fn_name]
        t0 = time.perf_counter()
        res = self._pool.map(fn, units, chunksize=1)
        return time.perf_counter() - t0, res

    def close(self):
        self._pool.close()
        self._pool.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self._pool.terminate()
        self._pool.join()


# ------------------------------------------------------------ work units ---
# Each returns (unit, result array); the inputs are raw storage words
# (uint16 bf16 bits, uint8 E4M3FN codes) decoded to fp64 inside the unit, so
# the decode of the cache is part of the timed work.

def decode_unit(u):
    """One sequence b and KV head g of a decode step: attention.decode for the
    G query heads of the group over the first ctx keys.
    u = (prefix, b, g, G, ctx, scale, dtype, mask_name or None), reading
    arrays prefix + "k" / "v" [B, Hkv, width, d] (or for a single-sequence
    fp8 layer [Hkv, width, d]), prefix + "q" [B, Hq, d] (bf16 bits),
    and for fp8 prefix + "ks" / "vs" [Hkv] fp32 scales."""
    prefix, b, g, G, ctx, scale, dtype, mask_name = u
    K = _ARRAYS[prefix + "k"]
    V = _ARRAYS[prefix + "v"]
    if K.ndim == 3:
        kr, vr = K[g, :ctx], V[g, :ctx]
    else:
        kr, vr = K[b, g, :ctx], V[b, g, :ctx]
    ks = vs = None
    if dtype == C.FP8_E4M3:
        ks, vs = float(_ARRAYS[prefix + "ks"][g]), float(_ARRAYS[prefix + "vs"][g])
    kf = C.to_f64(kr, dtype, ks)[None]
    vf = C.to_f64(vr, dtype, vs)[None]
    qf = C.to_f64(_ARRAYS[prefix + "q"][b, g * G:(g + 1) * G], C.BF16)[None]
    mask = None if mask_name is None else _ARRAYS[mask_name][b:b + 1]
    out = A.decode(qf, [kf], [vf], [ctx], scale, key_mask=mask)
    return u, out[0]


def prefill_rows_unit(u):
    """Rows t0 .. t0 + n - 1 of query head h of a one-sequence causal
    prefill at position 0: attention.prefill of those rows with the keys
    below t0 given as the attended prefix (the same rows as the one-shot
    prefill computes).  u = (h, g, t0, n, scale); arrays "q" [Hq, N, d],
    "k" / "v" [Hkv, N, d] (bf16 bits)."""
    h, g, t0, n, scale = u
    q = C.to_f64(_ARRAYS["q"][h, t0:t0 + n], C.BF16)[None, None]
    k = C.to_f64(_ARRAYS["k"][g, :t0 + n], C.BF16)
    v = C.to_f64(_ARRAYS["v"][g, :t0 + n], C.BF16)
    out = A.prefill(q, k[None, None, t0:], v[None, None, t0:], [t0], [n], scale,
                    prefix_k=[k[None, :t0]], prefix_v=[v[None, :t0]], attend_prefix=True)
    return u, out[0, 0]


def quantize_unit(u):
    """fp8 cache contents of one KV head: the oracle's E4M3FN encoder on the
    bf16 rows, written into the shared array `dst` (input preparation for
    the fp8 decode units, not timed).  u = (src, dst, g, scale)."""
    src, dst, g, scale = u
    _ARRAYS[dst][g] = C.encode_rows(_ARRAYS[src][g], C.BF16, C.FP8_E4M3, scale)
    return u, None
