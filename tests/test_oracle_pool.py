"""The host-process pool that times the oracle for the benchmark's CPU
baseline: each work unit must return exactly what the oracle function it
wraps returns when called directly on the same inputs (the pool adds no
arithmetic), and the shared-memory inputs must be cleaned up."""
import math
import os

import numpy as np

from oracle import attention as A
from oracle import cache as C
from oracle import pool as P


def _bf16_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def test_pool_units_equal_direct_oracle_calls():
    rng = np.random.default_rng(90)
    B, Hq, Hkv, W, d = 3, 8, 2, 40, 16
    G = Hq // Hkv
    k, v, q = _bf16_bits(rng, (B, Hkv, W, d)), _bf16_bits(rng, (B, Hkv, W, d)), _bf16_bits(rng, (B, Hq, d))
    lens = [40, 17, 1]
    mask = (rng.random((B, W)) < 0.7).astype(np.uint8)
    # prefill inputs (one sequence): q [Hq, N, d], k/v [Hkv, N, d]
    N = 24
    pq, pk, pv = _bf16_bits(rng, (Hq, N, d)), _bf16_bits(rng, (Hkv, N, d)), _bf16_bits(rng, (Hkv, N, d))
    src = _bf16_bits(rng, (Hkv, 33, d))
    arrays = {"k": k, "v": v, "q": q, "mask": mask, "pq": pq, "pk": pk, "pv": pv,
              "src": src, "codes": np.zeros((Hkv, 33, d), np.uint8)}
    scale = 1 / math.sqrt(d)
    with P.SharedInputs(arrays) as shm:
        names = [spec[0] for spec in shm.specs.values()]
        with P.OraclePool(2, shm.specs) as pool:
            units = [("", b, g, G, lens[b], scale, C.BF16, m) for b in range(B) for g in range(Hkv)
                     for m in (None, "mask")]
            _, res = pool.run("decode_unit", units)
            for (pre, b, g, G_, ctx, sc, dt, m), out in res:
                want = A.decode(C.to_f64(q, C.BF16)[b:b + 1, g * G:(g + 1) * G],
                                [C.to_f64(k, C.BF16)[b, g:g + 1]], [C.to_f64(v, C.BF16)[b, g:g + 1]], [ctx], scale,
                                key_mask=None if m is None else mask[b:b + 1])
                np.testing.assert_array_equal(out, want[0])
            # prefill rows through the pool's prefill arrays (named q/k/v there)
            with P.SharedInputs({"q": pq, "k": pk, "v": pv}) as shm2, P.OraclePool(2, shm2.specs) as pool2:
                _, rows = pool2.run("prefill_rows_unit", [(h, h // G, t0, 5, scale) for h in (0, 5)
                                                          for t0 in (0, 7, 19)])
            full = A.prefill(C.to_f64(pq, C.BF16)[None], C.to_f64(pk, C.BF16)[None], C.to_f64(pv, C.BF16)[None],
                             [0], [N], scale)
            for (h, g, t0, n, _), out in rows:
                np.testing.assert_allclose(out, full[0, h, t0:t0 + n], rtol=1e-12, atol=1e-13)
            pool.run("quantize_unit", [("src", "codes", g, 0.75) for g in range(Hkv)])
            got = np.ndarray(src.shape, np.uint8, buffer=shm._blocks[-1].buf).copy()
            np.testing.assert_array_equal(got, C.encode_rows(src, C.BF16, C.FP8_E4M3, 0.75))
    for n in names:
        assert not os.path.exists("/dev/shm/" + n.lstrip("/"))
