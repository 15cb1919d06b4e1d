"""Storage formats -> exact fp64 values, and the OCP E4M3FN encoder.

Test infrastructure (see the package docstring); fp64 throughout.

The pages only say the cache may be stored as "FP8" to halve its bytes
([P1] "Use it" vLLM example with an fp8 KV-cache dtype; [P2] section
"(1) FP8 quantization: 50% memory saving").  The concrete format is the OCP
8-bit floating point E4M3 variant ("E4M3FN"): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest
finite magnitude 448.  Reading taken: values are quantised from an fp32
quotient x / scale with round-to-nearest-even and saturation to +-448; a
NaN quotient becomes 0x7F; the sign of the quotient is kept (so tiny
negatives give 0x80, negative zero).
"""
import numpy as np


def f32_to_f64(a):
    """fp32 array -> fp64 (exact)."""
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> fp64 (exact).

    A bfloat16 is the upper half of an IEEE fp32 word, so the value is the
    fp32 whose high 16 bits are the pattern and whose low 16 bits are zero.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e4m3_decode(codes):
    """OCP E4M3FN byte codes (uint8) -> fp64 values (exact; NaN for 0x7F/0xFF).

    value = (-1)^s * 2^(e-7) * (1 + m/8)   for exponent field e in 1..15
          = (-1)^s * 2^(-6)  * (m/8)       for e == 0 (subnormals, zero)
    and S.1111.111 is NaN (no infinities in this variant).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0,
                   np.ldexp(m / 8.0, -6),
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = np.where(s == 1, -mag, mag)
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return val.astype(np.float64)


# The 127 finite non-negative magnitudes, in code order (code 0..126); the
# format is monotonic in its code, so this list is sorted ascending.
_E4M3_POS = e4m3_decode(np.arange(0, 127, dtype=np.uint8))
E4M3_MAX = float(_E4M3_POS[-1])  # 448.0


def e4m3_encode_quotient(q):
    """Round fp32 quotients to E4M3FN codes: nearest, ties to even, saturating.

    q must already be the fp32 quotient x / scale.  For each |q| find the two
    neighbouring representable magnitudes and keep the nearer one; on an
    exact tie keep the one whose code (hence mantissa) is even.  |q| >= 448
    (including infinity) saturates to 448 (code 0x7E).  NaN -> 0x7F.  The
    sign bit of the result is the sign bit of q.
    """
    q = np.asarray(q, dtype=np.float32)
    a = np.abs(q).astype(np.float64)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # lo = largest code whose magnitude is <= a; hi = lo + 1 (clipped)
    lo = np.searchsorted(_E4M3_POS, a, side="right") - 1
    hi = np.minimum(lo + 1, len(_E4M3_POS) - 1)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1) & (hi != lo))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(q), code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code).astype(np.uint8)
    return code


def e4m3_quantize(x, scale):
    """x (fp32 values) / scale (fp32) in IEEE fp32, then e4m3_encode_quotient."""
    xq = np.asarray(x, dtype=np.float32) / np.float32(scale)
    return e4m3_encode_quotient(xq.astype(np.float32))
