"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad host arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from kv_cache_decode_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvattn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvattn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_exports():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.kvattn_version().decode().startswith("kvattn")


def test_status_strings():
    L = _lib.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.kvattn_status_string(code).decode() != "unknown status"


def test_cache_bytes_closed_forms_through_the_abi():
    L = _lib.lib()
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "kv_cache_bytes.txt")):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(line.split())
    for r in rows:
        assert L.kvattn_cache_bytes(*[int(x) for x in r[:6]]) == int(r[6]), r[7]
    assert L.kvattn_cache_bytes(1 << 40, 1 << 40, 2, 1, 1, 1) == 0  # overflow


def test_workspace_and_partition_sizing():
    L = _lib.lib()
    t = L.kvattn_decode_default_part_tokens(_lib.BF16, 32, 32, 8, 8193)
    assert t % 64 == 0 and 64 <= t <= 8192
    parts = (8193 + t - 1) // t
    assert L.kvattn_decode_workspace_bytes(_lib.BF16, 32, 32, 8, 128, 8193, t) == 32 * 32 * parts * 130 * 4
    assert L.kvattn_decode_workspace_bytes(_lib.BF16, 32, 32, 8, 128, 100, 512) == 0  # single partition
    assert L.kvattn_decode_default_part_tokens(_lib.BF16, 1, 3, 2, 100) == 0          # bad group
    assert L.kvattn_decode_default_part_tokens(9, 1, 8, 8, 100) == 0                  # bad dtype
    # the fp8 matrix-core pass: one workgroup per compute unit (256), keys
    # split as evenly as 64-key steps allow
    assert L.kvattn_decode_default_part_tokens(_lib.FP8_E4M3, 1, 64, 8, 131073) == 4160   # 8 x 32 partitions
    assert L.kvattn_decode_default_part_tokens(_lib.FP8_E4M3, 4, 32, 8, 32768) == 4096    # 32 x 8
    assert L.kvattn_decode_default_part_tokens(_lib.FP8_E4M3, 1, 64, 8, 1000) == 256      # floor
    assert L.kvattn_decode_default_part_tokens(_lib.FP8_E4M3, 64, 512, 64, 9000) == 8192  # ceiling
    for B, Hkv, n in [(1, 8, 131073), (2, 8, 100000), (3, 4, 77777), (1, 1, 50000)]:
        t = L.kvattn_decode_default_part_tokens(_lib.FP8_E4M3, B, 8 * Hkv, Hkv, n)
        assert t % 64 == 0 and B * Hkv * -(-n // t) <= 256 or t == 8192, (B, Hkv, n, t)


FAKE = 0x10000  # an aligned non-null address; host validation never dereferences it


def _cache(dtype=_lib.BF16, layout=_lib.PAGED, head_dim=128, hkv=8, num_blocks=64, capacity=256, rows=4):
    c = _lib.KvattnCache()
    c.dtype, c.layout, c.num_kv_heads, c.head_dim = dtype, layout, hkv, head_dim
    c.capacity, c.num_rows, c.num_blocks = capacity, rows, num_blocks
    c.k, c.v = FAKE, FAKE + 0x100000
    return c


def _decode(c, **kw):
    a = dict(batch=4, hq=32, q=FAKE, qd=_lib.BF16, lens=FAKE, maxlen=1000, table=FAKE, mb=64, mask=None,
             stride=0, scale=0.1, out=FAKE, ws=None, wsb=0, part=0)
    a.update(kw)
    L = _lib.lib()
    return L.kvattn_attn_decode(ctypes.byref(c) if c is not None else None, a["batch"], a["hq"], a["q"], a["qd"],
                                a["lens"], a["maxlen"], a["table"], a["mb"], a["mask"], a["stride"], a["scale"],
                                a["out"], a["ws"], a["wsb"], a["part"], None)


@pytest.mark.parametrize("kw,cache_kw,want", [
    ({}, {"head_dim": 96}, _lib.EUNSUPPORTED),
    ({"hq": 24}, {}, _lib.EUNSUPPORTED),              # group 3
    ({"qd": _lib.F32}, {}, _lib.EUNSUPPORTED),        # bf16 cache needs bf16 q
    ({"q": FAKE + 4}, {}, _lib.EINVAL),               # misaligned
    ({"lens": None}, {}, _lib.EINVAL),
    ({"table": None}, {}, _lib.EINVAL),               # paged without a table
    ({"part": 100}, {}, _lib.EINVAL),                 # not a multiple of 64
    ({"part": 4096}, {}, _lib.EINVAL),                # 4096 * group 4 > 8192 scores
    ({"mask": FAKE, "stride": 10}, {}, _lib.EINVAL),  # stride < max_seq_len
    ({}, {}, _lib.EWORKSPACE),                        # several partitions, no workspace
    ({}, {"dtype": 7}, _lib.EINVAL),
    ({}, {"layout": 5}, _lib.EINVAL),
    ({}, {"layout": _lib.CONTIGUOUS, "capacity": 100}, _lib.EINVAL),  # not a multiple of 16
    ({"batch": 8}, {"layout": _lib.CONTIGUOUS, "rows": 4}, _lib.EINVAL),
    ({}, {"dtype": _lib.FP8_E4M3}, _lib.EINVAL),      # fp8 without scales
])
def test_decode_host_errors(kw, cache_kw, want):
    assert _decode(_cache(**cache_kw), **kw) == want
    assert _lib.lib().kvattn_last_error().decode() != ""


def test_decode_null_cache():
    assert _decode(None) == _lib.EINVAL


def test_decode_workspace_too_small():
    assert _decode(_cache(), ws=FAKE, wsb=64) == _lib.EWORKSPACE


def test_append_host_errors():
    L = _lib.lib()
    c = _cache()
    args = [ctypes.byref(c), 4, 1, FAKE, FAKE, _lib.BF16, FAKE, None, FAKE, 64, None]
    bad = list(args)
    bad[5] = _lib.F32  # f32 into a bf16 cache
    assert L.kvattn_kv_append(*bad) == _lib.EUNSUPPORTED
    bad = list(args)
    bad[6] = None  # positions
    assert L.kvattn_kv_append(*bad) == _lib.EINVAL
    bad = list(args)
    bad[3] = FAKE + 8
    assert L.kvattn_kv_append(*bad) == _lib.EINVAL
    zero = list(args)
    zero[2] = 0  # n_new == 0: a no-op that never launches
    assert L.kvattn_kv_append(*zero) == _lib.OK


def test_prefill_host_errors():
    L = _lib.lib()

    def call(cache=None, hq=32, hkv=8, d=128, n=16, dtype=_lib.BF16, attend_prefix=0, q=FAKE):
        return L.kvattn_attn_prefill(ctypes.byref(cache) if cache is not None else None, 1, hq, hkv, d, n, q, FAKE,
                                     FAKE, dtype, None, None, None, 0, None, 0, 1, attend_prefix, 0.1, FAKE, None)

    assert call(d=80) == _lib.EUNSUPPORTED
    assert call(hq=12) == _lib.EUNSUPPORTED
    assert call(dtype=_lib.FP8_E4M3) == _lib.EINVAL
    assert call(attend_prefix=1) == _lib.EINVAL
    assert call(q=FAKE + 2) == _lib.EINVAL
    assert call(cache=_cache(hkv=4)) == _lib.EINVAL  # shape mismatch
    assert call(n=0) == _lib.OK


def test_decode_append_host_errors():
    L = _lib.lib()

    def call(c=None, k_new=FAKE, v_new=FAKE, in_dtype=_lib.BF16, batch=4, ws=None, wsb=0):
        c = c if c is not None else _cache()
        return L.kvattn_attn_decode_append(ctypes.byref(c), batch, 32, FAKE, _lib.BF16, k_new, v_new, in_dtype, FAKE,
                                           100, FAKE, 64, None, 0, 0.1, FAKE, ws, wsb, 512, None)

    assert call(in_dtype=_lib.F32) == _lib.EUNSUPPORTED    # f32 rows into a bf16 cache
    assert call(in_dtype=_lib.FP8_E4M3) == _lib.EINVAL     # rows must be f32 or bf16
    assert call(in_dtype=-1) == _lib.EINVAL
    assert call(k_new=None) == _lib.EINVAL
    assert call(v_new=FAKE + 4) == _lib.EINVAL             # misaligned
    assert call(c=_cache(head_dim=96)) == _lib.EUNSUPPORTED
    assert call(batch=0) == _lib.OK                        # nothing to do, nothing launched
    assert call(batch=0, k_new=None) == _lib.OK
    assert _lib.lib().kvattn_last_error().decode() == ""


def test_reorder_and_copy_host_errors():
    L = _lib.lib()
    P = FAKE

    def rows(n=4, src_rows=4, mb=8, perm=P, st=P, sl=P, dt=FAKE + 0x100000, dl=FAKE + 0x200000):
        return L.kvattn_reorder_rows(n, perm, src_rows, st, sl, mb, dt, dl, None)

    assert rows(n=70000) == _lib.EINVAL
    assert rows(mb=0) == _lib.EINVAL
    assert rows(perm=None) == _lib.EINVAL
    assert rows(dl=None) == _lib.EINVAL                # lengths in but not out
    assert rows(dt=FAKE + 16) == _lib.EINVAL           # destination overlaps the source table
    assert rows(n=0, perm=None) == _lib.OK

    src = _cache(layout=_lib.CONTIGUOUS, rows=4)
    dst = _cache(layout=_lib.CONTIGUOUS, rows=4)
    dst.k, dst.v = FAKE + 0x4000000, FAKE + 0x8000000

    def cache(s=src, d=dst, n=4, perm=P, sl=None, dl=None):
        return L.kvattn_reorder_cache(ctypes.byref(s), ctypes.byref(d), n, perm, sl, dl, None)

    assert cache(s=_cache()) == _lib.EINVAL            # paged source
    assert cache(d=_cache(layout=_lib.CONTIGUOUS, rows=4)) == _lib.EINVAL   # dst memory == src memory
    other = _cache(layout=_lib.CONTIGUOUS, rows=4, capacity=512)
    other.k, other.v = dst.k, dst.v
    assert cache(d=other) == _lib.EINVAL               # capacity differs
    assert cache(n=8) == _lib.EINVAL                   # dst has 4 rows
    assert cache(dl=FAKE) == _lib.EINVAL               # dst_lens without src_lens
    assert cache(perm=None) == _lib.EINVAL
    assert cache(n=0, perm=None) == _lib.OK

    assert L.kvattn_copy_blocks(ctypes.byref(_cache(layout=_lib.CONTIGUOUS)), 4, P, P, None) == _lib.EINVAL
    assert L.kvattn_copy_blocks(ctypes.byref(_cache()), 4, None, P, None) == _lib.EINVAL
    assert L.kvattn_copy_blocks(ctypes.byref(_cache()), -1, P, P, None) == _lib.EINVAL
    assert L.kvattn_copy_blocks(None, 4, P, P, None) == _lib.EINVAL
    assert L.kvattn_copy_blocks(ctypes.byref(_cache()), 0, None, None, None) == _lib.OK


def _decode_multi(c, n_q=4, hq=32, k_new=None, v_new=None, in_dtype=-1, part=0):
    L = _lib.lib()
    return L.kvattn_attn_decode_multi(ctypes.byref(c), 4, hq, n_q, FAKE, _lib.BF16, k_new, v_new, in_dtype, FAKE, 1000,
                                      FAKE, 64, None, 0, 0.1, FAKE, None, 0, part, None)


@pytest.mark.parametrize("kw,want", [
    ({"n_q": 0}, _lib.EINVAL),
    ({"n_q": 17}, _lib.EINVAL),
    ({"hq": 8, "n_q": 3}, _lib.EUNSUPPORTED),                          # G 1 x 3 queries = 3 columns
    ({"hq": 64, "n_q": 4}, _lib.EUNSUPPORTED),                         # G 8 x 4 = 32 columns > 16
    ({"k_new": FAKE}, _lib.EINVAL),                                    # k_new without v_new / dtype
    ({"k_new": FAKE, "v_new": FAKE, "in_dtype": 7}, _lib.EINVAL),
    ({"k_new": FAKE, "in_dtype": _lib.BF16}, _lib.EINVAL),            # v_new missing
    ({"k_new": FAKE, "v_new": FAKE, "in_dtype": _lib.F32}, _lib.EUNSUPPORTED),  # f32 rows into a bf16 cache
    ({}, _lib.EWORKSPACE),                                             # valid up to the workspace
])
def test_decode_multi_host_errors(kw, want):
    assert _decode_multi(_cache(), **kw) == want
    assert _lib.lib().kvattn_last_error().decode() != ""


def test_stream_read_host_errors():
    L = _lib.lib()
    assert L.kvattn_stream_read(FAKE, 100, FAKE + 0x1000, None) == _lib.EINVAL       # not a multiple of 16
    assert L.kvattn_stream_read(FAKE, -16, FAKE + 0x1000, None) == _lib.EINVAL
    assert L.kvattn_stream_read(None, 64, FAKE + 0x1000, None) == _lib.EINVAL
    assert L.kvattn_stream_read(FAKE, 64, None, None) == _lib.EINVAL
    assert L.kvattn_stream_read(FAKE + 8, 64, FAKE + 0x1000, None) == _lib.EINVAL    # src not 16-byte aligned
    assert L.kvattn_stream_read(FAKE, 64, FAKE + 0x1002, None) == _lib.EINVAL        # sink not 4-byte aligned
    assert L.kvattn_stream_read(None, 0, None, None) == _lib.OK                     # nothing to read
