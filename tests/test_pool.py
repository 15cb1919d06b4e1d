"""The library's host block pool (kvattn_pool_*) against the oracle's
reference pool, and the fragmentation study against the oracle's closed
forms.  Host code only: no GPU needed.

Both pools hand out the lowest free id first, so tables, copy pairs and
reference counts must agree exactly after every operation.
"""
import numpy as np
import pytest

from kv_cache_decode_attn_amd import _lib, api, fragmentation, synth
from oracle import paging as P

MB = 6


def _same(pool, ref):
    assert pool.num_free() == ref.num_free()
    assert [pool.refcount(b) for b in range(ref.num_blocks)] == ref.ref


def _status(fn, *a):
    try:
        return fn(*a), 0
    except _lib.KvattnError as e:
        return None, e.status


@pytest.mark.parametrize("seed", range(6))
def test_pool_random_operations_match_reference(seed):
    """Random forks, appends (with copy-on-write), reorders and frees on both
    pools; every result and every failure must agree."""
    rng = np.random.default_rng([seed, 77])
    nb = int(rng.integers(8, 40))
    pool, ref = api.BlockPool(nb), P.RefPool(nb)
    rows = 5
    tables = np.full((rows, MB), -1, dtype=np.int32)
    lens = np.zeros(rows, dtype=np.int32)
    for _ in range(300):
        op = rng.integers(0, 4)
        if op == 0:                                   # grow every row by a random amount
            new = np.minimum(lens + rng.integers(0, 20, size=rows), 16 * MB).astype(np.int32)
            t = tables.copy()
            got, st = _status(pool.prepare_append, t, lens.copy(), new)
            try:
                want_t, pairs = ref.prepare_append(tables.tolist(), lens.tolist(), new.tolist())
                want_st = 0
            except P.NoSpace:
                want_st = _lib.ENOSPACE
            assert st == want_st
            if st == 0:
                np.testing.assert_array_equal(t, np.array(want_t, dtype=np.int32))
                assert list(zip(got[0].tolist(), got[1].tolist())) == pairs
                tables, lens = t, new
            else:
                np.testing.assert_array_equal(t, tables)       # all-or-nothing
        elif op == 1:                                 # fork row a's prefix into row b
            a, b = rng.choice(rows, 2, replace=False)
            n = int(rng.integers(0, lens[a] + 1))
            ref.free_seq(tables[b].tolist(), int(lens[b]))
            pool.free_seq(tables[b], int(lens[b]))
            want = ref.fork(tables[a].tolist(), n, MB)
            pool.fork(tables[a], n, tables[b])
            np.testing.assert_array_equal(tables[b], want)
            lens[b] = n
        elif op == 2:                                 # beam reorder with repeats
            perm = rng.integers(0, rows, size=rows).astype(np.int32)
            wt, wl = ref.reorder(tables, lens, perm)
            gt, gl = pool.reorder(perm, tables, lens)
            np.testing.assert_array_equal(gt, wt)
            np.testing.assert_array_equal(gl, wl)
            tables, lens = gt, gl.astype(np.int32)
        else:                                         # a sequence ends
            r = int(rng.integers(0, rows))
            want = ref.free_seq(tables[r].tolist(), int(lens[r]))
            pool.free_seq(tables[r], int(lens[r]))
            np.testing.assert_array_equal(tables[r], want)
            lens[r] = 0
        _same(pool, ref)
    for r in range(rows):
        pool.free_seq(tables[r], int(lens[r]))
    assert pool.num_free() == nb


def test_pool_errors_leave_state_unchanged():
    pool = api.BlockPool(4)
    ids = pool.alloc(3)
    np.testing.assert_array_equal(ids, [0, 1, 2])
    with pytest.raises(_lib.KvattnError) as e:
        pool.alloc(2)
    assert e.value.status == _lib.ENOSPACE
    with pytest.raises(_lib.KvattnError) as e:
        pool.release(np.array([0, 0], dtype=np.int32))      # held once
    assert e.value.status == _lib.EINVAL
    with pytest.raises(_lib.KvattnError):
        pool.retain(np.array([3], dtype=np.int32))          # free block
    with pytest.raises(_lib.KvattnError):
        pool.release(np.array([9], dtype=np.int32))         # out of range
    assert [pool.refcount(b) for b in range(4)] == [1, 1, 1, 0] and pool.refcount(4) == -1
    row = np.array([0, 1, -1], dtype=np.int32)
    with pytest.raises(_lib.KvattnError):
        pool.fork(row, 40)                                  # 3 blocks named, third is -1
    with pytest.raises(_lib.KvattnError):
        pool.free_seq(row.copy(), 49)                       # does not fit 3 entries
    t = np.array([[0, 1, -1]], dtype=np.int32)
    with pytest.raises(_lib.KvattnError):                   # shrinking is not an append
        pool.prepare_append(t, np.array([20], np.int32), np.array([10], np.int32))
    np.testing.assert_array_equal(t, [[0, 1, -1]])
    assert pool.num_free() == 1
    assert _lib.lib().kvattn_pool_create(0) is None


def test_pool_copy_on_write_needs_one_free_block():
    pool = api.BlockPool(2)
    t = np.full((2, 2), -1, dtype=np.int32)
    pool.prepare_append(t[:1], np.array([0], np.int32), np.array([20], np.int32))   # blocks 0, 1
    pool.fork(t[0], 20, t[1])
    with pytest.raises(_lib.KvattnError) as e:              # the shared partial block needs a copy
        pool.prepare_append(t, np.array([20, 20], np.int32), np.array([21, 21], np.int32))
    assert e.value.status == _lib.ENOSPACE
    assert pool.refcount(1) == 2
    pool.free_seq(t[1], 20)
    cs, cd = pool.prepare_append(t, np.array([20, 0], np.int32), np.array([21, 0], np.int32))
    assert len(cs) == 0                                     # sole holder again: written in place


@pytest.mark.parametrize("prefix", [0, 40])
def test_fragmentation_study_matches_closed_forms(prefix):
    """1,000 synthetic chat completions ([P1] "Exercises", hard): the pool's
    blocks in use equal the closed form at every step."""
    p, o = synth.chat_lengths(1000, (11, synth.T_LENS), max_len=4096, prefix=prefix)
    trace, copies = fragmentation.run(p, o, 64, 4096, prefix)
    want = P.fragmentation_trace(p, o, 64, 4096, shared_prefix=prefix)
    for k in want:
        np.testing.assert_array_equal(trace[k], want[k], err_msg=k)
    assert copies == (1000 if prefix % 16 else 0)          # one copy per request sharing a partial block
    s = fragmentation.summary(trace, 131072)
    assert s["contiguous"]["unused_mean_bytes"] > 100 * abs(s["paged"]["unused_mean_bytes"])
    if not prefix:
        assert 0 <= s["paged"]["unused_peak_bytes"] < 16 * 64 * 131072
