"""Pins for the paged-cache bookkeeping in the oracle (oracle/paging.py):
printed examples, hand-worked cases, numpy routines and invariants.

Page keys as in test_oracle_pins.py:
  [P1] "KV Cache, Flash Attention and Inference Optimization"
  [P2] "KV Cache Fully Explained: The Core of LLM Inference Memory"
  [P4] "Transformer Attention Masks and KV-Cache Inference"
"""
import os

import numpy as np
import pytest

from kv_cache_decode_attn_amd import synth
from oracle import paging as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


# ------------------------------------------------------------- reorder ---

def test_reorder_matches_printed_beam_example():
    """[P4] "Batch and beam reorder": [A0, A1, B0] with perm [2, 1, 0]
    becomes [B0, A1, A0] - for table rows, lengths and contiguous rows."""
    before, perm, after = _rows("beam_reorder.txt")
    perm = [int(x) for x in perm]
    code = {name: i for i, name in enumerate(sorted(set(before)))}
    # a table row and a length per named beam, all distinct
    table = np.array([[10 * code[n] + j for j in range(3)] for n in before], dtype=np.int32)
    lens = np.array([5 + code[n] for n in before], dtype=np.int32)
    t, l = P.reorder_rows(table, lens, perm)
    want = np.array([[10 * code[n] + j for j in range(3)] for n in after], dtype=np.int32)
    np.testing.assert_array_equal(t, want)
    np.testing.assert_array_equal(l, [5 + code[n] for n in after])
    # contiguous rows: every byte of a row carries its beam's code
    src = np.stack([np.full((2, 4, 3), code[n], dtype=np.uint16) for n in before])
    out, _ = P.reorder_contiguous(src, np.zeros_like(src), perm)
    np.testing.assert_array_equal(out[:, 0, 0, 0], [code[n] for n in after])


def test_reorder_equals_numpy_take_and_inverts():
    rng = np.random.default_rng(3)
    table = rng.integers(0, 1000, size=(7, 5)).astype(np.int32)
    lens = rng.integers(0, 80, size=7).astype(np.int32)
    perm = rng.permutation(7)
    t, l = P.reorder_rows(table, lens, perm)
    np.testing.assert_array_equal(t, np.take(table, perm, axis=0))
    np.testing.assert_array_equal(l, np.take(lens, perm))
    inv = np.argsort(perm)
    t2, l2 = P.reorder_rows(t, l, inv)
    np.testing.assert_array_equal(t2, table)
    np.testing.assert_array_equal(l2, lens)


def test_reorder_duplicates_and_invalid_entries():
    """Beam search keeps a parent's cache in several children (perm with
    repeats); an index outside the rows gives an empty row."""
    table = np.arange(6, dtype=np.int32).reshape(3, 2)
    lens = np.array([3, 17, 30], dtype=np.int32)
    t, l = P.reorder_rows(table, lens, [1, 1, -1, 3])
    np.testing.assert_array_equal(t, [[2, 3], [2, 3], [-1, -1], [-1, -1]])
    np.testing.assert_array_equal(l, [17, 17, 0, 0])


def test_reorder_contiguous_copies_only_valid_prefix():
    rng = np.random.default_rng(4)
    src = rng.integers(0, 65535, size=(3, 2, 8, 4)).astype(np.uint16)
    dst = rng.integers(0, 65535, size=(4, 2, 8, 4)).astype(np.uint16)
    lens = np.array([5, 0, 11], dtype=np.int32)
    perm = [2, 0, 7, 1]
    out, nl = P.reorder_contiguous(src, dst, perm, lens)
    np.testing.assert_array_equal(nl, [11, 5, 0, 0])
    np.testing.assert_array_equal(out[0], src[2])            # 11 clamps to the capacity 8
    np.testing.assert_array_equal(out[1, :, :5], src[0, :, :5])
    np.testing.assert_array_equal(out[1, :, 5:], dst[1, :, 5:])
    np.testing.assert_array_equal(out[2], dst[2])            # invalid index: untouched
    np.testing.assert_array_equal(out[3], dst[3])            # length 0: untouched


# --------------------------------------------------------- block copies ---

def test_copy_blocks_moves_only_named_blocks():
    rng = np.random.default_rng(5)
    pool = rng.integers(0, 255, size=(6, 2, 16, 8)).astype(np.uint8)
    out = P.copy_blocks(pool, [0, 3, 9, 2], [4, 5, 1, -1])
    np.testing.assert_array_equal(out[4], pool[0])
    np.testing.assert_array_equal(out[5], pool[3])
    for b in (0, 1, 2, 3):                                   # out-of-range pairs skipped
        np.testing.assert_array_equal(out[b], pool[b])


def test_copy_blocks_pairs_are_simultaneous():
    pool = np.arange(3, dtype=np.int32).reshape(3, 1)
    np.testing.assert_array_equal(P.copy_blocks(pool, [0, 1], [1, 0])[:, 0], [1, 0, 2])


# ------------------------------------------------------ reference pool ---

def test_pool_free_list_lowest_first_and_all_or_nothing():
    """[P1] "Exercises" (hard): a free list of fixed blocks, returned to the
    pool when a sequence ends."""
    pool = P.RefPool(4)
    assert pool.alloc(3) == [0, 1, 2]
    assert pool.num_free() == 1
    with pytest.raises(P.NoSpace):
        pool.alloc(2)
    assert pool.ref == [1, 1, 1, 0]
    pool.release([1])
    assert pool.alloc(1) == [1]
    with pytest.raises(P.BadBlock):
        pool.release([3])                                    # never allocated
    with pytest.raises(P.BadBlock):
        pool.release([0, 0])                                 # held once
    assert pool.ref == [1, 1, 1, 0]


def test_pool_prefix_share_then_copy_on_write():
    """[P2] "(4) PagedAttention": sharers point at one physical block; the
    first writer of a shared, partly filled block gets a copy."""
    pool = P.RefPool(8)
    (parent,), _ = pool.prepare_append([[-1] * 4], [0], [20])    # 2 blocks, second partly filled
    assert parent[:2] == [0, 1] and pool.ref[:2] == [1, 1]
    child = pool.fork(parent, 20, 4)
    assert child[:2] == [0, 1] and pool.ref[:2] == [2, 2]
    (child,), pairs = pool.prepare_append([child], [20], [21])
    assert pairs == [(1, 2)] and child[:2] == [0, 2]
    assert pool.ref[:3] == [2, 1, 1]
    (parent,), pairs = pool.prepare_append([parent], [20], [21])   # now sole holder of block 1
    assert pairs == [] and parent[:2] == [0, 1]
    # a shared full block is never copied: appends start a new block
    c2 = pool.fork(parent, 16, 4)
    (c2,), pairs = pool.prepare_append([c2], [16], [40])
    assert pairs == [] and c2[:3] == [0, 3, 4] and pool.ref[0] == 3
    for row, n in ((parent, 21), (child, 21), (c2, 40)):
        pool.free_seq(row, n)
    assert pool.num_free() == 8


def test_pool_batch_prepare_is_sequential_and_atomic():
    pool = P.RefPool(3)
    (a,), _ = pool.prepare_append([[-1, -1]], [0], [5])
    b = pool.fork(a, 5, 2)
    # both sharers append: the first copies, the second is then sole holder
    (a2, b2), pairs = pool.prepare_append([a, b], [5, 5], [6, 6])
    assert pairs == [(0, 1)] and a2[0] == 1 and b2[0] == 0
    # needs 2 new blocks with 1 free: nothing changes
    ref = list(pool.ref)
    with pytest.raises(P.NoSpace):
        pool.prepare_append([a2, b2], [6, 6], [17, 17])
    assert pool.ref == ref


def test_pool_reorder_moves_references():
    pool = P.RefPool(6)
    tables, _ = pool.prepare_append([[-1, -1]] * 3, [0, 0, 0], [17, 5, 9])
    tables = np.array(tables, dtype=np.int32)
    lens = np.array([17, 5, 9], dtype=np.int32)
    t, l = pool.reorder(tables, lens, [2, 0, 0])
    np.testing.assert_array_equal(t, [[3, -1], [0, 1], [0, 1]])
    np.testing.assert_array_equal(l, [9, 17, 17])
    assert pool.ref == [2, 2, 0, 1, 0, 0]                     # row 1's block returned


# ------------------------------------------------- fragmentation ---

def test_reserved_tokens_closed_forms():
    for L, want in ((0, 0), (1, 16), (15, 16), (16, 16), (17, 32), (4096, 4096)):
        assert P.reserved_tokens_paged(L) == want
    for L in range(0, 200):
        assert 0 <= P.reserved_tokens_paged(L) - L < 16
        assert P.reserved_tokens_contiguous(L, 4096) == 4096


def test_fragmentation_trace_matches_hand_worked_run():
    want = np.array([[int(x) for x in r] for r in _rows("fragmentation_tiny.txt")], dtype=np.int64)
    tr = P.fragmentation_trace([3, 15], [2, 2], slots=1, max_len=32)
    got = np.stack([tr["active"], tr["live_tokens"], tr["paged_reserved"], tr["contiguous_reserved"]], axis=1)
    np.testing.assert_array_equal(got, want)


def _pool_driven_trace(prompts, outputs, slots, max_len, prefix):
    """The same schedule run on RefPool itself (tables, forks, copy-on-write),
    measuring the blocks actually held: a route independent of the closed
    forms in fragmentation_trace."""
    mb = P.blocks_for(max_len)
    pool = P.RefPool(slots * mb + mb)
    root = None
    if prefix:
        (root,), _ = pool.prepare_append([[-1] * mb], [0], [prefix])
    queue, active, held = 0, [], []
    while queue < len(prompts) or active:
        while queue < len(prompts) and len(active) < slots:
            row = pool.fork(root, prefix, mb) if prefix else [-1] * mb
            active.append([row, prefix, int(prompts[queue]), 0, queue])
            queue += 1
        # new requests: prefix -> prompt + 1; running ones: L -> L + 1
        cur = [s[1] for s in active]
        new = [(s[2] if s[3] == 0 else s[1]) + 1 for s in active]
        tables, _ = pool.prepare_append([s[0] for s in active], cur, new)
        for s, t, n in zip(active, tables, new):
            s[0], s[1], s[3] = t, n, s[3] + 1
        held.append((pool.num_blocks - pool.num_free()) * 16)
        keep = []
        for s in active:
            if s[3] < int(outputs[s[4]]):
                keep.append(s)
            else:
                pool.free_seq(s[0], s[1])
        active = keep
    if prefix:
        pool.free_seq(root, prefix)
    assert pool.num_free() == pool.num_blocks
    return np.asarray(held, dtype=np.int64)


@pytest.mark.parametrize("prefix", [0, 40, 48])
def test_fragmentation_trace_equals_pool_simulation(prefix):
    p, o = synth.chat_lengths(120, (9, synth.T_LENS), max_len=1024, prefix=prefix, prompt_median=100,
                              output_median=60)
    tr = P.fragmentation_trace(p, o, slots=16, max_len=1024, shared_prefix=prefix)
    np.testing.assert_array_equal(tr["paged_reserved"], _pool_driven_trace(p, o, 16, 1024, prefix))
    assert np.all(tr["contiguous_reserved"] == 1024 * tr["active"])
    assert int(tr["live_tokens"].max()) <= 16 * 1024
    if not prefix:
        assert np.all(tr["paged_reserved"] - tr["live_tokens"] < 16 * tr["active"])
