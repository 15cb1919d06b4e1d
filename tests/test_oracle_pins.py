"""Pins for the CPU oracle: each test ties an oracle function to something
other than itself - values the pages print, closed forms, a library routine,
brute force on tiny inputs, or an invariant that a plausible mistake breaks.

Page keys used in test names and comments:
  [P1] "KV Cache, Flash Attention and Inference Optimization"
  [P2] "KV Cache Fully Explained: The Core of LLM Inference Memory"
  [P3] "KV Cache" (heepie.pages.dev)
  [P4] "Transformer Attention Masks and KV-Cache Inference"
"""
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention as A
from oracle import cache as C
from oracle import codec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ----------------------------------------------------------------- masks ---

def test_causal_allow_matches_printed_4x4():
    """[P4] "Causal mask and future positions" prints the 4x4 allow matrix."""
    want = np.array([[int(x) for x in r] for r in _load_rows("causal_allow_4x4.txt")], dtype=np.uint8)
    assert want.shape == (4, 4)
    np.testing.assert_array_equal(A.causal_allow(4), want)


def test_causal_weights_position0_reads_nothing_after_it():
    """[P4] "Implementation and verification procedure": with a length-4
    causal prompt, position 0 must not read positions 1-3 and position 3
    reads 0-3.  Weights are exactly 0 above the diagonal."""
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((4, 8)), rng.standard_normal((4, 8))
    w = A.attention_weights(q, k, A.causal_allow(4), 1 / math.sqrt(8))
    assert np.all(w[np.triu_indices(4, 1)] == 0.0)
    assert np.all(w[np.tril_indices(4)] > 0.0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_weights_equal_library_softmax():
    """softmax of the scaled scores over allowed keys == scipy.special.softmax."""
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((5, 16)), rng.standard_normal((9, 16))
    allow = rng.random((5, 9)) < 0.7
    allow[:, 0] = True
    scale = 1 / math.sqrt(16)
    w = A.attention_weights(q, k, allow, scale)
    for t in range(5):
        idx = np.nonzero(allow[t])[0]
        ref = scipy.special.softmax((q[t] @ k[idx].T) * scale)
        np.testing.assert_allclose(w[t, idx], ref, rtol=1e-13, atol=0)
        assert np.all(w[t, ~allow[t]] == 0.0)


def test_one_hot_values_read_back_weights():
    """V = identity rows: output row t equals weight row t (pin used on GPU too)."""
    rng = np.random.default_rng(3)
    n = 6
    q, k = rng.standard_normal((n, 4)), rng.standard_normal((n, 4))
    allow = A.causal_allow(n)
    out = A.sdpa(q, k, np.eye(n), allow, 0.5)
    np.testing.assert_allclose(out, A.attention_weights(q, k, allow, 0.5), rtol=0, atol=1e-15)


def test_padding_rows_equal_unpadded_run_and_ignore_pad_values():
    """[P4] "Padding mask and batch length": two real length-3 sequences
    padded to 5 ([A,B,C,PAD,PAD]); real rows equal the unpadded computation,
    and PAD K/V (set to NaN here) never reach the output."""
    rng = np.random.default_rng(4)
    d = 8
    for causal in (False, True):
        for _ in range(2):
            q = rng.standard_normal((5, d))
            k = rng.standard_normal((5, d))
            v = rng.standard_normal((5, d))
            k[3:] = np.nan
            v[3:] = np.nan
            key_mask = np.array([1, 1, 1, 0, 0], dtype=np.uint8)
            allow = np.broadcast_to(key_mask, (5, 5)).copy()
            if causal:
                allow &= A.causal_allow(5)
            padded = A.sdpa(q, k, v, allow, 0.3)
            ref_allow = A.causal_allow(3) if causal else np.ones((3, 3), np.uint8)
            unpadded = A.sdpa(q[:3], k[:3], v[:3], ref_allow, 0.3)
            assert np.all(np.isfinite(padded[:3]))
            np.testing.assert_array_equal(padded[:3], unpadded)


def test_all_masked_row_is_zero():
    """[P4] "Implementation and verification procedure": all-masked rows are
    implementation-defined (NaN or uniform); the reading taken is 0."""
    out = A.sdpa(np.ones((2, 4)), np.ones((3, 4)), np.ones((3, 4)), np.zeros((2, 3), np.uint8), 1.0)
    assert np.all(out == 0.0)


# ------------------------------------------------------ closed forms ------

def test_two_key_closed_form_is_logistic():
    """Two keys: weight of key 1 = 1 / (1 + exp(-(z1 - z0))) with z = scale q.k.
    Catches a dropped scale, a sign error, or a transposed product."""
    a, scale = 1.7, 0.25
    q = np.array([[a, 0.0, 0.0]])
    k = np.array([[0.0, 0.0, 0.0], [1.0, 2.0, -3.0]])
    v = np.array([[1.0, 2.0, 3.0], [-4.0, 5.0, 0.5]])
    w1 = 1.0 / (1.0 + math.exp(-a * scale))
    want = (1 - w1) * v[0] + w1 * v[1]
    np.testing.assert_allclose(A.sdpa(q, k, v, np.ones((1, 2)), scale)[0], want, rtol=1e-15, atol=1e-15)


def test_single_allowed_key_returns_its_value_exactly():
    rng = np.random.default_rng(5)
    q, k, v = rng.standard_normal((1, 8)), rng.standard_normal((7, 8)), rng.standard_normal((7, 8))
    allow = np.zeros((1, 7), np.uint8)
    allow[0, 4] = 1
    np.testing.assert_array_equal(A.sdpa(q, k, v, allow, 0.9)[0], v[4])


def test_zero_query_or_identical_keys_give_mean_of_allowed_values():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((9, 5))
    allow = np.array([[1, 0, 1, 1, 0, 1, 1, 0, 1]], np.uint8)
    mean = v[allow[0] == 1].mean(axis=0)
    np.testing.assert_allclose(A.sdpa(np.zeros((1, 5)), rng.standard_normal((9, 5)), v, allow, 1.0)[0],
                               mean, rtol=0, atol=1e-15)
    same = np.tile(rng.standard_normal((1, 5)), (9, 1))
    np.testing.assert_allclose(A.sdpa(rng.standard_normal((1, 5)), same, v, allow, 1.0)[0],
                               mean, rtol=0, atol=1e-14)


def test_rows_sum_to_one_constant_values():
    """Softmax rows sum to 1 ([P3] "Self-Attention": the scores are
    normalised so that they sum to 1): with V == 1 the output is 1."""
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal((6, 16)), rng.standard_normal((6, 16)) * 4
    out = A.sdpa(q, k, np.ones((6, 3)), A.causal_allow(6), 0.25)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)


def test_brute_force_tiny():
    """Pure-Python loops with math.exp on a 3x4 case."""
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((3, 2)), rng.standard_normal((4, 2)), rng.standard_normal((4, 3))
    allow = np.array([[1, 1, 0, 1], [0, 1, 1, 1], [1, 0, 0, 0]], np.uint8)
    out = A.sdpa(q, k, v, allow, 0.7)
    for t in range(3):
        keys = [s for s in range(4) if allow[t][s]]
        zs = [0.7 * sum(q[t][i] * k[s][i] for i in range(2)) for s in keys]
        ex = [math.exp(z) for z in zs]
        tot = sum(ex)
        for j in range(3):
            ref = sum(ex[i] / tot * v[s][j] for i, s in enumerate(keys))
            assert abs(out[t][j] - ref) < 1e-14


# ---------------------------------------------------------- second route ---

@pytest.mark.parametrize("tile", [1, 3, 4, 16])
def test_tiled_running_max_equals_one_shot(tile):
    """[P1] "Flash Attention", numerical trick: the running (max, sum)
    route is exact, not an approximation - equal to the plain definition."""
    rng = np.random.default_rng(10 + tile)
    n, d = 37, 16
    q, k, v = rng.standard_normal(d), rng.standard_normal((n, d)) * 3, rng.standard_normal((n, d))
    allow = rng.random(n) < 0.8
    allow[0] = False  # a masked key inside the first tile
    got = A.tiled_fold(q, k, v, 0.25, tile, allow)
    want = A.sdpa(q[None], k, v, allow[None], 0.25)[0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_tiled_with_masked_first_tiles():
    """Leading tiles entirely masked keep m = -inf and must not poison the state."""
    rng = np.random.default_rng(20)
    q, k, v = rng.standard_normal(8), rng.standard_normal((20, 8)), rng.standard_normal((20, 8))
    allow = np.zeros(20, bool)
    allow[13:] = True
    np.testing.assert_allclose(A.tiled_fold(q, k, v, 0.5, 4, allow),
                               A.sdpa(q[None], k, v, allow[None], 0.5)[0], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("part", [1, 5, 16, 64, 1000])
def test_split_partials_merge_equals_direct(part):
    rng = np.random.default_rng(30 + part)
    n, d = 200, 8
    q, k, v = rng.standard_normal(d), rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d))
    allow = rng.random(n) < 0.5
    allow[:40] = False  # whole empty partitions for small `part`
    got = A.merge_partials(A.split_partials(q, k, v, 0.3, part, allow))
    want = A.sdpa(q[None], k, v, allow[None], 0.3)[0]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_merge_all_empty_partitions_is_zero():
    parts = A.split_partials(np.ones(4), np.ones((8, 4)), np.ones((8, 4)), 1.0, 4, np.zeros(8, bool))
    assert np.all(A.merge_partials(parts) == 0.0)


# -------------------------------------------------- decode and prefill ----

def _rand_cache(rng, B, Hkv, cap, d):
    return [rng.standard_normal((Hkv, cap, d)) for _ in range(B)], [rng.standard_normal((Hkv, cap, d)) for _ in range(B)]


def test_decode_equals_last_row_of_full_recompute():
    """[P4] "Implementation and verification procedure": the cached path and
    the uncached path give the same result; [P3] "AS-IS" / "TO-BE"."""
    rng = np.random.default_rng(40)
    n, d = 23, 16
    qa, ka, va = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal((n, d))
    full = A.full_recompute_last_row(qa, ka, va, 0.25)
    dec = A.decode(qa[-1][None, None], [ka[None]], [va[None]], [n], 0.25)[0, 0]
    np.testing.assert_allclose(dec, full, rtol=1e-13, atol=1e-14)


def test_prefill_rows_equal_token_by_token_decode():
    """[P4] "Implementation and verification procedure": full prefill vs
    token-by-token decode at the same positions."""
    rng = np.random.default_rng(41)
    B, Hq, Hkv, N, d = 2, 4, 2, 9, 8
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    pre = A.prefill(q, k, v, [0, 0], [N, N], 0.35)
    for t in range(N):
        dec = A.decode(q[:, :, t], [k[b] for b in range(B)], [v[b] for b in range(B)], [t + 1, t + 1], 0.35)
        np.testing.assert_allclose(pre[:, :, t], dec, rtol=1e-13, atol=1e-14)


def test_chunked_prefill_equals_matching_rows_of_full_prefill():
    """A second chunk attending the cached first chunk reproduces the rows of
    a one-shot prefill (the append-then-attend contract of [P4] "Prefill and
    decode stages" applied to several new tokens)."""
    rng = np.random.default_rng(42)
    Hq, Hkv, N, d, c = 2, 1, 12, 8, 5
    q = rng.standard_normal((1, Hq, N, d))
    k = rng.standard_normal((1, Hkv, N, d))
    v = rng.standard_normal((1, Hkv, N, d))
    full = A.prefill(q, k, v, [0], [N], 0.4)
    second = A.prefill(q[:, :, c:], k[:, :, c:], v[:, :, c:], [c], [N - c], 0.4,
                       prefix_k=[k[0]], prefix_v=[v[0]], attend_prefix=True)
    np.testing.assert_allclose(second[:, :, :N - c], full[:, :, c:], rtol=1e-13, atol=1e-14)


# ------------------------------------------ prefill masking branches ------
#
# Each case below runs oracle.attention.prefill and compares every output row
# with a brute force written from the definition alone: pure-Python loops
# over absolute key positions with math.exp, no numpy linear algebra and no
# call into the oracle.


def _brute_prefill(q, k_new, v_new, positions, q_lens, scale, causal, key_mask=None,
                   prefix_k=None, prefix_v=None, attend_prefix=False):
    """out[b, h, t] for the rows t < q_lens[b]; rows past q_lens[b] are 0.
    Query t of sequence b sits at absolute position P + t (P = positions[b]);
    it may read key position s iff lo <= s < P + q_lens[b] (lo = 0 with a
    cached prefix, else P), s <= P + t when causal, and key_mask[b][s] != 0
    when a mask is given (the mask is indexed by ABSOLUTE position).  Key s
    comes from the prefix when s < P, else from new row s - P."""
    B, Hq, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k_new[0])
    G = Hq // Hkv
    dv = len(v_new[0][0][0])
    out = np.zeros((B, Hq, N, dv))
    for b in range(B):
        P, n = int(positions[b]), int(q_lens[b])
        for h in range(Hq):
            g = h // G
            for t in range(n):
                keys = []
                for s in range(0 if attend_prefix else P, P + n):
                    if causal and s > P + t:
                        continue
                    if key_mask is not None and not key_mask[b][s]:
                        continue
                    keys.append(s)
                if not keys:
                    continue
                krow = lambda s: prefix_k[b][g][s] if s < P else k_new[b][g][s - P]
                vrow = lambda s: prefix_v[b][g][s] if s < P else v_new[b][g][s - P]
                z = [scale * sum(float(q[b][h][t][i]) * float(krow(s)[i]) for i in range(d)) for s in keys]
                zmax = max(z)
                e = [math.exp(x - zmax) for x in z]
                tot = sum(e)
                for j in range(dv):
                    out[b, h, t, j] = sum(e[i] / tot * float(vrow(s)[j]) for i, s in enumerate(keys))
    return out


def _padded_batch(rng, d=6):
    """The padding example of [P4] "Padding mask and batch length": real
    length 3 ([A, B, C]) padded to a batch length of 5 ([A, B, C, PAD,
    PAD]), two such sequences; PAD K/V are NaN so that any leak shows."""
    B, Hq, Hkv, N = 2, 2, 1, 5
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    k[:, :, 3:] = np.nan
    v[:, :, 3:] = np.nan
    mask = np.array([[1, 1, 1, 0, 0], [1, 1, 1, 0, 0]], np.uint8)
    return q, k, v, mask


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_padding_example_padded_rows_zero(causal):
    """[P4] "Padding mask and batch length" and "Implementation and
    verification procedure" (two length-3 inputs padded into one batch, PAD
    influence checked): with q_lens = [3, 3] the PAD query rows are 0 and the
    real rows equal the brute force over keys 0..2 - causal or not."""
    rng = np.random.default_rng(70)
    q, k, v, mask = _padded_batch(rng)
    scale = 1 / math.sqrt(6)
    got = A.prefill(q, k, v, [0, 0], [3, 3], scale, causal=causal, key_mask=mask)
    want = _brute_prefill(q, k, v, [0, 0], [3, 3], scale, causal, key_mask=mask)
    assert np.all(np.isfinite(got))
    assert np.all(got[:, :, 3:] == 0.0)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    # without the key mask the result is the same: keys past q_lens are not keys
    np.testing.assert_array_equal(A.prefill(q, k, v, [0, 0], [3, 3], scale, causal=causal), got)


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_padding_example_key_mask_blocks_pad(causal):
    """Same batch with every row a query (q_lens = [5, 5]) and the padding
    mask on the keys: PAD keys get weight 0, so every row - the PAD query
    rows included - is finite and equals the brute force over keys 0..2.
    Non-causal, rows 0..2 all see A, B, C (an encoder reads the future but
    never PAD)."""
    rng = np.random.default_rng(71)
    q, k, v, mask = _padded_batch(rng)
    scale = 0.37
    got = A.prefill(q, k, v, [0, 0], [5, 5], scale, causal=causal, key_mask=mask)
    want = _brute_prefill(q, k, v, [0, 0], [5, 5], scale, causal, key_mask=mask)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    if not causal:
        # every query of a sequence reads the same three keys
        w = A.attention_weights(q[0, 0], k[0, 0, :3], np.ones((5, 3)), scale)
        np.testing.assert_allclose(got[0, 0], w @ v[0, 0, :3], rtol=1e-12, atol=1e-13)


def test_prefill_non_causal_equals_library_softmax():
    """causal=False: every query row reads every real key; each row equals
    scipy's softmax of the scaled scores applied to V."""
    rng = np.random.default_rng(72)
    B, Hq, Hkv, N, d = 2, 4, 2, 7, 5
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    lens = [7, 4]
    got = A.prefill(q, k, v, [0, 0], lens, 0.45, causal=False)
    for b in range(B):
        for h in range(Hq):
            g = h // 2
            for t in range(N):
                if t >= lens[b]:
                    assert np.all(got[b, h, t] == 0.0)
                    continue
                w = scipy.special.softmax(0.45 * k[b, g, :lens[b]] @ q[b, h, t])
                np.testing.assert_allclose(got[b, h, t], w @ v[b, g, :lens[b]], rtol=1e-12, atol=1e-13)


def test_prefill_at_offset_without_prefix():
    """positions > 0 with attend_prefix=False: only the new keys are read,
    causal by absolute position - the same as the same tokens at position 0,
    and as the brute force; a key mask indexed by absolute position."""
    rng = np.random.default_rng(73)
    B, Hq, Hkv, N, d = 2, 2, 1, 6, 4
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    pos, lens = [9, 4], [6, 5]
    got = A.prefill(q, k, v, pos, lens, 0.6)
    np.testing.assert_allclose(got, A.prefill(q, k, v, [0, 0], lens, 0.6), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(got, _brute_prefill(q, k, v, pos, lens, 0.6, True), rtol=1e-12, atol=1e-13)
    mask = (rng.random((B, 16)) < 0.6).astype(np.uint8)
    got_m = A.prefill(q, k, v, pos, lens, 0.6, key_mask=mask)
    np.testing.assert_allclose(got_m, _brute_prefill(q, k, v, pos, lens, 0.6, True, key_mask=mask),
                               rtol=1e-12, atol=1e-13)


def _prefix_case(rng):
    B, Hq, Hkv, N, d = 2, 4, 2, 5, 4
    pos = [7, 11]
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    pk = [rng.standard_normal((Hkv, 16, d)) for _ in range(B)]
    pv = [rng.standard_normal((Hkv, 16, d)) for _ in range(B)]
    lens = [5, 3]
    # a mask whose absolute and relative (s - P) readings differ
    mask = (rng.random((B, 20)) < 0.55).astype(np.uint8)
    for b in range(B):
        mask[b, pos[b]] = 1
        assert any(mask[b, s] != mask[b, s - pos[b]] for s in range(pos[b], pos[b] + lens[b]))
    return q, k, v, pk, pv, pos, lens, mask


@pytest.mark.parametrize("causal", [True, False])
def test_prefill_prefix_key_mask_is_absolute(causal):
    """attend_prefix with a key mask: the mask is read at the absolute key
    position ([P4] "Causal mask and future positions": position IDs are
    absolute token positions), for prefix and new keys alike."""
    rng = np.random.default_rng(74)
    q, k, v, pk, pv, pos, lens, mask = _prefix_case(rng)
    got = A.prefill(q, k, v, pos, lens, 0.5, causal=causal, key_mask=mask,
                    prefix_k=pk, prefix_v=pv, attend_prefix=True)
    want = _brute_prefill(q, k, v, pos, lens, 0.5, causal, key_mask=mask,
                          prefix_k=pk, prefix_v=pv, attend_prefix=True)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_prefill_pins_catch_planted_slips():
    """The brute-force comparison above is strong enough to catch the slips it
    guards against, planted here in copies of the oracle's inputs/outputs:
    a key mask read at the relative index s - P, a padded row that is not
    zeroed, and a causal test with the wrong sign."""
    rng = np.random.default_rng(74)
    q, k, v, pk, pv, pos, lens, mask = _prefix_case(rng)
    want = _brute_prefill(q, k, v, pos, lens, 0.5, True, key_mask=mask,
                          prefix_k=pk, prefix_v=pv, attend_prefix=True)
    # relative indexing of the mask = an absolute mask shifted by P
    rel = np.zeros_like(mask)
    for b in range(2):
        rel[b, pos[b]:] = mask[b, :mask.shape[1] - pos[b]]
    slip = A.prefill(q, k, v, pos, lens, 0.5, key_mask=rel, prefix_k=pk, prefix_v=pv, attend_prefix=True)
    assert np.abs(slip - want).max() > 1e-3
    # a padded row left unzeroed (the row computed as if it were real)
    q2, k2, v2, m2 = _padded_batch(np.random.default_rng(70))
    ref = _brute_prefill(q2, k2, v2, [0, 0], [3, 3], 0.4, True, key_mask=m2)
    unzeroed = A.prefill(q2, k2, v2, [0, 0], [5, 5], 0.4, key_mask=m2)
    assert np.abs(unzeroed - ref).max() > 1e-3
    # the causal direction flipped (future allowed, past blocked)
    flipped = A.sdpa(q2[0, 0, :3], k2[0, 0, :3], v2[0, 0, :3], A.causal_allow(3).T, 0.4)
    assert np.abs(flipped - ref[0, 0, :3]).max() > 1e-3


def test_gqa_equals_mha_with_repeated_kv_heads():
    """[P2] "(2) GQA": several query heads share one KV head.  GQA over Hkv
    heads == MHA whose KV heads are the shared heads repeated per group
    (query head h -> KV head h // G)."""
    rng = np.random.default_rng(43)
    B, Hq, Hkv, cap, d = 2, 8, 2, 30, 8
    G = Hq // Hkv
    q = rng.standard_normal((B, Hq, d))
    ks, vs = _rand_cache(rng, B, Hkv, cap, d)
    lens = [30, 17]
    gqa = A.decode(q, ks, vs, lens, 0.3)
    mha = A.decode(q, [np.repeat(x, G, axis=0) for x in ks], [np.repeat(x, G, axis=0) for x in vs], lens, 0.3)
    np.testing.assert_array_equal(gqa, mha)
    # and a wrong mapping (h % Hkv) gives a different answer on this data
    wrong = A.decode(q, [np.tile(x, (G, 1, 1)) for x in ks], [np.tile(x, (G, 1, 1)) for x in vs], lens, 0.3)
    assert np.abs(wrong - gqa).max() > 1e-3


def test_decode_key_mask_and_length_bound():
    rng = np.random.default_rng(44)
    B, H, cap, d = 2, 2, 20, 4
    q = rng.standard_normal((B, H, d))
    ks, vs = _rand_cache(rng, B, H, cap, d)
    mask = (rng.random((B, cap)) < 0.6).astype(np.uint8)
    mask[:, 0] = 1
    lens = [13, 20]
    got = A.decode(q, ks, vs, lens, 0.5, key_mask=mask)
    for b in range(B):
        for h in range(H):
            keep = np.nonzero(mask[b, :lens[b]])[0]
            w = scipy.special.softmax(0.5 * ks[b][h][keep] @ q[b, h])
            np.testing.assert_allclose(got[b, h], w @ vs[b][h][keep], rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- codec ---

def test_e4m3_decode_all_codes_matches_library():
    codes = np.arange(256, dtype=np.uint8)
    mine = codec.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(mine[ok], lib[ok])
    assert np.isnan(mine[0x7F]) and np.isnan(mine[0xFF]) and np.isnan(mine).sum() == 2


def test_e4m3_spec_constants():
    """OCP 8-bit floating point spec, E4M3: max normal 448 = S.1111.110,
    min normal 2^-6 = S.0001.000, min subnormal 2^-9 = S.0000.001."""
    assert codec.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert codec.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6
    assert codec.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert codec.e4m3_decode(np.array([0xFE]))[0] == -448.0


def test_e4m3_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = codec.e4m3_decode(codes).astype(np.float32)
    np.testing.assert_array_equal(codec.e4m3_encode_quotient(vals), codes)


def test_e4m3_encode_matches_library_in_range_and_saturates():
    rng = np.random.default_rng(50)
    x = np.concatenate([rng.standard_normal(100000) * 40, rng.standard_normal(10000) * 1e-3,
                        np.array([464.0, -464.0, 465.0, 1e6, -1e30, np.inf, -np.inf, 0.0, -0.0])]).astype(np.float32)
    mine = codec.e4m3_encode_quotient(x)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    inr = np.abs(x) <= 448.0
    np.testing.assert_array_equal(mine[inr], lib[inr])
    big = np.abs(x) > 448.0
    np.testing.assert_array_equal(mine[big], np.where(x[big] < 0, 0xFE, 0x7E).astype(np.uint8))
    assert codec.e4m3_encode_quotient(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_ties_go_to_even():
    # 1.0 (0x38) and 1.125 (0x39): midpoint 1.0625 -> even code 0x38;
    # 1.125 and 1.25 (0x3A): midpoint 1.1875 -> 0x3A.
    got = codec.e4m3_encode_quotient(np.array([1.0625, 1.1875, -1.0625, 2 ** -10, 3 * 2 ** -10], np.float32))
    np.testing.assert_array_equal(got, np.array([0x38, 0x3A, 0xB8, 0x00, 0x02], np.uint8))


def test_e4m3_quantize_divides_in_fp32():
    x = np.array([3.0, -7.5, 100.0], np.float32)
    s = np.float32(1.7)
    want = codec.e4m3_encode_quotient((x / s).astype(np.float32))
    np.testing.assert_array_equal(codec.e4m3_quantize(x, s), want)


def test_bf16_bits_decode():
    vals = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 65280.0], np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    np.testing.assert_array_equal(codec.bf16_bits_to_f64(bits), vals.astype(np.float64))
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(codec.bf16_bits_to_f64(bits), lib)


# ----------------------------------------------------------------- cache ---

def test_cache_bytes_printed_examples():
    rows = _load_rows("kv_cache_bytes.txt")
    assert len(rows) >= 8
    for r in rows:
        args = [int(x) for x in r[:6]]
        assert C.cache_bytes(*args) == int(r[6]), r[7]


def test_op_counts_printed_example():
    """[P1] "Build it", Step 3: 100 generated tokens cost 5050 attention
    computations naively and 100 with the cache."""
    assert C.op_counts(100) == (5050, 100)


def test_sequence_store_append_contract():
    """[P4] "Position IDs and the append contract": appending at a position
    other than the stored length is an error."""
    st = C.SequenceStore(2, 2, 4)
    st.store(0, 0, np.ones((2, 3, 4)), np.zeros((2, 3, 4)))
    assert st.stored(0) == 3 and st.stored(1) == 0
    with pytest.raises(ValueError):
        st.store(0, 5, np.ones((2, 1, 4)), np.ones((2, 1, 4)))
    with pytest.raises(ValueError):
        st.store(1, 1, np.ones((2, 1, 4)), np.ones((2, 1, 4)))
    st.store(0, 3, 2 * np.ones((2, 1, 4)), np.ones((2, 1, 4)))
    k, v = st.head(0, 1)
    assert k.shape == (4, 4) and k[3, 0] == 2.0 and v[3, 0] == 1.0 and v[0, 0] == 0.0


def test_predict_append_paged_roundtrip_and_canaries():
    """Append through a permuted block table, read back through the table:
    the logical rows come back bit-exact and untouched slots keep their bytes."""
    rng = np.random.default_rng(60)
    B, Hkv, d, nblk = 3, 2, 8, 12
    perm = rng.permutation(nblk)
    table = perm[:B * 4].reshape(B, 4)
    pool_k = rng.integers(0, 2 ** 16, (nblk, Hkv, 16, d)).astype(np.uint16)
    pool_v = rng.integers(0, 2 ** 16, (nblk, Hkv, 16, d)).astype(np.uint16)
    pos = np.array([0, 15, 33])
    n = 5
    kn = rng.integers(0, 2 ** 16, (B, Hkv, n, d)).astype(np.uint16)
    vn = rng.integers(0, 2 ** 16, (B, Hkv, n, d)).astype(np.uint16)
    nk, nv = C.predict_append(pool_k, pool_v, kn, vn, pos, n, True, table)
    written = np.zeros((nblk, Hkv, 16), bool)
    for b in range(B):
        rows_k = C.gather_sequence(nk, True, b, 0, pos[b] + n, table)
        np.testing.assert_array_equal(rows_k[pos[b]:], kn[b, 0])
        rows_v = C.gather_sequence(nv, True, b, 1, pos[b] + n, table)
        np.testing.assert_array_equal(rows_v[pos[b]:], vn[b, 1])
        for i in range(n):
            p = pos[b] + i
            written[table[b][p // 16], :, p % 16] = True
    np.testing.assert_array_equal(nk[~written], pool_k[~written])
    np.testing.assert_array_equal(nv[~written], pool_v[~written])


def test_predict_append_fp8_uses_per_head_scale():
    rng = np.random.default_rng(61)
    B, Hkv, d = 1, 2, 4
    cache = np.zeros((B, Hkv, 8, d), np.uint8)
    x = rng.standard_normal((B, Hkv, 1, d)).astype(np.float32)
    bits = x.view(np.uint32)
    scales = np.array([0.5, 2.0], np.float32)
    nk, _ = C.predict_append(cache, cache, bits, bits, [3], 1, False, in_dtype=C.F32,
                             cache_dtype=C.FP8_E4M3, k_scale=scales, v_scale=scales)
    for g in range(2):
        want = torch.from_numpy(x[0, g, 0] / scales[g]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        np.testing.assert_array_equal(nk[0, g, 3], want)
        deq = C.to_f64(nk[0, g, 3], C.FP8_E4M3, scales[g])
        assert np.abs(deq - x[0, g, 0]).max() <= 0.0625 * scales[g] * 4


def test_beam_reorder_printed_example():
    """[P4] "Batch and beam reorder": rows [A0, A1, B0] reordered to
    [B0, A1, A0] by the permutation [2, 1, 0]."""
    assert C.beam_reorder(["A0", "A1", "B0"], [2, 1, 0]) == ["B0", "A1", "A0"]
