"""Scaled dot-product attention against a KV cache, by its definition, in fp64.

Test infrastructure (see the package docstring).  Sources are cited by the
short keys [P1]..[P4] defined there.

Readings taken where the pages leave a step open (each is also listed in
the design notes):
  * mask direction: a uint8 "allow" value, 1 = the query may read the key
    ([P4] section "Causal mask and future positions" prints the allow matrix
    with 1 = allowed);
  * a forbidden key is excluded outright - weight exactly 0, its K/V never
    read - which is the limit of adding a large negative number
    ([P4] section "State of scaled dot-product attention");
  * a query row with no allowed key outputs 0 ([P4] section
    "Implementation and verification procedure" says such rows give NaN or a
    uniform distribution depending on the implementation; we fix one);
  * the score scale is 1/sqrt(d_head) ([P3] section "Self-Attention",
    [P4] section "State of scaled dot-product attention"); it is passed in;
  * grouped-query attention: query head h reads KV head h // (Hq / Hkv)
    ([P2] section "(2) GQA": several query heads share one KV head).
"""
import numpy as np


def causal_allow(n):
    """Causal allow matrix for n positions, 0-based: query t reads key s iff s <= t.

    [P4] section "Causal mask and future positions": the diagonal and
    everything left of it is allowed, the future (right) is blocked.
    """
    t = np.arange(n)[:, None]
    s = np.arange(n)[None, :]
    return (s <= t).astype(np.uint8)


def sdpa(q, K, V, allow, scale):
    """Plain masked scaled dot-product attention for one head.

    [P4] section "State of scaled dot-product attention":
        scores = Q K^T / sqrt(d_head); weights = softmax(scores + mask);
        output = weights V.
    q: [n_q, d], K: [n_k, d], V: [n_k, dv], allow: [n_q, n_k] (nonzero = may
    attend).  Keys not allowed are dropped before the softmax (weight 0); a
    row with nothing allowed returns zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    allow = np.asarray(allow).astype(bool)
    out = np.zeros((q.shape[0], V.shape[1]), dtype=np.float64)
    for t in range(q.shape[0]):
        idx = np.nonzero(allow[t])[0]
        if idx.size == 0:
            continue
        z = (K[idx] @ q[t]) * scale
        e = np.exp(z - z.max())
        out[t] = (e / e.sum()) @ V[idx]
    return out


def attention_weights(q, K, allow, scale):
    """The softmax weights of sdpa as a dense [n_q, n_k] matrix (0 where forbidden)."""
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    allow = np.asarray(allow).astype(bool)
    w = np.zeros((q.shape[0], K.shape[0]), dtype=np.float64)
    for t in range(q.shape[0]):
        idx = np.nonzero(allow[t])[0]
        if idx.size == 0:
            continue
        z = (K[idx] @ q[t]) * scale
        e = np.exp(z - z.max())
        w[t, idx] = e / e.sum()
    return w


def softmax_state(z, V):
    """Unnormalised softmax state (m, l, o) of a set of scaled scores z and
    their value rows V: m = max z, l = sum exp(z - m), o = sum exp(z - m) v.
    An empty set has the state (-inf, 0, 0)."""
    z = np.asarray(z, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    if z.size == 0:
        return (-np.inf, 0.0, np.zeros(V.shape[1], dtype=np.float64))
    m = float(z.max())
    e = np.exp(z - m)
    return (m, float(e.sum()), e @ V)


def combine_states(a, b):
    """State of the union of two disjoint key sets from their two states:
    both are brought to the common maximum M = max(m_a, m_b) by the factors
    exp(m_a - M) and exp(m_b - M), then l and o add.  [P1] section "Flash
    Attention - tiling trick", numerical trick: keeping the running maximum
    and sum is what makes a tiled softmax exact."""
    ma, la, oa = a
    mb, lb, ob = b
    if mb == -np.inf:
        return a
    if ma == -np.inf:
        return b
    M = max(ma, mb)
    fa, fb = np.exp(ma - M), np.exp(mb - M)
    return (M, la * fa + lb * fb, oa * fa + ob * fb)


def tiled_fold(q, K, V, scale, tile, allow=None):
    """One query against K/V, the keys consumed `tile` at a time: each tile's
    own state (softmax_state of its allowed keys) is folded into the running
    state with combine_states, and the output is o / l at the end - the
    second route to the result of sdpa, which never holds more than one tile
    of scores ([P1] section "Flash Attention - tiling trick"; the pages'
    version of this algorithm has no score scale and no mask, both added
    here).  A query that sees no key returns zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = K.shape[0]
    allow = np.ones(n, dtype=bool) if allow is None else np.asarray(allow).astype(bool)
    state = softmax_state(np.zeros(0), V[:0])
    for lo in range(0, n, tile):
        idx = lo + np.flatnonzero(allow[lo:lo + tile])
        state = combine_states(state, softmax_state((K[idx] @ q) * scale, V[idx]))
    _, l, o = state
    return o / l if l > 0 else o


def split_partials(q, K, V, scale, part, allow=None):
    """Split the keys into consecutive partitions of `part` keys and return,
    per partition, the softmax_state (m, l, o) of its allowed keys: the
    exact-renormalisation identity of [P1] "Flash Attention - tiling trick",
    numerical trick, applied across partitions instead of tiles.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = K.shape[0]
    allow = np.ones(n, dtype=bool) if allow is None else np.asarray(allow).astype(bool)
    parts = []
    for lo in range(0, n, part):
        idx = lo + np.flatnonzero(allow[lo:lo + part])
        parts.append(softmax_state((K[idx] @ q) * scale, V[idx]))
    return parts


def merge_partials(parts):
    """Combine (m, l, o) partition states: M = max m_p, L = sum l_p e^(m_p - M),
    O = sum o_p e^(m_p - M) / L; all partitions empty (L == 0) -> zeros."""
    dv = parts[0][2].shape[0]
    ms = np.array([p[0] for p in parts], dtype=np.float64)
    if not np.isfinite(ms).any():
        return np.zeros(dv)
    M = ms[np.isfinite(ms)].max()
    L = 0.0
    O = np.zeros(dv)
    for m, l, o in parts:
        if m == -np.inf:
            continue
        w = np.exp(m - M)
        L += l * w
        O += o * w
    return O / L if L > 0 else np.zeros(dv)


def decode(q, keys, values, seq_lens, scale, key_mask=None):
    """Single-token decode against a per-layer cache, after the append.

    [P4] section "Prefill and decode stages": the new token's K/V are
    appended first and the new query then attends over the whole cache;
    [P3] section "TO-BE": Q_5 with cache K_1..5, V_1..5 - the token sees
    itself.  seq_lens[b] is therefore the number of keys including the new
    one.

    q:        [B, Hq, d] fp64 query of the new token per head
    keys[b]:  [Hkv, >= seq_lens[b], d] fp64 logical cache of sequence b,
              position-indexed (position s is row s)
    values[b]: same for V
    key_mask: optional [B, >= max(seq_lens)] uint8, 1 = attend; ANDed with
              s < seq_lens[b] ([P4] section "Padding mask and batch length")
    Returns [B, Hq, d] fp64.  Query head h uses KV head h // (Hq / Hkv).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = np.asarray(keys[0]).shape[0]
    G = Hq // Hkv
    out = np.zeros((B, Hq, np.asarray(values[0]).shape[2]), dtype=np.float64)
    for b in range(B):
        ctx = int(seq_lens[b])
        allow = np.ones(ctx, dtype=bool)
        if key_mask is not None:
            allow &= np.asarray(key_mask[b][:ctx]).astype(bool)
        for h in range(Hq):
            g = h // G
            K = np.asarray(keys[b][g][:ctx], dtype=np.float64)
            V = np.asarray(values[b][g][:ctx], dtype=np.float64)
            out[b, h] = sdpa(q[b, h][None, :], K, V, allow[None, :], scale)[0]
    return out


def prefill(q, k_new, v_new, positions, q_lens, scale, causal=True, key_mask=None,
            prefix_k=None, prefix_v=None, attend_prefix=False):
    """Multi-token attention of new tokens (prefill; also chunked prefill when
    a cached prefix is attended).

    [P4] section "Prefill and decode stages": the prompt is processed once and
    every layer stores its K/V; section "Causal mask and future positions"
    and section "Padding mask and batch length" give the two masks, which
    are independent and are ANDed.  [P4] section "Position IDs and the append
    contract": positions are 0-based absolute token positions.

    q:      [B, Hq, N, d] fp64      k_new, v_new: [B, Hkv, N, d] fp64
    positions[b]: absolute position of new token 0 of sequence b
    q_lens[b]:    number of real new tokens (<= N); rows t >= q_lens[b] -> 0
    Query t sits at p_t = positions[b] + t.  Keys are the absolute positions
      s in [0, positions[b] + q_lens[b])            if attend_prefix,
      s in [positions[b], positions[b] + q_lens[b]) otherwise,
    where s < positions[b] is read from prefix_k/prefix_v[b] (position-indexed
    [Hkv, >= positions[b], d]) and s >= positions[b] from the new K/V row
    s - positions[b].  Allowed iff (not causal or s <= p_t) and
    key_mask[b, s] != 0 (when given).
    Returns [B, Hq, N, d] fp64.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k_new.shape[1]
    G = Hq // Hkv
    dv = v_new.shape[3]
    out = np.zeros((B, Hq, N, dv), dtype=np.float64)
    for b in range(B):
        P = int(positions[b])
        n = int(q_lens[b])
        if n == 0:
            continue
        lo = 0 if attend_prefix else P
        key_pos = np.arange(lo, P + n)
        p_t = P + np.arange(n)
        allow = np.ones((n, key_pos.size), dtype=bool)
        if causal:
            allow &= key_pos[None, :] <= p_t[:, None]
        if key_mask is not None:
            allow &= np.asarray(key_mask[b])[key_pos].astype(bool)[None, :]
        for h in range(Hq):
            g = h // G
            new_k = np.asarray(k_new[b, g, :n], dtype=np.float64)
            new_v = np.asarray(v_new[b, g, :n], dtype=np.float64)
            if attend_prefix and P > 0:
                K = np.concatenate([np.asarray(prefix_k[b][g][:P], dtype=np.float64), new_k])
                V = np.concatenate([np.asarray(prefix_v[b][g][:P], dtype=np.float64), new_v])
            else:
                K, V = new_k, new_v
            out[b, h, :n] = sdpa(q[b, h, :n], K, V, allow, scale)
    return out


def full_recompute_last_row(q_all, k_all, v_all, scale):
    """The naive decoder's view of one step: recompute causal attention over
    the whole prefix and keep the last row ([P3] section "AS-IS";
    [P1] section "Problem").  Cached decode must equal it
    ([P4] section "Implementation and verification procedure").
    q_all/k_all/v_all: [n, d] for one head; returns [d]."""
    n = np.asarray(q_all).shape[0]
    return sdpa(q_all, k_all, v_all, causal_allow(n), scale)[-1]
