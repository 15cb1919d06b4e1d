"""Paged-cache bookkeeping: batch/beam reorder, physical-block copies, a
reference block pool (free list, reference counts, copy-on-write) and the
reserved-memory closed forms of contiguous versus 16-token paged allocation.

Test infrastructure (see the package docstring).  Sources are cited by the
short keys [P1]..[P4] defined there.  Every result here is integer or byte
work: the library must match it exactly.

Block tables are int32 arrays [rows, max_blocks]; entry j of a row names the
physical block holding positions 16j .. 16j+15 of that sequence, -1 = none.
A row of length L uses its first ceil(L / 16) entries.
"""
import numpy as np

BLOCK_TOKENS = 16


def blocks_for(length):
    """Blocks a sequence of `length` positions occupies: ceil(length / 16)."""
    length = int(length)
    return -(-length // BLOCK_TOKENS)


# ------------------------------------------------------- batch/beam reorder ---

def reorder_rows(table, lens, perm):
    """Block table and lengths after a batch/beam reorder of a paged cache.

    [P4] section "Batch and beam reorder": when the beam order changes, the
    cache rows must follow the same permutation, new row i = old row perm[i]
    ([A0, A1, B0] -> [B0, A1, A0] with perm [2, 1, 0]).  For a paged cache a
    row is its block-table row plus its length, so the reorder moves ids, not
    K/V bytes.  A perm entry outside [0, rows) gives an empty row (all -1,
    length 0): our reading of an invalid index.
    """
    table = np.asarray(table, dtype=np.int32)
    rows, mb = table.shape
    out_t = np.full((len(perm), mb), -1, dtype=np.int32)
    out_l = np.zeros(len(perm), dtype=np.int32)
    for i, p in enumerate(perm):
        p = int(p)
        if 0 <= p < rows:
            out_t[i] = table[p]
            if lens is not None:
                out_l[i] = int(lens[p])
    return out_t, (out_l if lens is not None else None)


def reorder_contiguous(src, dst, perm, lens=None):
    """Contiguous cache rows after a batch/beam reorder ([P4] section "Batch
    and beam reorder": gather the cache tensor rows with the beam
    permutation).

    src, dst: raw storage [rows, Hkv, capacity, d].  Row i of the result
    holds, at positions < L, the bytes of src row perm[i], with
    L = min(lens[perm[i]], capacity) (all `capacity` positions when lens is
    None); its other positions keep dst's bytes.  A perm entry outside
    [0, src rows) leaves dst row i unchanged and gives length 0.  Returns
    (new dst array, new lengths or None).
    """
    out = np.array(dst, copy=True)
    cap = src.shape[2]
    new_l = np.zeros(len(perm), dtype=np.int32)
    for i, p in enumerate(perm):
        p = int(p)
        if not 0 <= p < src.shape[0]:
            continue
        n = cap if lens is None else max(0, min(int(lens[p]), cap))
        out[i, :, :n] = src[p, :, :n]
        if lens is not None:
            new_l[i] = int(lens[p])
    return out, (new_l if lens is not None else None)


# ----------------------------------------------------------- block copies ---

def copy_blocks(pool, src, dst):
    """Physical pool after copy-on-write block copies.

    [P2] section "(4) PagedAttention", prefix sharing: requests with a
    common prefix point at the same physical blocks, and a shared block is
    copied before one of its holders writes into it.  pool: raw storage
    [num_blocks, ...]; for each pair i, block dst[i] receives the bytes of
    block src[i].  Pairs with an id outside [0, num_blocks) are skipped.
    The pairs are taken as simultaneous: every source is read before any
    destination is written (the library requires destinations that are
    distinct and not sources, where order cannot matter).
    """
    before = np.array(pool, copy=True)
    out = np.array(pool, copy=True)
    n = pool.shape[0]
    for s, d in zip(src, dst):
        s, d = int(s), int(d)
        if 0 <= s < n and 0 <= d < n:
            out[d] = before[s]
    return out


# ------------------------------------------------------ reference block pool ---

class NoSpace(Exception):
    """The pool has fewer free blocks than the request needs."""


class BadBlock(Exception):
    """A table names a block that is out of range or not allocated."""


class RefPool:
    """A fixed set of physical blocks with a free list and reference counts.

    [P1] section "Exercises" (hard): a toy PagedAttention splits the cache
    into fixed 16-token blocks, keeps a free list, and returns a sequence's
    blocks to the pool when it ends.  [P1] section "PagedAttention": the page
    table lets parallel branches (beam search, parallel sampling) share KV
    blocks.  [P2] section "(4) PagedAttention": shared prefix blocks are
    copy-on-write.

    Our readings (the pages fix none of these): a block's reference count is
    the number of table rows that name it, it is free at count 0, and the
    free list hands out the lowest free id first.  Every operation is
    all-or-nothing: on NoSpace or BadBlock the pool and the tables are left
    as they were.
    """

    def __init__(self, num_blocks):
        self.ref = [0] * int(num_blocks)

    @property
    def num_blocks(self):
        return len(self.ref)

    def num_free(self):
        return sum(1 for r in self.ref if r == 0)

    def _check_held(self, ids):
        held = {}
        for b in ids:
            b = int(b)
            if not 0 <= b < len(self.ref):
                raise BadBlock(b)
            held[b] = held.get(b, 0) + 1
            if held[b] > self.ref[b]:
                raise BadBlock(b)

    def alloc(self, n):
        free = [i for i, r in enumerate(self.ref) if r == 0]
        if len(free) < n:
            raise NoSpace(n)
        ids = free[:n]
        for i in ids:
            self.ref[i] = 1
        return ids

    def retain(self, ids):
        for b in ids:
            if not 0 <= int(b) < len(self.ref) or self.ref[int(b)] == 0:
                raise BadBlock(int(b))
        for b in ids:
            self.ref[int(b)] += 1

    def release(self, ids):
        self._check_held(ids)
        for b in ids:
            self.ref[int(b)] -= 1

    def fork(self, src_row, length, max_blocks):
        """Row sharing the first ceil(length/16) blocks of src_row (prefix
        sharing / a new beam or sample branch)."""
        nb = blocks_for(length)
        used = [int(x) for x in src_row[:nb]]
        self.retain(used)
        row = [-1] * max_blocks
        row[:nb] = used
        return row

    def free_seq(self, row, length):
        """Return the blocks of a finished sequence; the row becomes empty."""
        nb = blocks_for(length)
        self.release(row[:nb])
        row = list(row)
        row[:nb] = [-1] * nb
        return row

    def prepare_append(self, tables, cur_lens, new_lens):
        """Make positions cur_lens[b] .. new_lens[b]-1 of every row writable.

        Rows are handled in order.  A partially filled last block
        (cur_len % 16 != 0, new_len > cur_len) that another row also names
        is replaced by a fresh block, recorded as a copy pair (old, new) for
        the device copy that must run before the write; the old block loses
        one reference.  Entries ceil(cur_len/16) .. ceil(new_len/16)-1 get
        fresh blocks.  Returns (new tables, [(src, dst), ...]).
        """
        saved = list(self.ref)
        tables = [list(map(int, r)) for r in tables]
        pairs = []
        try:
            for b, row in enumerate(tables):
                cur, new = int(cur_lens[b]), int(new_lens[b])
                if new < cur or blocks_for(new) > len(row):
                    raise BadBlock(-1)
                self._check_held(row[:blocks_for(cur)])
                if new > cur and cur % BLOCK_TOKENS:
                    j = cur // BLOCK_TOKENS
                    old = row[j]
                    if self.ref[old] > 1:
                        (fresh,) = self.alloc(1)
                        self.ref[old] -= 1
                        row[j] = fresh
                        pairs.append((old, fresh))
                for j in range(blocks_for(cur), blocks_for(new)):
                    (row[j],) = self.alloc(1)
        except (NoSpace, BadBlock):
            self.ref = saved
            raise
        return tables, pairs

    def reorder(self, tables, lens, perm):
        """Host side of the beam reorder: the rows of reorder_rows, with the
        references moved along (rows no longer named lose their blocks, rows
        named twice share them)."""
        new_t, new_l = reorder_rows(tables, lens, perm)
        saved = list(self.ref)
        try:
            for i in range(len(perm)):
                self.retain(new_t[i, :blocks_for(new_l[i])])
            for r in range(len(tables)):
                self.release(np.asarray(tables[r])[:blocks_for(lens[r])])
        except BadBlock:
            self.ref = saved
            raise
        return new_t, new_l


# ------------------------------------------------- fragmentation closed forms ---

def reserved_tokens_paged(length):
    """Positions a 16-token paged cache reserves for one sequence:
    16 * ceil(L / 16) ([P1] section "PagedAttention": blocks are allocated
    as needed, so at most one partly filled block per sequence)."""
    return BLOCK_TOKENS * blocks_for(length)


def reserved_tokens_contiguous(length, max_len):
    """Positions a contiguous cache reserves for one sequence: the maximum
    sequence length, whatever the sequence's own length ([P2] section
    "(4) PagedAttention": the traditional cache pre-reserves max-length
    contiguous memory)."""
    del length
    return int(max_len)


def fragmentation_trace(prompt_lens, output_lens, slots, max_len, shared_prefix=0):
    """Per-step memory of a continuous-batching run of chat completions.

    [P1] section "Exercises" (hard): simulate many variable-length chat
    completions and compare the fragmentation of contiguous allocation with
    16-token paging.  Schedule (our reading): requests are admitted in order
    into at most `slots` concurrent sequences; in each step every admitted
    request first gets its prompt (prefill) if it is new, then every active
    sequence appends one generated token, the memory is measured, and
    sequences that have generated output_lens[r] tokens finish and release
    their memory.

    shared_prefix = S > 0: every prompt starts with the same S tokens, held
    once by a root sequence whose blocks the requests share
    ([P2] section "(4) PagedAttention", prefix sharing); a request of length
    L then holds its own blocks for positions >= 16 * floor(S / 16).  The
    contiguous cache stores the prefix in every row.

    Returns a dict of int64 arrays, one entry per step: active, live_tokens
    (sum of lengths), paged_reserved and contiguous_reserved (positions).
    """
    n = len(prompt_lens)
    queue = 0
    active = []  # [length, generated, request]
    steps = {"active": [], "live_tokens": [], "paged_reserved": [], "contiguous_reserved": []}
    root_blocks = blocks_for(shared_prefix) if shared_prefix else 0
    shared_full = shared_prefix // BLOCK_TOKENS
    while queue < n or active:
        while queue < n and len(active) < slots:
            active.append([int(prompt_lens[queue]), 0, queue])
            queue += 1
        for s in active:
            s[0] += 1
            s[1] += 1
        lens = [s[0] for s in active]
        steps["active"].append(len(active))
        steps["live_tokens"].append(sum(lens))
        if shared_prefix:
            paged = BLOCK_TOKENS * (root_blocks + sum(blocks_for(L) - shared_full for L in lens))
        else:
            paged = sum(reserved_tokens_paged(L) for L in lens)
        steps["paged_reserved"].append(paged)
        steps["contiguous_reserved"].append(sum(reserved_tokens_contiguous(L, max_len) for L in lens))
        active = [s for s in active if s[1] < int(output_lens[s[2]])]
    return {k: np.asarray(v, dtype=np.int64) for k, v in steps.items()}
