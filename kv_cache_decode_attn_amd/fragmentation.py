"""Fragmentation study: contiguous max-length reservation versus 16-token
paging, run on the library's host block pool (kvattn_pool_*).

"KV Cache, Flash Attention and Inference Optimization" (factory.pai-world.com),
section "Exercises" (hard): a toy PagedAttention with 16-token blocks and a
free list, blocks returned when a sequence ends, many variable-length chat
completions simulated, fragmentation compared with contiguous allocation.
"KV Cache Fully Explained" (techblog.paldyn.com), section "(4) PagedAttention":
a contiguous cache reserves the maximum sequence length per request up front,
which paging avoids; requests with one system prompt share its blocks
(copy-on-write).

Schedule: requests are admitted in order into at most `slots` concurrent
sequences.  In each step a newly admitted request stores its prompt, every
active sequence appends one generated token, the memory is measured, and the
sequences that have generated their last token finish.  Paged memory is what
the pool has handed out (blocks in use x 16 positions); contiguous memory is
max_len positions per active sequence.  The metric is reserved-but-unused
bytes: reserved positions minus stored positions, times the bytes one
position takes in every layer's K and V.

    python -m kv_cache_decode_attn_amd.fragmentation [--n 1000] [--slots 64]
"""
import argparse
import json

import numpy as np

from . import api, synth

BLOCK = api.BLOCK_TOKENS


def _blocks(n):
    return -(-int(n) // BLOCK)


def run(prompt_lens, output_lens, slots, max_len, shared_prefix=0):
    """Drive the schedule on a kvattn pool.  Returns a dict of per-step
    int64 arrays (active sequences, live_tokens, paged_reserved and
    contiguous_reserved positions) and the number of copy-on-write block
    copies the pool asked for."""
    mb = _blocks(max_len)
    pool = api.BlockPool(slots * mb + mb)
    tables = np.full((slots, mb), -1, dtype=np.int32)
    cur = np.zeros(slots, dtype=np.int32)
    new = np.zeros(slots, dtype=np.int32)
    length = np.zeros(slots, dtype=np.int64)
    generated = np.zeros(slots, dtype=np.int64)
    request = np.full(slots, -1, dtype=np.int64)
    root = np.full(mb, -1, dtype=np.int32)
    if shared_prefix:
        # the shared prompt prefix, stored once
        pool.prepare_append(root[None, :], np.zeros(1, np.int32), np.array([shared_prefix], np.int32))
    out = {"active": [], "live_tokens": [], "paged_reserved": [], "contiguous_reserved": []}
    copies = 0
    nxt, n = 0, len(prompt_lens)
    while True:
        free = [s for s in range(slots) if request[s] < 0]
        for s in free:
            if nxt >= n:
                break
            request[s] = nxt
            generated[s] = 0
            if shared_prefix:
                pool.fork(root, shared_prefix, tables[s])
                length[s] = shared_prefix
            else:
                length[s] = 0
            nxt += 1
        act = request >= 0
        if not act.any():
            break
        # new requests store their prompt and first token, the others one token
        cur[:] = np.where(act, length, 0)
        first = act & (generated == 0)
        new[:] = np.where(first, np.asarray(prompt_lens)[np.maximum(request, 0)] + 1, cur + act)
        cs, _ = pool.prepare_append(tables, cur, new)
        copies += len(cs)
        length[act] = new[act]
        generated[act] += 1
        out["active"].append(int(act.sum()))
        out["live_tokens"].append(int(length[act].sum()))
        out["paged_reserved"].append((pool.num_blocks - pool.num_free()) * BLOCK)
        out["contiguous_reserved"].append(int(act.sum()) * int(max_len))
        for s in np.nonzero(act)[0]:
            if generated[s] >= int(output_lens[request[s]]):
                pool.free_seq(tables[s], int(length[s]))
                request[s] = -1
    if shared_prefix:
        pool.free_seq(root, shared_prefix)
    leaked = pool.num_blocks - pool.num_free()
    if leaked:
        raise RuntimeError("%d blocks still held after every sequence finished" % leaked)
    res = {k: np.asarray(v, dtype=np.int64) for k, v in out.items()}
    return res, copies


def summary(trace, bytes_per_position):
    """Mean and peak reserved and reserved-but-unused bytes of both schemes.

    Live positions count a shared prefix once per request (as a contiguous
    cache stores it), so with prefix sharing paging can reserve less than
    the live positions and its "unused" figure goes negative."""
    live = trace["live_tokens"]
    r = {"steps": int(len(live)), "bytes_per_position": int(bytes_per_position)}
    for name in ("paged", "contiguous"):
        res = trace[name + "_reserved"]
        unused = res - live
        r[name] = {
            "reserved_mean_bytes": float(res.mean() * bytes_per_position),
            "reserved_peak_bytes": int(res.max() * bytes_per_position),
            "unused_mean_bytes": float(unused.mean() * bytes_per_position),
            "unused_peak_bytes": int(unused.max() * bytes_per_position),
            "unused_fraction_of_reserved": float(unused.sum() / max(res.sum(), 1)),
        }
    r["live_mean_bytes"] = float(live.mean() * bytes_per_position)
    r["reserved_ratio_contiguous_over_paged"] = float(trace["contiguous_reserved"].sum() /
                                                      max(trace["paged_reserved"].sum(), 1))
    return r


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--n", type=int, default=1000, help="chat completions")
    ap.add_argument("--slots", type=int, default=64, help="concurrent sequences")
    ap.add_argument("--max-len", type=int, default=4096)
    ap.add_argument("--shared-prefix", type=int, default=0)
    ap.add_argument("--seed", type=int, default=11)
    # bytes of one position's K and V over all layers: Llama-3-8B shape, bf16
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--kv-heads", type=int, default=8)
    ap.add_argument("--head-dim", type=int, default=128)
    ap.add_argument("--elem-bytes", type=int, default=2)
    a = ap.parse_args(argv)
    p, o = synth.chat_lengths(a.n, (a.seed, synth.T_LENS), max_len=a.max_len, prefix=a.shared_prefix)
    trace, copies = run(p, o, a.slots, a.max_len, a.shared_prefix)
    bpp = api.cache_bytes(a.layers, 1, a.kv_heads, 1, a.head_dim, a.elem_bytes)
    s = summary(trace, bpp)
    s["copy_on_write_copies"] = copies
    s["config"] = {"n": a.n, "slots": a.slots, "max_len": a.max_len, "shared_prefix": a.shared_prefix,
                   "seed": a.seed, "prompt_mean": float(p.mean()), "output_mean": float(o.mean())}
    print(json.dumps(s, indent=1))
    return s


if __name__ == "__main__":
    main()
