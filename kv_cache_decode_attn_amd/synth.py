"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.  Pure data generation: no attention arithmetic lives here.

Seeds are tuples (workload id, tensor id, layer), so every tensor of every
workload is reproducible on its own.  Small inputs are drawn with numpy's
PCG64 on the host; large ones with torch's Philox generator on the device
(the bytes are then copied back wherever an oracle needs them).  Normals are
drawn in fp32 and rounded to the storage type with round-to-nearest-even.
"""
import numpy as np
import torch

# tensor ids inside a seed tuple
T_Q, T_K, T_V, T_KNEW, T_VNEW, T_LENS, T_PERM, T_SCALE, T_MASK = range(9)


def rng(*seed):
    return np.random.default_rng([0] + [int(s) for s in seed])


def normal(shape, seed, dtype=torch.bfloat16, device="cpu", std=1.0):
    """N(0, std^2) values rounded to `dtype`, drawn on the host (small sizes)."""
    x = rng(*seed).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x = x * np.float32(std)
    return torch.from_numpy(x).to(dtype).to(device)


def normal_device(shape, seed, dtype=torch.bfloat16, device="cuda", std=1.0, out=None):
    """N(0, std^2) values rounded to `dtype`, drawn on the device (large sizes)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([0] + [int(s) for s in seed]).generate_state(1)[0]))
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=device)
    # fill in slabs so that the fp32 temporary stays small
    flat = out.view(-1)
    slab = 1 << 26
    for s in range(0, flat.numel(), slab):
        n = min(slab, flat.numel() - s)
        tmp = torch.randn(n, generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        flat[s:s + n].copy_(tmp)
    return out


def uniform_lengths(n, lo, hi, seed):
    """n integers uniform on [lo, hi] inclusive."""
    return rng(*seed).integers(lo, hi + 1, size=n).astype(np.int32)


def block_table(blocks_per_seq, max_blocks, seed, num_blocks=None):
    """Block table whose physical ids are a seeded permutation of
    range(num_blocks) handed out in (sequence, logical block) order.
    Unused entries are -1.  Returns (table int32 [B, max_blocks], num_blocks)."""
    blocks_per_seq = [int(x) for x in blocks_per_seq]
    total = sum(blocks_per_seq)
    if num_blocks is None:
        num_blocks = total
    perm = rng(*seed).permutation(num_blocks).astype(np.int32)
    table = np.full((len(blocks_per_seq), max_blocks), -1, dtype=np.int32)
    k = 0
    for b, nb in enumerate(blocks_per_seq):
        table[b, :nb] = perm[k:k + nb]
        k += nb
    return table, num_blocks


def blocks_for(length, block_tokens=16):
    return (int(length) + block_tokens - 1) // block_tokens


def padding_mask(lengths, width):
    """uint8 [B, width]: 1 for positions < length (right padding blocked)."""
    lengths = np.asarray(lengths)
    return (np.arange(width)[None, :] < lengths[:, None]).astype(np.uint8)


def random_mask(shape, keep, seed):
    return (rng(*seed).random(shape) < keep).astype(np.uint8)


def fp8_scales(n, seed, lo=0.5, hi=2.0):
    """Per-head fp32 dequantisation scales drawn from U[lo, hi]."""
    return rng(*seed).uniform(lo, hi, size=n).astype(np.float32)


def chat_lengths(n, seed, max_len=4096, prefix=0, prompt_median=256.0, output_median=200.0, sigma=1.0):
    """Prompt and completion lengths (int64 [n] each) of n synthetic chat
    completions: log-normal lengths with the given medians and log-space
    sigma, rounded, then clipped so that every prompt holds the shared
    prefix plus at least one token, every completion has at least one
    token, and prompt + completion <= max_len."""
    r = rng(*seed)
    p = np.rint(prompt_median * np.exp(sigma * r.standard_normal(n))).astype(np.int64)
    o = np.rint(output_median * np.exp(sigma * r.standard_normal(n))).astype(np.int64)
    p = np.clip(p, prefix + 1, max_len - 1)
    o = np.clip(o, 1, max_len - p)
    return p, o
