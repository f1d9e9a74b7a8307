"""Seeded synthetic inputs for the attention workloads.

This module draws random numbers and casts them; it holds none of the
attention arithmetic.  Both sides of every parity check (the fp64 CPU oracle
and the HIP library) take their inputs from here, so neither has to import the
other.

The workloads stand in for the shapes the FlashAttention pages measure on
(BERT-large at sequence 512, GPT-2 small at 1K, Path-X at 16K, Path-256 at 64K
with block sparsity; "FlashAttention: Fast and Memory-Efficient Exact
Attention with IO-Awareness", abstract and §4 Experiments).  No dataset is
read: Q, K, V and dO are iid N(0, 1).
"""
from __future__ import annotations

import math

import torch

# Block-mask granularity: one mask entry covers 128 query rows x 128 key rows.
MASK_BLOCK = 128

# name -> shape and flags.  "frac" is the fraction of off-diagonal mask blocks
# that are kept (diagonal blocks are always kept).
WORKLOADS = {
    "tiny_f32": dict(B=1, H=1, N=128, d=64, dtype="f32", causal=False, mask=False),
    "bert_large": dict(B=16, H=16, N=512, d=64, dtype="bf16", causal=False, mask=False),
    "gpt2_small": dict(B=8, H=12, N=1024, d=64, dtype="bf16", causal=True, mask=False),
    "long_d64": dict(B=1, H=16, N=16384, d=64, dtype="bf16", causal=True, mask=False),
    "long_d128": dict(B=1, H=16, N=16384, d=128, dtype="bf16", causal=True, mask=False),
    "blocksparse_64k": dict(B=1, H=16, N=65536, d=64, dtype="bf16", causal=False, mask=True, frac=0.125),
}

DATA_SEED = 0
MASK_SEED = 1
SAMPLE_SEED = 2


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def make_qkvdo(B: int, H: int, N: int, d: int, dtype: str = "bf16", seed: int = DATA_SEED):
    """Q, K, V, dO as CPU tensors of shape [B, H, N, d].

    Drawn as fp32 randn from one generator in the order Q, K, V, dO, then cast
    once (round-to-nearest-even) to bf16 when dtype == "bf16".
    """
    g = torch.Generator().manual_seed(seed)
    out = []
    for _ in range(4):
        t = torch.randn((B, H, N, d), generator=g, dtype=torch.float32)
        if dtype == "bf16":
            t = t.to(torch.bfloat16)
        elif dtype != "f32":
            raise ValueError(f"dtype {dtype!r}")
        out.append(t)
    return tuple(out)


def num_blocks(N: int) -> int:
    return (N + MASK_BLOCK - 1) // MASK_BLOCK


def make_blockmask(N: int, frac: float = 0.125, seed: int = MASK_SEED) -> torch.Tensor:
    """uint8 [nb, nb] mask, row = query block, column = key block.

    Every diagonal block is kept.  Of the nb*(nb-1) off-diagonal blocks exactly
    floor(frac * nb*(nb-1)) are kept, chosen uniformly without replacement by a
    seeded permutation.
    """
    nb = num_blocks(N)
    m = torch.zeros((nb, nb), dtype=torch.uint8)
    idx = torch.arange(nb)
    m[idx, idx] = 1
    total = nb * (nb - 1)
    keep = int(math.floor(frac * total))
    if keep > 0:
        g = torch.Generator().manual_seed(seed)
        pick = torch.randperm(total, generator=g)[:keep]
        r = pick // (nb - 1)
        c = pick % (nb - 1)
        c = c + (c >= r).to(c.dtype)
        m[r, c] = 1
    return m


def make_random_blockmask(N: int, density: float, seed: int, diagonal: bool = True) -> torch.Tensor:
    """Bernoulli(density) block mask for edge-case tests (rows may be empty
    when diagonal is False)."""
    nb = num_blocks(N)
    g = torch.Generator().manual_seed(seed)
    m = (torch.rand((nb, nb), generator=g) < density).to(torch.uint8)
    if diagonal:
        idx = torch.arange(nb)
        m[idx, idx] = 1
    return m


def sample_rows(B: int, H: int, N: int, count: int = 256, seed: int = SAMPLE_SEED):
    """`count` distinct (b, h, i) triples drawn uniformly from B x H x N."""
    g = torch.Generator().manual_seed(seed)
    total = B * H * N
    count = min(count, total)
    flat = torch.randperm(total, generator=g)[:count]
    flat, _ = torch.sort(flat)
    b = flat // (H * N)
    h = (flat // N) % H
    i = flat % N
    return b, h, i


def workload_inputs(name: str, seed: int = DATA_SEED):
    """(q, k, v, do, scale, causal, blockmask-or-None) for a named workload."""
    w = WORKLOADS[name]
    q, k, v, do = make_qkvdo(w["B"], w["H"], w["N"], w["d"], w["dtype"], seed)
    mask = make_blockmask(w["N"], w.get("frac", 0.125)) if w["mask"] else None
    return q, k, v, do, default_scale(w["d"]), w["causal"], mask
