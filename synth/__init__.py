"""Seeded synthetic looped-model KV and queries.

Shared by the tests, the benchmark and the CPU oracle's inputs; it holds none
of the method's arithmetic, only random draws with the shapes and statistics
of the workloads:

* reference (final-loop) K and V: N(0, 1) scaled per channel by a standard
  deviation drawn from LogNormal(0, 0.5) -- one draw per (layer, head,
  channel), separately for K and V -- to mimic the post-RoPE outlier channels
  the ResidualQuant page shows in its key-magnitude figures (Fig. 2, Fig. 5);
* an earlier loop l: c_l * reference + N(0, sigma_l^2), so loops are similar to
  the final loop, as the page observes (Abstract) and as its Table 1 trend
  suggests (later loops closer to the last-loop reference);
* queries: N(0, 1), one per loop.

Everything is drawn in float32 from a seeded torch.Generator and rounded to
bfloat16.  Tensors come back on `device`; the draw happens on the generator's
device (CPU by default, so that the oracle and the GPU see the same values).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import torch


@dataclass
class Workload:
    name: str
    n_loops: int
    batch: int
    heads: int
    d: int
    g: int
    n_ctx: int
    bits: List[int]                 # per residual loop (length n_loops - 1)
    c: List[float]                  # similarity coefficient per residual loop
    sigma: List[float]              # residual noise std per residual loop
    rotate: int = 1
    layers: int = 1
    steps: int = 0                  # append-decode steps after the prefill
    seed: int = 0
    ref_bits: int = 0               # 0: BF16 reference; 2/4: quantized anchor
    ref_group: int = 0              # the anchor's group size (0: g)
    group_loops: int = 0            # loops per anchor group (0: one group)
    ref_first: int = 0              # 1: first loop of each group is the reference
    alpha_mode: int = 0             # 0 least squares, 1 alpha = 1, 2 norm ratio
    ref_chain: int = 0              # 1: each loop refers to its neighbour towards the reference
    extra: dict = field(default_factory=dict)


# The workloads: a tiny CPU-checkable case, the 8k-context INT2 decode,
# mixed precision with appends, 32k context over 24 layers, the 8k
# peak-batch sweep, and per-loop decode with a quantized anchor.
WORKLOADS = {
    "tiny": Workload("tiny", n_loops=2, batch=1, heads=1, d=64, g=32, n_ctx=128,
                     bits=[2], c=[0.9], sigma=[0.1], rotate=0, seed=0),
    "int2-8k": Workload("int2-8k", n_loops=4, batch=16, heads=16, d=128, g=32, n_ctx=8192,
                        bits=[2, 2, 2], c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1],
                        rotate=1, seed=1),
    "mixed-8k-append": Workload("mixed-8k-append", n_loops=4, batch=64, heads=16, d=128, g=32,
                                n_ctx=8192, bits=[4, 2, 2], c=[0.8, 0.85, 0.9],
                                sigma=[0.15, 0.12, 0.1], rotate=1, steps=64, seed=2),
    "int2-32k-24l": Workload("int2-32k-24l", n_loops=4, batch=8, heads=16, d=128, g=32,
                             n_ctx=32768, bits=[2, 2, 2], c=[0.8, 0.85, 0.9],
                             sigma=[0.15, 0.12, 0.1], rotate=1, layers=24, seed=3),
    "peak-batch-8k": Workload("peak-batch-8k", n_loops=4, batch=0, heads=16, d=128, g=32,
                              n_ctx=8192, bits=[2, 2, 2], c=[0.8, 0.85, 0.9],
                              sigma=[0.15, 0.12, 0.1], rotate=1, layers=24, seed=4),
    # The pages' final configuration: [2,2,2,4] with an INT4 anchor at g=32 and
    # INT2 residuals at g=16, decoded loop by loop as a looped model runs,
    # with the 64 most recent tokens in BF16.
    "anchor-8k-perloop": Workload("anchor-8k-perloop", n_loops=4, batch=16, heads=16, d=128, g=16,
                                  n_ctx=8192, bits=[2, 2, 2], c=[0.8, 0.85, 0.9],
                                  sigma=[0.15, 0.12, 0.1], rotate=1, seed=5, ref_bits=4,
                                  ref_group=32, extra={"tail": 64}),
    # The same with chained references (Next-loop policy, Table 9): decoding
    # loop l rebuilds the chain from the anchor through loops L-2 .. l.
    "chain-8k-perloop": Workload("chain-8k-perloop", n_loops=4, batch=16, heads=16, d=128, g=16,
                                 n_ctx=8192, bits=[2, 2, 2], c=[0.8, 0.85, 0.9],
                                 sigma=[0.15, 0.12, 0.1], rotate=1, seed=8, ref_bits=4,
                                 ref_group=32, ref_chain=1, extra={"tail": 64}),
    # The pages' throughput grid (Fig. 4: g=32 everywhere; Fig. 6: INT2
    # residuals at g=16): 24 layers, contexts 2k-16k, power-of-two batches up
    # to a 250 GB KV budget, per-loop decode, against BF16 per-loop decode.
    "grid-g16": Workload("grid-g16", n_loops=4, batch=0, heads=16, d=128, g=16, n_ctx=0,
                         bits=[2, 2, 2], c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=1,
                         layers=24, seed=6, ref_bits=4, ref_group=32,
                         extra={"tail": 64, "contexts": [2048, 4096, 8192, 16384]}),
    "grid-g32": Workload("grid-g32", n_loops=4, batch=0, heads=16, d=128, g=32, n_ctx=0,
                         bits=[2, 2, 2], c=[0.8, 0.85, 0.9], sigma=[0.15, 0.12, 0.1], rotate=1,
                         layers=24, seed=7, ref_bits=4, ref_group=32,
                         extra={"tail": 64, "contexts": [2048, 4096, 8192, 16384]}),
}


def generator(seed: int, device: str = "cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def channel_std(gen: torch.Generator, heads: int, d: int) -> torch.Tensor:
    """Per (head, channel) standard deviation ~ LogNormal(0, 0.5)."""
    dev = gen.device
    return torch.exp(0.5 * torch.randn(heads, d, generator=gen, device=dev))


def draw_kv(gen: torch.Generator, n_loops: int, batch: int, heads: int, n: int, d: int,
            c: Sequence[float], sigma: Sequence[float], std: Optional[torch.Tensor] = None):
    """One side (K or V) of one layer.

    Returns (ref, loops): ref bf16 [B, H, n, d] is the final loop; loops bf16
    [L-1, B, H, n, d] are the earlier loops, loop l = c[l]*ref + N(0, sigma[l]^2)
    (computed in float32 before rounding)."""
    dev = gen.device
    if std is None:
        std = channel_std(gen, heads, d)
    ref = torch.randn(batch, heads, n, d, generator=gen, device=dev) * std[None, :, None, :]
    loops = torch.empty(n_loops - 1, batch, heads, n, d, dtype=torch.bfloat16, device=dev)
    for l in range(n_loops - 1):
        noise = torch.randn(batch, heads, n, d, generator=gen, device=dev)
        loops[l] = (c[l] * ref + sigma[l] * noise).to(torch.bfloat16)
    return ref.to(torch.bfloat16), loops


def draw_queries(gen: torch.Generator, n_loops: int, batch: int, heads: int, d: int):
    """bf16 [L, B, H, d], N(0, 1)."""
    return torch.randn(n_loops, batch, heads, d, generator=gen, device=gen.device).to(torch.bfloat16)


def draw_layer(w: Workload, seed: Optional[int] = None, batch: Optional[int] = None,
               n: Optional[int] = None, device: str = "cpu"):
    """K side, V side and queries for one layer of workload `w`.

    Returns dict(k_ref, k_loops, v_ref, v_loops, q) with tokens [0, n)."""
    gen = generator(w.seed if seed is None else seed, device)
    B = w.batch if batch is None else batch
    n = w.n_ctx if n is None else n
    k_std = channel_std(gen, w.heads, w.d)
    v_std = channel_std(gen, w.heads, w.d)
    k_ref, k_loops = draw_kv(gen, w.n_loops, B, w.heads, n, w.d, w.c, w.sigma, k_std)
    v_ref, v_loops = draw_kv(gen, w.n_loops, B, w.heads, n, w.d, w.c, w.sigma, v_std)
    q = draw_queries(gen, w.n_loops, B, w.heads, w.d)
    return dict(k_ref=k_ref, k_loops=k_loops, v_ref=v_ref, v_loops=v_loops, q=q,
                k_std=k_std, v_std=v_std)


def draw_tail(w: Workload, seed: int, batch: Optional[int] = None, n: int = 64,
              device: str = "cpu") -> dict:
    """Recent tokens kept in BF16: every loop's own K and V for n tokens,
    drawn like the cache (loop l = c_l * final loop + noise).  Returns
    dict(k, v), each bf16 [L, B, H, n, d] with the final loop last."""
    gen = generator(seed, device)
    B = w.batch if batch is None else batch
    out = {}
    for side in ("k", "v"):
        std = channel_std(gen, w.heads, w.d)
        ref, loops = draw_kv(gen, w.n_loops, B, w.heads, n, w.d, w.c, w.sigma, std)
        out[side] = torch.cat([loops, ref.unsqueeze(0)]).contiguous()
    return out


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (CPU)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
