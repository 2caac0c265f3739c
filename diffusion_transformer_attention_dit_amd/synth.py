"""Seeded synthetic inputs and the workload table.

This module holds no attention or rotary arithmetic: it only draws the
Q, K, V tensors that both the HIP path and the fp64 checker consume, so that
the two see identical inputs. The pages evaluate on two private talking-head
clips (77 and 240 frames) that are not available; Gaussian activations with
the latent shapes of one 25-frame decode window and of the 77-frame clip stand
in for the real Q/K/V (blog summary, "Methodology - deep read": 25-frame
windows, 77- and 240-frame test clips).

Seeds: base seed 0; each (workload, step, block) derives its own seed; the
draw order is Q, K, V, then the per-head scales.
"""
from dataclasses import dataclass
from typing import Optional, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]  # (T, H, W) latent grid
    std: float                  # Q/K/V ~ N(0, 1) * std
    input_dtype: str            # "f32" or "bf16" as drawn
    head_scale: Optional[Tuple[float, float]] = None  # per-head U(lo, hi) factor
    steps: int = 1              # sampling steps per window
    blocks: int = 1             # transformer blocks per step
    index: int = 0

    @property
    def tokens(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]

    @property
    def calls(self) -> int:
        return self.steps * self.blocks

    @property
    def flops_per_call(self) -> int:
        # Q K^T and P V, non-causal: 2 * N^2 * d each, per head.
        return 4 * self.tokens * self.tokens * self.head_dim * self.heads

    @property
    def bytes_per_call(self) -> int:
        # Read Q, K, V and write O once, bf16.
        return 4 * self.heads * self.tokens * self.head_dim * 2


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_1x64_n128", 1, 64, (2, 8, 8), 1.0, "f32", index=0),
        Workload("block_12x128_n1560", 12, 128, (4, 15, 26), 0.5, "bf16", index=1),
        Workload("ulysses_share_3x128_n10920", 3, 128, (7, 30, 52), 0.5, "bf16", index=2),
        Workload("window25_12x128_n10920", 12, 128, (7, 30, 52), 0.5, "bf16",
                 steps=4, blocks=30, index=3),
        Workload("clip77_12x128_n31200", 12, 128, (20, 30, 52), 0.5, "bf16",
                 head_scale=(0.25, 1.0), steps=4, blocks=30, index=4),
    ]
}

ORDER = [w.name for w in sorted(WORKLOADS.values(), key=lambda w: w.index)]


def seed_for(w: Workload, step: int = 0, block: int = 0, base_seed: int = 0) -> int:
    return (base_seed * 1_000_003 + w.index * 100_003 + step * 1_009 + block) & 0x7FFFFFFF


def make_qkv(w: Workload, step: int = 0, block: int = 0, device="cpu", base_seed: int = 0,
             dtype: torch.dtype = torch.bfloat16, grid=None, heads=None, std=None):
    """Draw (q, k, v), each [heads, T*H*W, head_dim], in `dtype`.

    fp32 draws are rounded once (round-to-nearest-even) when `dtype` is
    bfloat16. `grid`, `heads` and `std` override the workload's for edge-case
    tests.
    """
    grid = tuple(grid) if grid is not None else w.grid
    heads = heads if heads is not None else w.heads
    std = std if std is not None else w.std
    n = grid[0] * grid[1] * grid[2]
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(w, step, block, base_seed))
    shape = (heads, n, w.head_dim)
    q = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    fac = torch.full((heads, 1, 1), std, device=device, dtype=torch.float32)
    if w.head_scale is not None:
        lo, hi = w.head_scale
        s = torch.rand((heads,), generator=g, device=device, dtype=torch.float32)
        fac = fac * (lo + (hi - lo) * s).view(heads, 1, 1)
    q, k, v = (t.mul_(fac).to(dtype).contiguous() for t in (q, k, v))
    return q, k, v


# Conditioning context length for cross-attention. The pages name the
# text/image encoders the decoder is conditioned on but not how many tokens
# they hand over; 77 is the CLIP text encoder's fixed context.
CONTEXT_TOKENS = 77


def make_context(w: Workload, ctx_len: int = CONTEXT_TOKENS, step: int = 0, block: int = 0,
                 device="cpu", base_seed: int = 0, dtype: torch.dtype = torch.bfloat16):
    """Draw conditioning keys and values (k_ctx, v_ctx), each
    [heads, ctx_len, head_dim], N(0,1) * the workload's std, from a seed of
    their own (independent of make_qkv's)."""
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(w, step, block, base_seed) ^ 0x5EED_C7C7)
    shape = (w.heads, ctx_len, w.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * w.std
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * w.std
    return k.to(dtype).contiguous(), v.to(dtype).contiguous()


def make_block_inputs(w: Workload, step: int = 0, block: int = 0, device="cpu", base_seed: int = 0,
                      dtype: torch.dtype = torch.bfloat16):
    """Synthetic inputs of one self-attention block: hidden states x
    [T*H*W, heads*head_dim] ~ N(0, 1) and random-init weights in the
    [out][in] layout of a linear layer, w_qkv [3*hidden, hidden] and w_o
    [hidden, hidden], ~ N(0, 1/hidden) (no trained weights exist here), from
    a seed of their own."""
    hidden = w.heads * w.head_dim
    n = w.grid[0] * w.grid[1] * w.grid[2]
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(w, step, block, base_seed) ^ 0xB10C)
    x = torch.randn((n, hidden), generator=g, device=device, dtype=torch.float32)
    sd = hidden ** -0.5
    w_qkv = torch.randn((3 * hidden, hidden), generator=g, device=device, dtype=torch.float32) * sd
    w_o = torch.randn((hidden, hidden), generator=g, device=device, dtype=torch.float32) * sd
    return tuple(t.to(dtype).contiguous() for t in (x, w_qkv, w_o))


def sample_rows(n: int, count: int, seed: int, tile: int = 128):
    """A seeded sorted sample of query rows that always holds the first and
    last row and the rows on each side of every `tile` boundary it can fit."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    must = {0, n - 1}
    b = tile
    while b < n and len(must) < count // 2:
        must.update({b - 1, b})
        b += tile * max(1, (n // tile) // max(1, count // 4))
    rest = max(0, min(count, n) - len(must))
    pool = torch.randperm(n, generator=g).tolist()
    out = set(must)
    for r in pool:
        if len(out) >= len(must) + rest:
            break
        out.add(r)
    return sorted(out)
