"""Four-step sampler driver: one attention call per transformer block per
sampling step over one decode window.

The ReGenVC decoder is distilled to four sampling steps (arXiv 2607.28144,
blog summary "Key findings" and "Methodology - deep read"); each step runs
every block of the diffusion transformer once, and each block attends over
the window's latent tokens. Without trained weights, each (step, block) call
gets its own fresh seeded Q/K/V, drawn before timing starts.
"""
import torch

from . import synth
from .native import Attention


class WindowDriver:
    """Holds the library handle, the pre-drawn inputs of every call of one
    window and a pair of output buffers (alternating, as consecutive blocks
    would), or one output per call with keep_outputs (for checking every
    call of a window)."""

    def __init__(self, workload: synth.Workload, device="cuda", base_seed=0, steps=None,
                 blocks=None, keep_outputs=False):
        self.w = workload
        self.steps = steps if steps is not None else workload.steps
        self.blocks = blocks if blocks is not None else workload.blocks
        self.attn = Attention(workload.heads, workload.head_dim, workload.grid)
        self.inputs = [synth.make_qkv(workload, s, b, device=device, base_seed=base_seed)
                       for s in range(self.steps) for b in range(self.blocks)]
        self.keep = bool(keep_outputs)
        self.outs = [torch.empty_like(self.inputs[0][0]) for _ in range(self.calls if self.keep else 2)]

    @property
    def calls(self):
        return self.steps * self.blocks

    @property
    def flops(self):
        return self.calls * self.w.flops_per_call

    def run_window(self, stream=None):
        """Enqueue all steps x blocks attention calls on one stream."""
        for i, (q, k, v) in enumerate(self.inputs):
            self.attn.forward(q, k, v, out=self.outs[i if self.keep else i & 1], stream=stream)

    def output_of(self, call):
        """The output of call `call` of the last window (with the default two
        buffers, valid for the last two calls only)."""
        return self.outs[call if self.keep else call & 1]

    def close(self):
        self.attn.close()


class BlockWindowDriver:
    """One decode window of whole self-attention blocks: four steps x 30
    blocks of [Q|K|V] = X W_qkv^T, 3D-RoPE attention, Y = O W_o^T. Block b
    has its own random-init weights (the same in every step, as a trained
    model's would be); every (step, block) call gets its own seeded hidden
    states X, all drawn before timing starts."""

    def __init__(self, workload: synth.Workload, device="cuda", base_seed=0, steps=None, blocks=None):
        from .native import Block
        self.w = workload
        self.steps = steps if steps is not None else workload.steps
        self.blocks = blocks if blocks is not None else workload.blocks
        self.blk = Block(workload.heads, workload.head_dim, workload.grid)
        self.weights = []
        for b in range(self.blocks):
            _, w_qkv, w_o = synth.make_block_inputs(workload, 0, b, device=device, base_seed=base_seed)
            self.weights.append((w_qkv, w_o))
        self.xs = [synth.make_block_inputs(workload, s, b, device=device, base_seed=base_seed)[0]
                   for s in range(self.steps) for b in range(self.blocks)]
        self.outs = [torch.empty_like(self.xs[0]) for _ in range(2)]

    @property
    def calls(self):
        return self.steps * self.blocks

    @property
    def flops(self):
        """Attention (4 N^2 d heads) plus both projections (2 N hidden 4 hidden) per call."""
        hid = self.w.heads * self.w.head_dim
        return self.calls * (self.w.flops_per_call + 2 * self.w.tokens * hid * 4 * hid)

    def run_window(self, stream=None):
        for i, x in enumerate(self.xs):
            w_qkv, w_o = self.weights[i % self.blocks]
            self.blk.forward(x, w_qkv, w_o, out=self.outs[i & 1], stream=stream)

    def close(self):
        self.blk.close()
