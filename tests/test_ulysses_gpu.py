"""GPU parity of the Ulysses layouts (blog summary, "Methodology - deep
read", USP paragraph): the pack/unpack halves of the all-to-all (bit-exact
permutations) and attention taking the exchanged token-major layout
directly (REGEN_ATTN_TOKEN_MAJOR), through the C ABI against the oracle.
The all-to-all itself is the collective between devices; on one GPU it is
simulated by indexing, exactly as oracle.ulysses_exchange defines it.
Bars for attention outputs as in test_parity_gpu.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from diffusion_transformer_attention_dit_amd import native, synth

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
MEAN_REL = 1e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.float().cpu().double().numpy()


def check_o(got, ref, label):
    assert np.all(np.isfinite(got)), "non-finite output " + label
    d = np.abs(got - ref)
    ma, mr = float(d.max()), float(d.sum() / np.abs(ref).sum())
    say("  %s max_abs=%.3e mean_rel=%.3e" % (label, ma, mr))
    assert ma <= MAX_ABS and mr <= MEAN_REL, (label, ma, mr)


def token_major(t):
    return t.transpose(0, 1).contiguous()  # [heads, N, d] -> [N, heads, d]


def exchange(sends):
    """recv[dst][src] = send[src][dst] (the simulated all-to-all)."""
    g = len(sends)
    return [torch.stack([sends[s][d] for s in range(g)]).contiguous() for d in range(g)]


@pytest.mark.parametrize("nl,heads,d,groups", [
    (390, 12, 128, 4), (2730, 12, 128, 4), (7, 12, 128, 12), (33, 4, 64, 2), (5, 2, 64, 1),
])
def test_pack_unpack_bit_exact(nl, heads, d, groups):
    say("case pack/unpack Nl=%d H=%d d=%d G=%d" % (nl, heads, d, groups))
    g = torch.Generator().manual_seed(nl + heads + groups)
    x = torch.randn(nl, heads, d, generator=g).to(torch.bfloat16)
    send = native.ulysses_pack(x.cuda(), groups)
    y = native.ulysses_unpack(send)
    torch.cuda.synchronize()
    ref = oracle.ulysses_pack(x.view(torch.int16).numpy(), groups)
    assert np.array_equal(send.cpu().view(torch.int16).numpy(), ref)
    assert torch.equal(y.cpu(), x)


def test_token_major_attention_block():
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case token-major attention, block workload")
    q, k, v = synth.make_qkv(w, device="cuda")
    attn = native.Attention(w.heads, w.head_dim, w.grid, flags=native.REGEN_ATTN_TOKEN_MAJOR)
    o = attn.forward(token_major(q), token_major(k), token_major(v))
    torch.cuda.synchronize()
    attn.close()
    ref = oracle.rope_attention(f64(q), f64(k), f64(v), w.grid)
    check_o(f64(o.transpose(0, 1)), ref, "block token-major")


def test_token_major_attention_ulysses_share_sampled():
    # One GPU's share at the pages' Ulysses degree 4: 3 of 12 heads, all
    # 10920 tokens of the 25-frame window, in the layout the exchange delivers.
    w = synth.WORKLOADS["ulysses_share_3x128_n10920"]
    say("case token-major attention, 3 heads x 10920 (sampled rows)")
    q, k, v = synth.make_qkv(w, 2, 11, device="cuda")
    attn = native.Attention(w.heads, w.head_dim, w.grid, flags=native.REGEN_ATTN_TOKEN_MAJOR)
    o = attn.forward(token_major(q), token_major(k), token_major(v))
    o_hm = native.Attention(w.heads, w.head_dim, w.grid).forward(q, k, v)
    torch.cuda.synchronize()
    attn.close()
    # Same kernels on a different layout: identical bits to the head-major call.
    assert torch.equal(o.transpose(0, 1), o_hm)
    rows = synth.sample_rows(w.tokens, 256, seed=3)
    ref = oracle.rope_attention(f64(q), f64(k), f64(v), w.grid, rows=rows)
    check_o(f64(o.transpose(0, 1))[:, rows], ref, "ulysses share")


def test_token_major_ranges_with_lse():
    # Ulysses x Ring (USP): token-major layout and key runs together.
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case token-major ranges + lse")
    q, k, v = synth.make_qkv(w, device="cuda")
    qb, nq, kb, nk = 200, 900, 500, 1000
    attn = native.Attention(w.heads, w.head_dim, w.grid, flags=native.REGEN_ATTN_TOKEN_MAJOR)
    qs, ks, vs = (token_major(t[:, a:a + n]) for t, a, n in ((q, qb, nq), (k, kb, nk), (v, kb, nk)))
    o, lse = attn.forward_range(qs, qb, ks, vs, kb)
    torch.cuda.synchronize()
    attn.close()
    ref_o, ref_lse = oracle.rope_attention_range(f64(q[:, qb:qb + nq]), f64(k[:, kb:kb + nk]),
                                                 f64(v[:, kb:kb + nk]), w.grid, qb, kb)
    check_o(f64(o.transpose(0, 1)), ref_o, "tm range")
    assert np.abs(lse.cpu().double().numpy() - ref_lse).max() <= 2e-2


@pytest.mark.parametrize("name,groups,rows", [("block_12x128_n1560", 4, None),
                                              ("window25_12x128_n10920", 4, 64)])
def test_simulated_ulysses_pipeline(name, groups, rows):
    # Per device s: pack its token shard; exchange; attention of the head
    # group on the received layout; exchange O back; unpack. Compared with
    # attention of the whole tensor.
    w = synth.WORKLOADS[name]
    say("case simulated Ulysses G=%d on %s" % (groups, name))
    q, k, v = synth.make_qkv(w, device="cuda")
    N, H, d = w.tokens, w.heads, w.head_dim
    nl, hg = N // groups, H // groups
    assert nl * groups == N
    shards = [[token_major(t)[s * nl:(s + 1) * nl].contiguous() for s in range(groups)]
              for t in (q, k, v)]
    recv = [exchange([native.ulysses_pack(x, groups) for x in sh]) for sh in shards]
    attn = native.Attention(hg, d, w.grid, flags=native.REGEN_ATTN_TOKEN_MAJOR)
    outs = []
    for g in range(groups):
        qg, kg, vg = (r[g].view(N, hg, d) for r in recv)
        outs.append(attn.forward(qg, kg, vg).view(groups, nl, hg, d))
    back = exchange(outs)
    got = torch.cat([native.ulysses_unpack(b) for b in back])  # [N, H, d]
    torch.cuda.synchronize()
    attn.close()
    if rows is None:
        ref = oracle.rope_attention(f64(q), f64(k), f64(v), w.grid)
        check_o(f64(got.transpose(0, 1)), ref, "ulysses pipeline")
    else:
        sample = synth.sample_rows(N, rows, seed=9)
        ref = oracle.rope_attention(f64(q), f64(k), f64(v), w.grid, rows=sample)
        check_o(f64(got.transpose(0, 1))[:, sample], ref, "ulysses pipeline")


def test_pack_argument_errors():
    say("case pack/unpack argument errors")
    x = torch.zeros(8, 12, 128, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros_like(x)
    st = torch.cuda.current_stream().cuda_stream
    E = native.REGEN_ERR_INVALID_ARGUMENT
    assert native.regen_ulysses_pack(x.data_ptr(), y.data_ptr(), 8, 12, 128, 5, st) == E  # 12 % 5
    assert native.regen_ulysses_pack(x.data_ptr(), y.data_ptr(), 0, 12, 128, 4, st) == E
    assert native.regen_ulysses_pack(x.data_ptr(), x.data_ptr(), 8, 12, 128, 4, st) == E  # overlap
    assert native.regen_ulysses_unpack(x.data_ptr() + 2, y.data_ptr(), 8, 12, 128, 4, st) == E
    assert native.regen_ulysses_unpack(x.data_ptr(), y.data_ptr(), 8, 12, 1, 12, st) == E  # 2 bytes
    torch.cuda.synchronize()
