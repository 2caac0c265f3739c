"""GPU parity of cross-attention to conditioning tokens (the second
attention of a DiT block; the pages name the text/image encoders, not the
context length, so 77 tokens is assumed and other lengths are tested too),
through the C ABI against the fp64 oracle's plain (unrotated) attention.
Bars as in test_parity_gpu; LSE as in test_ring_gpu.
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


# 1..256 run in the short-context kernel (up to 128 with its O rows staged
# through LDS; 256: eight full key tiles), 257 and
# up in the persistent one.
@pytest.mark.parametrize("ctx_len", [1, 64, 77, 96, 97, 128, 129, 226, 256, 257, 512, 1000])
def test_cross_block_all_elements(ctx_len):
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case cross-attention block, ctx %d" % ctx_len)
    q, _, _ = synth.make_qkv(w, device="cuda")
    kc, vc = synth.make_context(w, ctx_len, device="cuda")
    attn = native.Attention(w.heads, w.head_dim, w.grid)
    o, lse = attn.forward_cross(q, kc, vc, lse=None)
    torch.cuda.synchronize()
    attn.close()
    ref_o, ref_lse = oracle.c_attention(f64(q), f64(kc), f64(vc), return_lse=True)
    check_o(f64(o), ref_o, "cross %d" % ctx_len)
    d = np.abs(lse.cpu().double().numpy() - ref_lse)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, (d.max(), d.mean())


@pytest.mark.parametrize("ctx_len", [77, 512])
def test_cross_window_sampled(ctx_len):
    w = synth.WORKLOADS["window25_12x128_n10920"]
    say("case cross-attention 25-frame window, ctx %d (sampled rows)" % ctx_len)
    q, _, _ = synth.make_qkv(w, 1, 3, device="cuda")
    kc, vc = synth.make_context(w, ctx_len, 1, 3, device="cuda")
    attn = native.Attention(w.heads, w.head_dim, w.grid)
    o, _ = attn.forward_cross(q, kc, vc)
    torch.cuda.synchronize()
    attn.close()
    rows = synth.sample_rows(w.tokens, 256, seed=ctx_len)
    ref = oracle.c_attention(f64(q)[:, rows], f64(kc), f64(vc))
    check_o(f64(o)[:, rows], ref, "cross window %d" % ctx_len)


@pytest.mark.parametrize("ctx_len", [1, 77, 128, 129, 200, 300])
def test_cross_head_dim_64(ctx_len):
    # head_dim 64 (one head, 1560 tokens); contexts up to 256 keys run in the
    # short-context kernel, longer ones in the persistent one.
    w = synth.WORKLOADS["tiny_1x64_n128"]
    grid = (4, 15, 26)
    say("case cross-attention head_dim 64, ctx %d" % ctx_len)
    q, _, _ = synth.make_qkv(w, device="cuda", grid=grid)
    kc, vc = synth.make_context(w, ctx_len, device="cuda")
    attn = native.Attention(w.heads, w.head_dim, grid)
    o, lse = attn.forward_cross(q, kc, vc, lse=None)
    torch.cuda.synchronize()
    attn.close()
    ref_o, ref_lse = oracle.c_attention(f64(q), f64(kc), f64(vc), return_lse=True)
    check_o(f64(o), ref_o, "cross d64 %d" % ctx_len)
    d = np.abs(lse.cpu().double().numpy() - ref_lse)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, (d.max(), d.mean())


def test_cross_more_heads_than_workgroups():
    # 300 heads of 32 tokens: fewer workgroups than heads, so each workgroup
    # of the short-context kernel takes whole heads, one context after another.
    heads, grid, ctx = 300, (1, 4, 8), 20
    say("case cross-attention, %d heads x %d tokens, ctx %d" % (heads, 32, ctx))
    g = torch.Generator().manual_seed(23)
    q = (torch.randn(heads, 32, 64, generator=g) * 0.5).to(torch.bfloat16)
    kc = (torch.randn(heads, ctx, 64, generator=g) * 0.5).to(torch.bfloat16)
    vc = (torch.randn(heads, ctx, 64, generator=g) * 0.5).to(torch.bfloat16)
    attn = native.Attention(heads, 64, grid)
    o, lse = attn.forward_cross(q.cuda(), kc.cuda(), vc.cuda(), lse=None)
    torch.cuda.synchronize()
    attn.close()
    ref_o, ref_lse = oracle.c_attention(f64(q), f64(kc), f64(vc), return_lse=True)
    check_o(f64(o), ref_o, "cross 300 heads")
    d = np.abs(lse.cpu().double().numpy() - ref_lse)
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, (d.max(), d.mean())


def test_cross_token_major_matches_head_major():
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case cross-attention token-major")
    q, _, _ = synth.make_qkv(w, device="cuda")
    kc, vc = synth.make_context(w, 77, device="cuda")
    a_hm = native.Attention(w.heads, w.head_dim, w.grid)
    a_tm = native.Attention(w.heads, w.head_dim, w.grid, flags=native.REGEN_ATTN_TOKEN_MAJOR)
    o_hm, _ = a_hm.forward_cross(q, kc, vc)
    tmj = lambda t: t.transpose(0, 1).contiguous()
    o_tm, _ = a_tm.forward_cross(tmj(q), tmj(kc), tmj(vc))
    torch.cuda.synchronize()
    a_hm.close()
    a_tm.close()
    assert torch.equal(o_tm.transpose(0, 1), o_hm)


def test_cross_does_not_rotate():
    # With context = the window's own K/V, cross-attention equals the
    # self-attention of a handle created without rotation.
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case cross-attention equals unrotated self-attention")
    q, k, v = synth.make_qkv(w, device="cuda")
    a = native.Attention(w.heads, w.head_dim, w.grid)
    b = native.Attention(w.heads, w.head_dim, w.grid, flags=native.REGEN_ATTN_NO_ROPE)
    o_cross, _ = a.forward_cross(q, k, v)
    o_self = b.forward(q, k, v)
    torch.cuda.synchronize()
    a.close()
    b.close()
    assert torch.equal(o_cross, o_self)


def test_cross_argument_errors():
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case cross-attention argument errors")
    q, _, _ = synth.make_qkv(w, device="cuda")
    kc, vc = synth.make_context(w, 77, device="cuda")
    o = torch.empty_like(q)
    a = native.Attention(w.heads, w.head_dim, w.grid)
    st = torch.cuda.current_stream().cuda_stream
    for n in (0, -1, w.tokens + 1):
        s = native.regen_attn_forward_cross(a.handle, q.data_ptr(), kc.data_ptr(), vc.data_ptr(), n,
                                            o.data_ptr(), None, st)
        assert s == native.REGEN_ERR_INVALID_ARGUMENT, n
    s = native.regen_attn_forward_cross(a.handle, q.data_ptr(), kc.data_ptr(), vc.data_ptr(), 77,
                                        q.data_ptr(), None, st)
    assert s == native.REGEN_ERR_INVALID_ARGUMENT  # o overlaps q
    torch.cuda.synchronize()
    a.close()
