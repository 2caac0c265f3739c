"""Throughput of the 3D-RoPE attention hot path over one decode window.

One step = one 25-frame decode window: 4 sampling steps x 30 transformer
blocks = 120 attention calls (12 heads x 10920 tokens x head_dim 128, latent
grid 7 x 30 x 52), each on its own pre-drawn seeded Q/K/V, all resident in
HBM before timing starts. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TFLOP/s and % bf16 MFMA peak; ms per 4-step decode window, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="window25_12x128_n10920")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-ring-split", action="store_true",
                    help="skip the key-split + merge leg (profiling runs of the window alone)")
    ap.add_argument("--ring-split-only", action="store_true",
                    help="run only the key-split + merge leg and print it")
    ap.add_argument("--no-ulysses", action="store_true",
                    help="skip the Ulysses layout leg (profiling runs of the window alone)")
    ap.add_argument("--ulysses-only", action="store_true",
                    help="run only the Ulysses layout leg and print it")
    ap.add_argument("--no-cross", action="store_true",
                    help="skip the cross-attention leg (profiling runs of the window alone)")
    ap.add_argument("--cross-only", action="store_true",
                    help="run only the cross-attention leg and print it")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the attention-block leg (profiling runs of the window alone)")
    ap.add_argument("--block-only", action="store_true",
                    help="run only the attention-block leg and print it")
    ap.add_argument("--no-clip", action="store_true",
                    help="skip the 77-frame clip window leg (profiling runs of the window alone)")
    ap.add_argument("--clip-only", action="store_true",
                    help="run only the 77-frame clip window leg and print it")
    ap.add_argument("--no-block-window", action="store_true",
                    help="skip the window of attention blocks (profiling runs of the window alone)")
    ap.add_argument("--block-window-only", action="store_true",
                    help="run only the window of attention blocks and print it")
    ap.add_argument("--summarize-rocprof", metavar="DIR", default=None,
                    help="write the profile summaries of the rocprofv3 passes under DIR (see "
                         "summarize_rocprof) into --summary-out and exit; needs no GPU")
    ap.add_argument("--summary-out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run 3 device-to-device copies of this many MiB (to scale HBM "
                         "byte counters against a copy of known size) and exit")
    return ap.parse_args()


def copy_calibration(mib):
    import torch
    n = mib * (1 << 20) // 4
    src = torch.arange(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_copy": n * 4,
                                           "bytes_written_per_copy": n * 4, "copies": 3}}))
    return 0


def counted_traffic(w, algorithmic_bytes):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    passes (FETCH_SIZE, WRITE_SIZE, scaled against a copy of known size), or
    None when the attention kernels' source (common.hpp + attention.hpp) or
    the build flags (build.py) have changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_%s_traffic.json" % w.name)
    try:
        doc = json.load(open(path))
        sha = kernel_source_sha256()
    except (OSError, ValueError):
        return None
    if doc.get("kernel_source_sha256") != sha:
        return None
    total = doc["fetch_bytes_per_launch"] + doc["write_bytes_per_launch"]
    return {"bytes_per_launch": round(total), "read_bytes": round(doc["fetch_bytes_per_launch"]),
            "write_bytes": round(doc["write_bytes_per_launch"]),
            "vs_algorithmic": round(total / algorithmic_bytes, 3)}


def cpu_baseline(w, target_s):
    """The fp64 oracle on a bounded row sample of one call of the workload."""
    import numpy as np
    import torch

    import oracle
    from diffusion_transformer_attention_dit_amd import synth

    q, k, v = synth.make_qkv(w, 0, 0, device="cpu")
    qd, kd, vd = (t.float().numpy().astype(np.float64) for t in (q, k, v))
    del q, k, v
    # K rotation of the whole window (once per call) is timed separately.
    t0 = time.perf_counter()
    oracle.c_rope_grid(kd, w.grid)
    rope_s = time.perf_counter() - t0
    # Calibrate the per-row cost, then size the sample to ~target_s.
    rows = synth.sample_rows(w.tokens, 4, seed=11)
    t0 = time.perf_counter()
    oracle.rope_attention(qd, kd, vd, w.grid, rows=rows)
    cal = time.perf_counter() - t0 - rope_s
    per_row = max(cal, 1e-3) / (len(rows) * w.heads)
    n_rows = int(max(8, min(w.tokens, target_s / per_row / w.heads)))
    rows = synth.sample_rows(w.tokens, n_rows, seed=12)
    t0 = time.perf_counter()
    oracle.rope_attention(qd, kd, vd, w.grid, rows=rows)
    el = time.perf_counter() - t0
    attn_s = max(el - rope_s, 1e-9)
    flops = 4.0 * w.head_dim * w.tokens * len(rows) * w.heads
    tflops = flops / attn_s / 1e12
    call_s = w.flops_per_call / (tflops * 1e12) + rope_s
    return {
        "value": tflops, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
        "sample": "%d query rows x %d heads of one %s call (%d keys each, fp64); K rotation of "
                  "the full call %.2f s; %.1f s total" % (len(rows), w.heads, w.name, w.tokens,
                                                          rope_s, el),
        "ms_per_window_extrapolated": call_s * w.calls * 1e3,
        "cpu_model": _cpu_model(),
    }


def ring_split(w, qkv, stream, reps=10):
    """The one-GPU piece of a Ring split with R = 2: attention of all queries
    over each key half (with log-sum-exp), then the exact merge, against one
    call over all keys. Also the merge kernel alone, against HBM bandwidth."""
    import torch

    from diffusion_transformer_attention_dit_amd import native
    q, k, v = qkv
    half = w.tokens // 2
    k1, v1 = k[:, :half].contiguous(), v[:, :half].contiguous()
    k2, v2 = k[:, half:].contiguous(), v[:, half:].contiguous()
    attn = native.Attention(w.heads, w.head_dim, w.grid)
    o_full, l_full = torch.empty_like(q), torch.empty(w.heads, w.tokens, device=q.device)
    o1, o2, o = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    l1, l2, lse = (torch.empty(w.heads, w.tokens, device=q.device) for _ in range(3))

    def split():
        attn.forward_range(q, 0, k1, v1, 0, out=o1, lse=l1, stream=stream)
        attn.forward_range(q, 0, k2, v2, half, out=o2, lse=l2, stream=stream)
        native.merge([o1, o2], [l1, l2], out=o, lse=lse, stream=stream)

    def full():
        attn.forward_range(q, 0, k, v, 0, out=o_full, lse=l_full, stream=stream)

    def merge_only():
        native.merge([o1, o2], [l1, l2], out=o, lse=lse, stream=stream)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_full, t_split, t_merge = timed(full), timed(split), timed(merge_only)
    attn.close()
    rows = w.heads * w.tokens
    merge_bytes = 2 * (rows * w.head_dim * 2 + rows * 4) + rows * w.head_dim * 2 + rows * 4
    gbs = merge_bytes / (t_merge * 1e-3) / 1e9
    return {
        "what": "all queries over key halves [0, %d) and [%d, %d) with lse, then the exact merge, "
                "vs one call over all keys with lse" % (half, half, w.tokens),
        "full_with_lse_ms": round(t_full, 4), "two_halves_and_merge_ms": round(t_split, 4),
        "merge_kernel": {"kernel": "merge_parts_kernel", "avg_launch_us": round(t_merge * 1e3, 2),
                         "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "algorithmic_bytes": merge_bytes},
    }


def block_leg(w, reps=10):
    """One self-attention block with random-init weights: QKV projection,
    3D-RoPE attention, output projection, timed as one unit, at the 1560-token
    block workload (12 x 128); the projection GEMM alone is also timed at the
    window's size, and so is the output projection."""
    import torch

    from diffusion_transformer_attention_dit_amd import native, synth
    window = w
    w = synth.WORKLOADS["block_12x128_n1560"]
    stream = torch.cuda.current_stream()
    x, w_qkv, w_o = synth.make_block_inputs(w, device="cuda")
    y = torch.empty_like(x)
    blk = native.Block(w.heads, w.head_dim, w.grid)
    blk.forward(x, w_qkv, w_o, out=y, stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        blk.forward(x, w_qkv, w_o, out=y, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    blk.close()
    t = a.elapsed_time(b) / reps * 1e-3
    hid = w.heads * w.head_dim
    gemm = 2.0 * w.tokens * hid * 3 * hid + 2.0 * w.tokens * hid * hid
    total = gemm + w.flops_per_call
    # The QKV projection GEMM alone at the window's token count.
    g = torch.Generator(device="cuda").manual_seed(5)
    xw = torch.randn(window.tokens, hid, generator=g, device="cuda").to(torch.bfloat16)
    wq = (torch.randn(3 * hid, hid, generator=g, device="cuda") * hid ** -0.5).to(torch.bfloat16)
    yq = torch.empty(window.tokens, 3 * hid, dtype=torch.bfloat16, device="cuda")
    for _ in range(5):  # warm-up
        native.linear(xw, wq, out=yq, stream=stream)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        native.linear(xw, wq, out=yq, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    tg = a.elapsed_time(b) / reps * 1e-3
    gf = 2.0 * window.tokens * hid * 3 * hid
    # The output projection alone at the window's token count.
    wo = (torch.randn(hid, hid, generator=g, device="cuda") * hid ** -0.5).to(torch.bfloat16)
    yo = torch.empty(window.tokens, hid, dtype=torch.bfloat16, device="cuda")
    for _ in range(5):  # warm-up
        native.linear(xw, wo, out=yo, stream=stream)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        native.linear(xw, wo, out=yo, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    to = a.elapsed_time(b) / reps * 1e-3
    go = 2.0 * window.tokens * hid * hid
    return {"what": "x[%d, %d] -> [Q|K|V] = x W_qkv^T -> attention -> y = O W_o^T (bf16, "
                    "random-init weights)" % (w.tokens, hid),
            "workload": w.name, "ms_per_block": round(t * 1e3, 4), "gflop": round(total / 1e9, 1),
            "tflops": round(total / t / 1e12, 2), "pct_peak": round(100 * total / t / 1e12 / PEAK_BF16_TFLOPS, 2),
            "projection_gflop": round(gemm / 1e9, 1), "attention_gflop": round(w.flops_per_call / 1e9, 1),
            "qkv_projection_window": {"kernel": "gemm_nt256_kernel", "shape": [window.tokens, hid, 3 * hid],
                                      "avg_launch_us": round(tg * 1e6, 2), "bound": "mfma",
                                      "achieved": round(gf / tg / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(gf / tg / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "o_projection_window": {"kernel": "gemm_nt256_kernel", "shape": [window.tokens, hid, hid],
                                    "avg_launch_us": round(to * 1e6, 2), "bound": "mfma",
                                    "achieved": round(go / to / 1e12, 2), "peak": PEAK_BF16_TFLOPS,
                                    "unit": "TFLOP/s", "frac": round(go / to / 1e12 / PEAK_BF16_TFLOPS, 4)}}


def cross_leg(w, reps=20):
    """Cross-attention of the window's tokens to conditioning tokens (77,
    the assumed encoder context, 226 and 512): time per call against the HBM
    roofline (reading Q and writing O dominate; the context is small)."""
    import torch

    from diffusion_transformer_attention_dit_amd import native, synth
    stream = torch.cuda.current_stream()
    q, _, _ = synth.make_qkv(w, device="cuda")
    o = torch.empty_like(q)
    attn = native.Attention(w.heads, w.head_dim, w.grid)
    out = {"what": "all %d tokens x %d heads attend to ctx_len conditioning tokens, no rotation"
                   % (w.tokens, w.heads)}
    for ctx in (synth.CONTEXT_TOKENS, 226, 512):
        kc, vc = synth.make_context(w, ctx, device="cuda")
        attn.forward_cross(q, kc, vc, out=o, stream=stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            attn.forward_cross(q, kc, vc, out=o, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        t = a.elapsed_time(b) / reps * 1e-3
        flops = 4.0 * w.tokens * ctx * w.head_dim * w.heads
        moved = 2 * w.heads * w.tokens * w.head_dim * 2 + 2 * w.heads * ctx * w.head_dim * 2
        gbs = moved / t / 1e9
        out["ctx_%d" % ctx] = {"us_per_call": round(t * 1e6, 2), "tflops": round(flops / t / 1e12, 2),
                               "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                               "algorithmic_bytes": moved}
    attn.close()
    return out


def ulysses_leg(w, groups=4, reps=20):
    """One device's share of Ulysses degree 4 at the window's shape: pack its
    token shard of Q for the all-to-all, attention of its head group on the
    exchanged token-major layout (against the head-major call), and unpack
    of its O shard after the reverse exchange."""
    import torch

    from diffusion_transformer_attention_dit_amd import native, synth
    N, H, d = w.tokens, w.heads, w.head_dim
    nl, hg = N // groups, H // groups
    stream = torch.cuda.current_stream()
    g = torch.Generator(device="cuda").manual_seed(77)
    x = torch.randn(nl, H, d, generator=g, device="cuda").to(torch.bfloat16)
    send = torch.empty(groups, nl, hg, d, dtype=torch.bfloat16, device="cuda")
    back = torch.empty_like(x)
    share = synth.WORKLOADS["ulysses_share_3x128_n10920"]
    q, k, v = synth.make_qkv(share, device="cuda")
    qt, kt, vt = (t.transpose(0, 1).contiguous() for t in (q, k, v))
    o = torch.empty_like(q)
    ot = torch.empty_like(qt)
    a_hm = native.Attention(hg, d, w.grid)
    a_tm = native.Attention(hg, d, w.grid, flags=native.REGEN_ATTN_TOKEN_MAJOR)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_pack = timed(lambda: native.ulysses_pack(x, groups, out=send, stream=stream))
    t_unpack = timed(lambda: native.ulysses_unpack(send, out=back, stream=stream))
    t_hm = timed(lambda: a_hm.forward(q, k, v, out=o, stream=stream))
    t_tm = timed(lambda: a_tm.forward(qt, kt, vt, out=ot, stream=stream))
    a_hm.close()
    a_tm.close()
    moved = 2 * nl * H * d * 2  # read + write of one shard

    def leg(t_ms, kernel):
        gbs = moved / (t_ms * 1e-3) / 1e9
        return {"kernel": kernel, "avg_launch_us": round(t_ms * 1e3, 2), "bound": "hbm",
                "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": moved}
    return {
        "what": "Ulysses degree %d at %d tokens x %d heads: pack of one %d-token shard, attention "
                "of one %d-head group on the exchanged token-major layout vs head-major, unpack "
                "of one shard" % (groups, N, H, nl, hg),
        "pack": leg(t_pack, "block_transpose_kernel"),
        "unpack": leg(t_unpack, "block_transpose_kernel"),
        "attention_token_major_ms": round(t_tm, 4), "attention_head_major_ms": round(t_hm, 4),
    }


def clock_leg(stream):
    """GPU core clock under a pure bf16 MFMA load (regen_clock_probe), and
    that load's TFLOP/s: the clock the chip settles at on this machine."""
    from diffusion_transformer_attention_dit_amd import native
    ghz, tflops, secs = native.clock_probe(stream=stream)
    return {"gpu_clock_ghz": round(ghz, 4), "mfma_probe_tflops": round(tflops, 1),
            "probe_ms": round(secs * 1e3, 2)}


def block_window_leg(w, reps=2):
    """A whole decode window of attention blocks at the window's size:
    4 steps x 30 blocks, each QKV projection (N x 1536 -> 4608), 3D-RoPE
    attention and output projection, per-block weights and per-call hidden
    states resident in HBM before timing."""
    import torch

    from diffusion_transformer_attention_dit_amd.sampler import BlockWindowDriver
    stream = torch.cuda.current_stream()
    print("bench: drawing the block window's inputs", file=sys.stderr, flush=True)
    drv = BlockWindowDriver(w, device="cuda")
    drv.run_window(stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        drv.run_window(stream)
    b.record(stream)
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / reps * 1e-3
    out = {"what": "%d self-attention blocks (%d steps x %d blocks) at %d tokens x %d hidden: "
                   "QKV projection, 3D-RoPE attention, output projection, bf16, random-init weights"
                   % (drv.calls, drv.steps, drv.blocks, w.tokens, w.heads * w.head_dim),
           "windows_timed": reps, "ms_per_window": round(t * 1e3, 3),
           "ms_per_block": round(t * 1e3 / drv.calls, 4),
           "tflops": round(drv.flops / t / 1e12, 2),
           "pct_peak": round(100 * drv.flops / t / 1e12 / PEAK_BF16_TFLOPS, 2),
           "gflop_per_window": round(drv.flops / 1e9, 1)}
    drv.close()
    del drv
    torch.cuda.empty_cache()
    return out


def clip_window_leg(reps=1):
    """The 77-frame clip window (12 heads x 31200 tokens x 128, per-head scale
    U(0.25, 1)): 120 calls with fresh seeded inputs (34.5 GB, resident in HBM)
    timed end to end in one event pair per window; the attention kernel's own
    duration from the library's kernel events over one more window."""
    import torch

    from diffusion_transformer_attention_dit_amd import native, synth
    from diffusion_transformer_attention_dit_amd.sampler import WindowDriver
    c = synth.WORKLOADS["clip77_12x128_n31200"]
    stream = torch.cuda.current_stream()
    print("bench: drawing %d calls of %s" % (c.calls, c.name), file=sys.stderr, flush=True)
    drv = WindowDriver(c, device="cuda")
    for (q, k, v) in drv.inputs[:2]:
        drv.attn.forward(q, k, v, out=drv.outs[0], stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        drv.run_window(stream)
    b.record(stream)
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / reps * 1e-3
    prof = native.Attention(c.heads, c.head_dim, c.grid, flags=native.REGEN_ATTN_PROFILE)
    for i, (q, k, v) in enumerate(drv.inputs):
        prof.forward(q, k, v, out=drv.outs[i & 1], stream=stream)
    prep_ms, attn_ms, merge_ms, n = prof.profile_read()
    prof.close()
    drv.close()
    del drv
    torch.cuda.empty_cache()
    t_attn = attn_ms / n * 1e-3
    return {"workload": c.name, "windows_timed": reps, "calls_per_window": c.calls,
            "ms_per_window": round(t * 1e3, 2),
            "tflops": round(c.flops_per_call * c.calls / t / 1e12, 2),
            "pct_peak": round(100 * c.flops_per_call * c.calls / t / 1e12 / PEAK_BF16_TFLOPS, 2),
            "attention_kernel": {"kernel": "attn_fwd_kernel", "avg_launch_us": round(t_attn * 1e6, 1),
                                 "bound": "mfma", "achieved": round(c.flops_per_call / t_attn / 1e12, 2),
                                 "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                 "frac": round(c.flops_per_call / t_attn / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "prep_us": round(prep_ms / n * 1e3, 1), "merge_us": round(merge_ms / n * 1e3, 1)}


# ---------------------------------------------------------------------------
# rocprofv3 summaries (--summarize-rocprof DIR): turns the CSV output of the
# profiling passes under DIR into the markdown tables and the traffic record
# kept in profiles/. Expected passes (subdirectories, each a rocprofv3 -d
# target with -o run --output-format csv): trace (--kernel-trace --stats of
# the window bench; its stdout JSON line in trace/bench.json), fetch / write
# (--pmc FETCH_SIZE / WRITE_SIZE of one window), calf / calw (the same
# counters over --copy-calibration-mib 512), sq1, sq2 (instruction and cycle
# counters of one window); commands*.txt hold the commands, one per line.
# Any other subdirectory with a kernel trace gets a duration table.
# ---------------------------------------------------------------------------

def _kernel_short(name):
    n = name.strip().strip('"')
    if n.startswith("void "):
        n = n[5:]
    depth, out = 0, []
    for ch in n:  # cut the parameter list (the first '(' outside template brackets)
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).replace("regen::", "").strip()


def _find(dirpath, suffix):
    hits = []
    for root, _, files in os.walk(dirpath):
        hits += [os.path.join(root, f) for f in files if f.endswith(suffix)]
    return sorted(hits)


def _read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _stats(pass_dir):
    """{kernel: (calls, avg_us, min_us, max_us, pct)} from *_kernel_stats.csv."""
    out = {}
    for f in _find(pass_dir, "_kernel_stats.csv"):
        for r in _read_csv(f):
            out[_kernel_short(r["Name"])] = (int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                                             float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                                             float(r["Percentage"]))
    return out


def _counters(pass_dir):
    """{kernel: {counter: mean per dispatch}} and {kernel: mean dispatch us}."""
    acc, dur = {}, {}
    for f in _find(pass_dir, "_counter_collection.csv"):
        for r in _read_csv(f):
            k = _kernel_short(r["Kernel_Name"])
            acc.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            dur.setdefault(k, {})[r["Dispatch_Id"]] = d
    mean = {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}
    return mean, {k: sum(v.values()) / len(v) for k, v in dur.items()}


def _pick(d, prefix):
    for k in d:
        if k.startswith(prefix):
            return k
    return None


def kernel_source_sha256():
    """Hash of the attention kernels' source and the build flags: the traffic
    record applies only to the build it was measured on."""
    import hashlib
    csrc = os.path.join(ROOT, "diffusion_transformer_attention_dit_amd")
    h = hashlib.sha256()
    for name in ("csrc/common.hpp", "csrc/attention.hpp", "build.py"):
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()


def summarize_rocprof(run_dir, out_dir, workload="window25_12x128_n10920"):
    from diffusion_transformer_attention_dit_amd import synth
    w = synth.WORKLOADS[workload]
    os.makedirs(out_dir, exist_ok=True)
    cmds = []
    for cname in sorted(os.listdir(run_dir)):  # commands.txt, commands_*.txt (one per GPU session)
        if cname.startswith("commands") and cname.endswith(".txt"):
            cmds += [c.rstrip("\n") for c in open(os.path.join(run_dir, cname)) if c.strip()]
    L = ["# Kernel profile: 3D-RoPE attention, %s (%d heads x %d tokens x head_dim %d, bf16)"
         % (w.name, w.heads, w.tokens, w.head_dim), "",
         "Measured on one MI355X (gfx950) with rocprofv3, each pass its own run of the committed "
         "bench.py, all in one GPU session; this file and the traffic record beside it were written by "
         "`python bench.py --summarize-rocprof <dir>` from the passes' CSV output. Commands (run from "
         "/tmp with TMPDIR=/tmp; $REPO is the repository root):", ""]
    own = ("trace", "fetch", "write", "calf", "calw", "sq1", "sq2", "sq3")
    L += ["    " + c for c in cmds if any(("/%s " % sub) in c or ("/%s/" % sub) in c for sub in own)] + [""]
    trace = _stats(os.path.join(run_dir, "trace"))
    bench = None
    bpath = os.path.join(run_dir, "trace", "bench.json")
    if os.path.exists(bpath):
        for line in open(bpath):
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                bench = json.loads(line)
    attn = _pick(trace, "attn_fwd_kernel")
    L += ["## Kernel durations (`--kernel-trace --stats`)", "",
          "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for k, (n, avg, mn, mx, pct) in sorted(trace.items(), key=lambda kv: -kv[1][4]):
        L.append("| %s | %d | %.1f | %.1f | %.1f | %.2f |" % (k[:60], n, avg, mn, mx, pct))
    L.append("")
    record = {"workload": w.name, "kernel": "attn_fwd_kernel"}
    if attn:
        avg = trace[attn][1]
        tf = w.flops_per_call / (avg * 1e-6) / 1e12
        L.append("%s: %.1f us average -> %.1f TFLOP/s (4 N^2 d heads = %.1f GFLOP per launch), %.1f%% of the "
                 "%.1f TFLOP/s bf16 dense peak (256 CU x 4096 flop/clk x 2.4 GHz)."
                 % (attn, avg, tf, w.flops_per_call / 1e9, 100 * tf / PEAK_BF16_TFLOPS, PEAK_BF16_TFLOPS))
        record["avg_launch_us_rocprof"] = avg
        if bench:
            rl, ck = bench.get("roofline", {}), bench.get("clock", {})
            ghz = rl.get("gpu_clock_ghz")
            if ghz:
                cus = ck.get("compute_units", 256)
                peak_c = cus * 4096 * ghz * 1e9 / 1e12
                cyc = avg * 1e-6 * ghz * 1e9
                record.update({"gpu_clock_ghz": ghz, "gpu_cycles_per_launch": round(cyc)})
                L += ["", "GPU clock during this traced run (regen_clock_probe, pure bf16 MFMA load, before and "
                      "after the timed windows): %.3f GHz. At that clock the MFMA peak is %.1f TFLOP/s, so the "
                      "kernel runs at %.1f%% of the peak of the clock it ran at; %.3f M GPU cycles per launch."
                      % (ghz, peak_c, 100 * tf / peak_c, cyc / 1e6)]
            L += ["", "The same run's bench line (library HIP events on the launch stream, under the profiler): "
                  "%.3f ms per window of %d calls; attention kernel %.1f us average."
                  % (bench.get("ms_per_window", float("nan")), w.calls, rl.get("avg_launch_us", float("nan")))]
    L.append("")

    # traffic
    fetch, fdur = _counters(os.path.join(run_dir, "fetch"))
    write, _ = _counters(os.path.join(run_dir, "write"))
    calf, _ = _counters(os.path.join(run_dir, "calf"))
    calw, _ = _counters(os.path.join(run_dir, "calw"))
    if fetch and write and calf and calw:
        copy_bytes = 512 * (1 << 20)
        ck = [k for k in calf if "copy" in k.lower() or "elementwise" in k.lower()]
        fk = calf[ck[0]]["FETCH_SIZE"] if ck else None
        wk = calw[ck[0]]["WRITE_SIZE"] if ck and ck[0] in calw else None
        if fk and wk:
            fs, ws = copy_bytes / (fk * 1024), copy_bytes / (wk * 1024)
            L += ["## HBM traffic (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`, separate runs)", "",
                  "Calibration: a device copy of 512 MiB reads FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB "
                  "per copy, so FETCH_SIZE is scaled by %.3f and WRITE_SIZE by %.3f." % (fk, wk, fs, ws), "",
                  "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | algorithmic MB | ratio |",
                  "|---|---|---|---|---|---|---|"]
            algo = {"attn_fwd_kernel": w.bytes_per_call, "rope_k_vt_kernel": w.bytes_per_call}
            for k in sorted(fetch):
                if k not in write:
                    continue
                fr = fetch[k].get("FETCH_SIZE", 0) * 1024 * fs
                wr = write[k].get("WRITE_SIZE", 0) * 1024 * ws
                a = next((v for p_, v in algo.items() if k.startswith(p_)), None)
                L.append("| %s | %.0f | %.0f | %.1f | %.1f | %s | %s |" % (
                    k[:60], fetch[k].get("FETCH_SIZE", 0), write[k].get("WRITE_SIZE", 0), fr / 1e6, wr / 1e6,
                    "%.1f" % (a / 1e6) if a else "-", "%.2f" % ((fr + wr) / a) if a else "-"))
                if k.startswith("attn_fwd_kernel"):
                    record.update({"fetch_bytes_per_launch": fr, "write_bytes_per_launch": wr,
                                   "fetch_scale": fs, "write_scale": ws})
            L += ["", "Algorithmic bytes: attention reads Q, rotated K and transposed V once and writes O once "
                  "(4 x heads x N x d x 2 B); the K-rotation / V-transpose pass reads K, V and writes Kr, Vt. "
                  "Reads above that are K/V blocks fetched again from beyond L2 by workgroups of other XCDs.", ""]

    # instruction / cycle counters
    sq = {}
    for pname in ("sq1", "sq2", "sq3"):
        c, d = _counters(os.path.join(run_dir, pname))
        k = _pick(c, "attn_fwd_kernel")
        if k:
            sq.update(c[k])
            sq.setdefault("_dispatch_us_" + pname, d.get(k))
    if sq:
        L += ["## Instruction and utilisation counters of attn_fwd_kernel (per launch, averaged)", ""]
        L += ["- %s: %.0f" % (c, v) for c, v in sorted(sq.items()) if not c.startswith("_")]
        L.append("")
        xcd = 8
        gpu_cyc = sq.get("GRBM_GUI_ACTIVE", 0) / xcd
        busy = sq.get("SQ_VALU_MFMA_BUSY_CYCLES")
        der = []
        if gpu_cyc and busy:
            per_simd = busy / (256 * 4)
            der.append("MFMA busy %.0f cycles per SIMD of %.0f GPU-busy cycles per XCD (%.1f%%)"
                       % (per_simd, gpu_cyc, 100 * per_simd / gpu_cyc))
            dus = sq.get("_dispatch_us_sq1")
            if dus:
                der.append("clock in the counter pass %.0f cycles / %.1f us = %.3f GHz" % (gpu_cyc, dus, gpu_cyc / dus / 1e3))
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in sq and busy:
            der.append("VALU co-issued with MFMA during %.1f%% of MFMA-busy cycles" % (100 * sq["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy))
        if "SQ_INSTS_MFMA" in sq:
            need = w.flops_per_call / (2 * 32 * 32 * 16) / 64 * 64
            der.append("MFMA instructions %.0f vs %.0f needed for 4 N^2 d heads (ratio %.3f, tile padding)"
                       % (sq["SQ_INSTS_MFMA"], need, sq["SQ_INSTS_MFMA"] / need))
            if "SQ_INSTS_LDS" in sq:
                der.append("LDS instructions per MFMA %.3f" % (sq["SQ_INSTS_LDS"] / sq["SQ_INSTS_MFMA"]))
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in sq:
            der.append("SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 = %.1f GFLOP" % (sq["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / 1e9))
        if der:
            L += ["Derived: " + "; ".join(der) + ".", ""]
        record["mfma_busy_frac"] = (busy / (256 * 4) / gpu_cyc) if gpu_cyc and busy else None
    record["kernel_source_sha256"] = kernel_source_sha256()
    with open(os.path.join(out_dir, "attn_fwd_%s.md" % w.name), "w") as f:
        f.write("\n".join(L) + "\n")
    if "fetch_bytes_per_launch" in record:
        with open(os.path.join(out_dir, "attn_fwd_%s_traffic.json" % w.name), "w") as f:
            json.dump(record, f, indent=1)
            f.write("\n")

    # duration tables of the other traced legs
    for sub in sorted(os.listdir(run_dir)):
        if sub in ("trace", "fetch", "write", "calf", "calw", "sq1", "sq2", "sq3"):
            continue
        st = _stats(os.path.join(run_dir, sub))
        if not st:
            continue
        M = ["# Kernel durations: %s" % sub, "",
             "rocprofv3 `--kernel-trace --stats`, written by `python bench.py --summarize-rocprof <dir>`. "
             "Command:", ""]
        M += ["    " + c for c in cmds if ("/%s " % sub) in c or ("/%s/" % sub) in c] + [""]
        M += ["| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
        for k, (n, avg, mn, mx, pct) in sorted(st.items(), key=lambda kv: -kv[1][4]):
            M.append("| %s | %d | %.2f | %.2f | %.2f | %.2f |" % (k[:60], n, avg, mn, mx, pct))
        with open(os.path.join(out_dir, "%s.md" % sub), "w") as f:
            f.write("\n".join(M) + "\n")
    return 0


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.summarize_rocprof:
        return summarize_rocprof(args.summarize_rocprof, args.summary_out, args.workload)
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2
    import torch

    from diffusion_transformer_attention_dit_amd import native, synth
    from diffusion_transformer_attention_dit_amd.sampler import WindowDriver

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration_mib:
        return copy_calibration(args.copy_calibration_mib)
    native.lib()  # fail loudly if the HIP library is missing
    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    if args.block_only:
        print(json.dumps({"workload": w.name, "block": block_leg(w)}), flush=True)
        return 0
    if args.cross_only:
        print(json.dumps({"workload": w.name, "cross": cross_leg(w)}), flush=True)
        return 0
    if args.ulysses_only:
        print(json.dumps({"workload": w.name, "ulysses": ulysses_leg(w)}), flush=True)
        return 0
    if args.clip_only:
        print(json.dumps({"workload": w.name, "clip77": clip_window_leg()}), flush=True)
        return 0
    if args.block_window_only:
        print(json.dumps({"workload": w.name, "block_window": block_window_leg(w)}), flush=True)
        return 0
    if args.ring_split_only:
        qkv = synth.make_qkv(w, 0, 0, device="cuda")
        print(json.dumps({"workload": w.name, "ring_split": ring_split(
            w, qkv, torch.cuda.current_stream())}), flush=True)
        return 0
    print("bench: drawing %d calls of %s" % (w.calls, w.name), file=sys.stderr, flush=True)
    drv = WindowDriver(w, device="cuda")
    # A second handle with kernel events, used for the per-kernel timing of
    # the same calls.
    prof = native.Attention(w.heads, w.head_dim, w.grid, flags=native.REGEN_ATTN_PROFILE)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        drv.run_window(stream)
    torch.cuda.synchronize()
    print("bench: warmup done", file=sys.stderr, flush=True)
    clock_before = clock_leg(stream)

    # ---- timed region: K whole windows -----------------------------------
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        drv.run_window(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_total = start.elapsed_time(end)
    ms_per_window = ms_total / args.steps
    value = drv.flops * args.steps / (ms_total * 1e-3) / 1e12
    print("bench: timed %d windows, %.2f ms/window" % (args.steps, ms_per_window),
          file=sys.stderr, flush=True)
    clock_after = clock_leg(stream)
    ghz = 0.5 * (clock_before["gpu_clock_ghz"] + clock_after["gpu_clock_ghz"])
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    peak_at_clock = cus * 4096 * ghz * 1e9 / 1e12  # TFLOP/s at the measured clock

    # ---- per-kernel durations from HIP events on the launch stream -------
    prof.profile_read()
    for _ in range(max(1, args.steps // 2)):
        for (q, k, v), i in zip(drv.inputs, range(len(drv.inputs))):
            prof.forward(q, k, v, out=drv.outs[i & 1], stream=stream)
    prep_ms, attn_ms, merge_ms, n_calls = prof.profile_read()
    prof.close()
    attn_avg_s = attn_ms / n_calls * 1e-3
    prep_avg_s = prep_ms / n_calls * 1e-3
    merge_avg_s = merge_ms / n_calls * 1e-3
    attn_tflops = w.flops_per_call / attn_avg_s / 1e12
    prep_bytes = 4 * w.heads * w.tokens * w.head_dim * 2  # read K, V; write Kr, Vt
    traffic = counted_traffic(w, w.bytes_per_call)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_window, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "heads": w.heads, "head_dim": w.head_dim,
            "latent_grid": list(w.grid), "tokens": w.tokens,
            "calls_per_window": w.calls, "steps_per_window": w.steps, "blocks": w.blocks,
        },
        "pct_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "ms_per_window": round(ms_per_window, 3),
        "ms_per_call": round(ms_total / (args.steps * w.calls), 4),
        "wall_s_timed": round(wall_s, 3),
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": (traffic or {}).get("bytes_per_launch"),
            "traffic_detail": traffic,
            "avg_launch_us": round(attn_avg_s * 1e6, 2),
            "launches": n_calls,
            "gpu_clock_ghz": round(ghz, 4),
            "peak_at_measured_clock": round(peak_at_clock, 1),
            "frac_at_measured_clock": round(attn_tflops / peak_at_clock, 4),
            "gpu_cycles_per_launch": round(attn_avg_s * ghz * 1e9),
        },
        "clock": {"before": clock_before, "after": clock_after, "compute_units": cus,
                  "window_frac_at_measured_clock": round(value / peak_at_clock, 4)},
        "prep_kernel": {
            "kernel": "rope_k_vt_kernel", "bound": "hbm",
            "avg_launch_us": round(prep_avg_s * 1e6, 2),
            "achieved": round(prep_bytes / prep_avg_s / 1e9, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(prep_bytes / prep_avg_s / 1e9 / PEAK_HBM_GBS, 4),
        },
        "merge_kernel": {"kernel": "merge_kernel", "avg_launch_us": round(merge_avg_s * 1e6, 2)},
    }
    if not args.no_ring_split:
        line["ring_split"] = ring_split(w, drv.inputs[0], stream)
    if not args.no_ulysses:
        line["ulysses"] = ulysses_leg(w)
    if not args.no_cross:
        line["cross"] = cross_leg(w)
    if not args.no_block:
        line["block"] = block_leg(w)
    drv.close()
    del drv
    torch.cuda.empty_cache()
    if not args.no_block_window:
        line["block_window"] = block_window_leg(w)
    if not args.no_clip:
        line["clip77"] = clip_window_leg()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 oracle sample on the host", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
