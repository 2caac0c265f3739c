"""One handle used from several streams at once, with no ordering between the
streams from the caller: the library fences its own per-call buffers, so
every output must be bit-identical to the same calls issued one after the
other on one stream. The decoder's pipeline runs its stages on independent
threads and streams (blog summary, "Methodology - deep read"), which is why
a handle is read-only from the caller's side.
"""
import sys
import threading

import pytest
import torch

from diffusion_transformer_attention_dit_amd import native, synth

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sequential(attn, inputs):
    outs = [attn.forward(q, k, v) for (q, k, v) in inputs]
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("nstreams", [2, 3])
def test_forwards_on_several_streams_unordered(nstreams):
    # The 3-head share: about 0.2 ms per call, so calls on different streams
    # overlap on the device. Three streams share two slots, so the least
    # recently used one is handed over between streams through its event.
    w = synth.WORKLOADS["ulysses_share_3x128_n10920"]
    say("case %d streams, one handle, %s" % (nstreams, w.name))
    inputs = [synth.make_qkv(w, 0, b, device="cuda") for b in range(6)]
    attn = native.Attention(w.heads, w.head_dim, w.grid)
    ref = sequential(attn, inputs)
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    for s in streams:  # inputs were written on the default stream
        s.wait_stream(torch.cuda.current_stream())
    outs = [torch.empty_like(inputs[0][0]) for _ in inputs]
    for rep in range(3):
        for i, (q, k, v) in enumerate(inputs):
            s = streams[(i + rep) % nstreams]
            attn.forward(q, k, v, out=outs[i], stream=s)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(len(inputs)):
            assert torch.equal(outs[i], ref[i]), (rep, i)
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
    attn.close()


def test_forwards_from_two_host_threads():
    # Two host threads, each with its own stream, share one handle.
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case two host threads, one handle, %s" % w.name)
    inputs = [synth.make_qkv(w, 0, b, device="cuda") for b in range(8)]
    attn = native.Attention(w.heads, w.head_dim, w.grid)
    ref = sequential(attn, inputs)
    outs = [torch.empty_like(inputs[0][0]) for _ in inputs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    errors = []

    def worker(j):
        try:
            for i in range(j, len(inputs), 2):
                q, k, v = inputs[i]
                for _ in range(4):
                    attn.forward(q, k, v, out=outs[i], stream=streams[j])
        except Exception as e:  # surfaced in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(j,)) for j in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    attn.close()
    assert not errors, errors
    for i in range(len(inputs)):
        assert torch.equal(outs[i], ref[i]), i


def test_block_on_two_streams_unordered():
    w = synth.WORKLOADS["block_12x128_n1560"]
    say("case attention block on two streams")
    sets = [synth.make_block_inputs(w, 0, b, device="cuda") for b in range(4)]
    blk = native.Block(w.heads, w.head_dim, w.grid)
    ref = [blk.forward(*s) for s in sets]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = [torch.empty_like(sets[0][0]) for _ in sets]
    for i, s in enumerate(sets):
        blk.forward(*s, out=outs[i], stream=streams[i % 2])
    for s in streams:
        torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    blk.close()
    for i in range(len(sets)):
        assert torch.equal(outs[i], ref[i]), i
