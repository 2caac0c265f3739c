"""Every access of every launch configuration the library makes stays inside
its buffer: a CPU replay (tests/launch_replay.py) of the host's launch
decisions and of each kernel's address arithmetic, at the five workloads'
full sizes, the ranged and token-major calls, the attention block at 128,
1560 and 10920 tokens, and the GEMM shapes of the linear-layer tests. Also
checks the invariants the schedule relies on: every (query tile, key block)
pair is computed exactly once, every split tile's parts are written to
distinct slots and read back by the merge from exactly those slots, and
every GEMM output element is stored exactly once.
"""
import numpy as np
import pytest

import launch_replay as R
from diffusion_transformer_attention_dit_amd import synth

# Resident attention workgroups: one per CU on MI355X (256); other counts
# cover other devices and the clamp P = min(slots, units).
P_VALUES = (256, 1, 7, 80, 304)


def handle_P(slots, heads, tokens):
    units = heads * -(-tokens // R.KBM) * -(-tokens // R.KBN)
    return min(slots, units)


@pytest.mark.parametrize("name", synth.ORDER)
@pytest.mark.parametrize("slots", P_VALUES)
def test_attention_forward_in_bounds(name, slots):
    w = synth.WORKLOADS[name]
    P = handle_P(slots, w.heads, w.tokens)
    R.attention_forward(w.heads, w.head_dim, w.tokens, P)


@pytest.mark.parametrize("slots", (256, 80))
def test_token_major_share_in_bounds(slots):
    w = synth.WORKLOADS["ulysses_share_3x128_n10920"]
    R.attention_forward(w.heads, w.head_dim, w.tokens, handle_P(slots, w.heads, w.tokens),
                        token_major=True)


@pytest.mark.parametrize("case", [
    # (q_begin, nq, kv_begin, nk): key halves of the window, ragged query runs
    (0, 10920, 0, 5460), (0, 10920, 5460, 5460), (100, 257, 3000, 65), (10919, 1, 0, 10920),
    (0, 1, 10919, 1),
])
def test_ranged_calls_in_bounds(case):
    w = synth.WORKLOADS["window25_12x128_n10920"]
    qb, nq, kb, nk = case
    P = handle_P(256, w.heads, w.tokens)
    R.attention_forward(w.heads, w.head_dim, w.tokens, P, q_begin=qb, nq=nq, kv_begin=kb, nk=nk,
                        lse=True)


@pytest.mark.parametrize("name", ["tiny_1x64_n128", "block_12x128_n1560", "window25_12x128_n10920"])
@pytest.mark.parametrize("slots", [(256, 512), (304, 608), (80, 160)])
def test_block_in_bounds(name, slots):
    """The self-attention block at its three tested sizes, including the
    25-frame window's 10920 tokens x 1536 hidden: QKV GEMM (10920 x 1536 ->
    4608: 774 tiles of 256 x 256, 6 of them as eighths), rope_k_vt and the
    attention on the fused projection output (token stride 3 x 1536), the
    split-tile merge, and the output GEMM (258 tiles, 2 as eighths)."""
    w = synth.WORKLOADS[name]
    big, small = slots
    P = handle_P(big, w.heads, w.tokens)
    buf = R.block_forward(w.heads, w.head_dim, w.tokens, P, big_slots=big, small_slots=small)
    # the attention's largest read reaches the last V element of the last token
    hid = w.heads * w.head_dim
    assert buf.touched["qkv"][1] == w.tokens * 3 * hid
    assert buf.touched["attn_out"][1] == w.tokens * hid


@pytest.mark.parametrize("rows,fin,fout", [
    (1, 64, 1), (37, 64, 100), (128, 128, 128), (1000, 256, 129), (300, 1536, 4608),
    (1560, 1536, 4608), (10920, 1536, 1536), (10920, 1536, 4608), (4100, 256, 2000),
    (4100, 256, 4100), (2600, 64, 9216), (4096, 128, 6144),
])
def test_gemm_in_bounds_and_covered(rows, fin, fout):
    buf = R.Buffers(x=rows * fin, w=fout * fin, y=rows * fout)
    R.gemm_call(buf, a_name="x", a_base=0, lda=fin, b_name="w", b_base=0, ldb=fin, c_name="y",
                c_base=0, ldc=fout, M=rows, N=fout, K=fin)
    assert buf.touched["y"] == [0, rows * fout]


def test_replay_detects_planted_overrun():
    """The replay itself must catch an access one element past a buffer."""
    buf = R.Buffers(a=100)
    buf.access("a", 0, 100, "ok")
    with pytest.raises(R.OutOfBounds):
        buf.access("a", 0, 101, "one past the end")
    with pytest.raises(R.OutOfBounds):
        buf.rsrc("a", 10, 182, 2, "resource one past the end")
    # a stride that overruns the fused projection output is caught
    w = synth.WORKLOADS["block_12x128_n1560"]
    hid = w.heads * w.head_dim
    tp = -(-w.tokens // R.PREP_KEYS) * R.PREP_KEYS
    bad = R.Buffers(qkv=w.tokens * 3 * hid, o=w.tokens * hid, kr=w.heads * tp * w.head_dim,
                    vt=w.heads * tp * w.head_dim, part_o=2 * 256 * R.KBM * w.head_dim,
                    part_ml=2 * 256 * R.KBM * 2)
    with pytest.raises(R.OutOfBounds):
        R.attention_call(bad, heads=w.heads, D=w.head_dim, nq=w.tokens, nk=w.tokens, tokens_pad=tp,
                         P=256, q_name="qkv", q_base=0, qh=w.head_dim, qn=3 * hid + 8, k_name="qkv",
                         k_base=hid, v_name="qkv", v_base=2 * hid, kh=w.head_dim, kn=3 * hid,
                         o_name="o", o_base=0, oh=w.head_dim, on=hid)


def test_claimed_pieces_where_the_leftover_is_small():
    """Whole-tile passes followed by a leftover of at most 8 key blocks per
    workgroup use claimed pieces (the 25-frame window); no whole-tile pass
    (3-head share, 1560 tokens) or a large leftover (77-frame clip) keep the
    static split. Pieces cover the leftover tiles exactly and fit 2P slots."""
    assert R.make_sched(12, 10920, 10920, 256)["dyn"] == 1
    for heads, n in ((3, 10920), (12, 1560), (12, 31200)):
        assert R.make_sched(heads, n, n, 256)["dyn"] == 0
    # short key runs (a 512-token cross-attention context) keep the static split
    assert R.make_sched(12, 10920, 512, 256)["dyn"] == 0
    for heads, n, P in ((12, 10920, 256), (2, 32800, 256), (12, 6400, 256), (12, 10920, 240)):
        sc = R.make_sched(heads, n, n, P)
        if not sc["dyn"]:
            continue
        assert sc["npieces"] <= 2 * P
        covered = {}
        for i in range(sc["npieces"]):
            t, kv0, kv1 = R.piece_segment(sc, i)
            for b in range(kv0, kv1):
                assert (t, b) not in covered
                covered[(t, b)] = i
        assert len(covered) == sc["rem_tiles"] * sc["nkv"]
    assert R.make_sched(2, 32800, 32800, 256)["dyn"] == 1
    R.attention_forward(2, 128, 32800, 256)  # every access of that call in bounds


def test_schedule_replay_matches_closed_forms():
    """The leftover ranges partition the leftover units: rem_begin is
    floor(p * units / Prem) for every p, and rem_owner inverts it."""
    for heads, n, P in ((12, 10920, 256), (3, 10920, 256), (12, 31200, 256), (1, 128, 2), (12, 1560, 256)):
        sc = R.make_sched(heads, n, n, P)
        if sc["rem_units"] == 0:
            continue
        for p in range(sc["Prem"] + 1):
            assert R.rem_begin(sc, p) == p * sc["rem_units"] // sc["Prem"]
        for y in np.linspace(0, sc["rem_units"] - 1, 200).astype(int):
            p = R.rem_owner(sc, int(y))
            assert R.rem_begin(sc, p) <= y < R.rem_begin(sc, p + 1)
