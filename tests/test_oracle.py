"""Pins of the fp64 oracle against what the definition and mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
closed form, an invariant of exact softmax attention or of rotary embeddings,
a library routine for a special case, an independently written brute force,
or a hand-derived fixture (tests/golden). A plausible slip in the oracle (a
dropped scale, a wrong sign, a transposed operand, the wrong axis, pairing or
token order) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from diffusion_transformer_attention_dit_amd import synth

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(12345)


def _rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# --------------------------------------------------------------------------
# Token order and positions
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n,grid,expect", [
    (0, (2, 8, 8), (0, 0, 0)),
    (1, (2, 8, 8), (0, 0, 1)),
    (8, (2, 8, 8), (0, 1, 0)),
    (64, (2, 8, 8), (1, 0, 0)),
    (127, (2, 8, 8), (1, 7, 7)),
    (26 * 15 + 26 + 3, (4, 15, 26), (1, 1, 3)),
    (10919, (7, 30, 52), (6, 29, 51)),
])
def test_token_coords_hand_cases(n, grid, expect):
    assert oracle.token_coords(n, grid) == expect


def test_token_coords_match_numpy_positions():
    grid = (4, 15, 26)
    pos = oracle.np_positions(grid)
    for n in range(0, grid[0] * grid[1] * grid[2], 37):
        assert tuple(int(x) for x in pos[n]) == oracle.token_coords(n, grid)


def test_default_pairs_split():
    assert oracle.default_pairs(128) == (22, 21, 21)
    assert oracle.default_pairs(64) == (12, 10, 10)


# --------------------------------------------------------------------------
# Rotary embedding
# --------------------------------------------------------------------------

def test_rope_position_zero_is_identity_exactly():
    x = _rand(4, 128)
    y = oracle.c_rope_positions(x, np.zeros((4, 3)))
    assert np.array_equal(x, y)


@pytest.mark.parametrize("pos,pair,angle", [
    ((1, 0, 0), 0, 1.0),   # t axis, pair 0
    ((0, 2, 0), 1, 2.0),   # h axis, pair 1
    ((0, 0, 3), 2, 3.0),   # w axis, pair 2
])
def test_rope_hand_case_d6(pos, pair, angle):
    # head_dim 6, one pair per axis: theta = base^0 = 1, so pair a turns by
    # exactly pos_a radians, counter-clockwise, and the others stay put.
    for comp in (0, 1):
        x = np.zeros((1, 6))
        x[0, 2 * pair + comp] = 1.0
        y = oracle.c_rope_positions(x, np.array([pos], dtype=float), pairs=(1, 1, 1))
        c, s = math.cos(angle), math.sin(angle)
        want = np.zeros(6)
        if comp == 0:
            want[2 * pair], want[2 * pair + 1] = c, s
        else:
            want[2 * pair], want[2 * pair + 1] = -s, c
        assert np.allclose(y[0], want, atol=1e-15, rtol=0)


def test_rope_hand_case_ladder_d12():
    # pairs 2/2/2, base 10000: the second pair of each axis has
    # theta = 10000^(-1/2) = 0.01, so positions (5, 7, 9) turn pairs 1, 3, 5
    # by 0.05, 0.07, 0.09 rad and pairs 0, 2, 4 by 5, 7, 9 rad.
    x = np.zeros((1, 12))
    x[0, 0::2] = 1.0
    y = oracle.c_rope_positions(x, np.array([[5.0, 7.0, 9.0]]), pairs=(2, 2, 2))
    angles = [5.0, 0.05, 7.0, 0.07, 9.0, 0.09]
    for i, a in enumerate(angles):
        assert y[0, 2 * i] == pytest.approx(math.cos(a), abs=1e-15)
        assert y[0, 2 * i + 1] == pytest.approx(math.sin(a), abs=1e-15)


def test_rope_ladder_per_axis_d128():
    # At d=128 (22/21/21) pair 22 is the first pair of the h axis: theta = 1.
    # Pair 21 is the last of the t axis: theta = 10000^(-21/22).
    x = np.zeros((1, 128))
    x[0, 0::2] = 1.0
    y = oracle.c_rope_positions(x, np.array([[3.0, 2.0, 1.0]]))
    assert y[0, 44] == pytest.approx(math.cos(2.0), abs=1e-15)
    assert y[0, 42] == pytest.approx(math.cos(3.0 * 10000 ** (-21 / 22)), abs=1e-15)
    assert y[0, 86] == pytest.approx(math.cos(1.0), abs=1e-15)  # pair 43: first w pair


def test_rope_preserves_pair_norms():
    x = _rand(64, 128)
    pos = RNG.uniform(0, 60, size=(64, 3))
    y = oracle.c_rope_positions(x, pos)
    nx = np.hypot(x[:, 0::2], x[:, 1::2])
    ny = np.hypot(y[:, 0::2], y[:, 1::2])
    assert np.max(np.abs(nx - ny) / nx) < 1e-14


def test_rope_composition():
    x = _rand(16, 128)
    p1 = RNG.integers(0, 30, size=(16, 3)).astype(float)
    p2 = RNG.integers(0, 30, size=(16, 3)).astype(float)
    twice = oracle.c_rope_positions(oracle.c_rope_positions(x, p1), p2)
    once = oracle.c_rope_positions(x, p1 + p2)
    assert np.max(np.abs(twice - once)) < 1e-12


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_rope_relative_position_invariance(axis):
    # Scores of rotated vectors depend only on position differences.
    q = _rand(24, 128)
    k = _rand(24, 128)
    pq = RNG.integers(0, 20, size=(24, 3)).astype(float)
    pk = RNG.integers(0, 20, size=(24, 3)).astype(float)
    s0 = oracle.c_rope_positions(q, pq) @ oracle.c_rope_positions(k, pk).T
    shift = np.zeros(3)
    shift[axis] = 13.0
    s1 = oracle.c_rope_positions(q, pq + shift) @ oracle.c_rope_positions(k, pk + shift).T
    assert np.max(np.abs(s0 - s1)) < 1e-12


def test_c_rope_matches_numpy_complex_rope():
    for grid, d in (((4, 15, 26), 128), ((2, 8, 8), 64)):
        x = _rand(2, grid[0] * grid[1] * grid[2], d)
        a = oracle.c_rope_grid(x, grid)
        b = oracle.np_rope(x, grid)
        assert np.max(np.abs(a - b)) < 1e-13


def test_rope_rejects_bad_split():
    with pytest.raises(ValueError):
        oracle.c_rope_positions(_rand(1, 128), np.zeros((1, 3)), pairs=(22, 22, 21))


# --------------------------------------------------------------------------
# Exact attention
# --------------------------------------------------------------------------

def test_softmax_rows_sum_to_one_numpy():
    q, k, v = _rand(2, 200, 64), _rand(2, 200, 64), _rand(2, 200, 64)
    _, p = oracle.np_attention(q, k, v, return_probs=True)
    assert np.max(np.abs(p.sum(-1) - 1.0)) < 1e-13


def test_v_all_ones_gives_ones():
    q, k = _rand(3, 300, 128, scale=2.0), _rand(3, 300, 128, scale=2.0)
    v = np.ones((3, 300, 128))
    o = oracle.c_attention(q, k, v)
    assert np.max(np.abs(o - 1.0)) < 1e-13


def test_identical_keys_give_mean_of_v():
    q = _rand(2, 100, 64)
    k = np.repeat(_rand(2, 1, 64), 100, axis=1)
    v = _rand(2, 100, 64)
    o = oracle.c_attention(q, k, v)
    mean = v.mean(axis=1, keepdims=True)
    assert np.max(np.abs(o - mean)) < 1e-13


def test_one_hot_selection():
    # N <= d distinct unit keys; q_m = alpha * k_j(m). Off-target weights are
    # each exp(-alpha/sqrt(d)) of the target's, so the error is bounded by
    # (N-1) * exp(-alpha/sqrt(d)) * max|v|.
    d, n, alpha = 64, 48, 40.0 * 8.0
    k = np.zeros((1, n, d))
    k[0, np.arange(n), np.arange(n)] = 1.0
    target = RNG.permutation(n)
    q = alpha * k[:, target, :]
    v = _rand(1, n, d)
    o = oracle.c_attention(q, k, v)
    bound = (n - 1) * math.exp(-alpha / math.sqrt(d)) * np.abs(v).max()
    assert np.max(np.abs(o[0] - v[0, target])) <= bound + 1e-15


def test_permuting_keys_and_values_together():
    q, k, v = _rand(2, 257, 128), _rand(2, 257, 128), _rand(2, 257, 128)
    perm = RNG.permutation(257)
    o1 = oracle.c_attention(q, k, v)
    o2 = oracle.c_attention(q, k[:, perm], v[:, perm])
    assert np.max(np.abs(o1 - o2)) < 1e-13


def test_no_rope_matches_torch_sdpa_fp64():
    q, k, v = (torch.from_numpy(_rand(3, 333, 128)) for _ in range(3))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()
    o = oracle.c_attention(q.numpy(), k.numpy(), v.numpy())
    assert np.max(np.abs(o - ref)) < 1e-12


def test_scale_is_inverse_sqrt_head_dim():
    # Two keys: q.k1 = a, q.k2 = 0 -> weight of v1 is 1 / (1 + exp(-a/sqrt(d))).
    d = 64
    q = np.zeros((1, 1, d)); q[0, 0, 0] = 3.0
    k = np.zeros((1, 2, d)); k[0, 0, 0] = 2.0
    v = np.zeros((1, 2, d)); v[0, 0, 0] = 1.0
    o = oracle.c_attention(q, k, v)
    assert o[0, 0, 0] == pytest.approx(1.0 / (1.0 + math.exp(-6.0 / 8.0)), abs=1e-15)


def test_large_logits_do_not_overflow():
    q, k, v = _rand(1, 64, 64, scale=30.0), _rand(1, 64, 64, scale=30.0), _rand(1, 64, 64)
    o = oracle.c_attention(q, k, v)
    assert np.all(np.isfinite(o))
    ref = oracle.np_attention(q, k, v)
    assert np.max(np.abs(o - ref)) < 1e-12


# --------------------------------------------------------------------------
# Whole path: C oracle vs independent brute force, and the golden fixture
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny_1x64_n128", "block_12x128_n1560"])
def test_c_oracle_matches_numpy_brute_force(name):
    w = synth.WORKLOADS[name]
    heads = w.heads if name.startswith("tiny") else 2
    q, k, v = (t.double().numpy() for t in synth.make_qkv(w, dtype=torch.float32, heads=heads))
    a = oracle.rope_attention(q, k, v, w.grid)
    b = oracle.np_rope_attention(q, k, v, w.grid)
    assert np.max(np.abs(a - b)) < 1e-12


def test_row_subset_matches_full():
    w = synth.WORKLOADS["block_12x128_n1560"]
    q, k, v = (t.double().numpy() for t in synth.make_qkv(w, heads=2))
    rows = synth.sample_rows(w.tokens, 40, seed=3)
    full = oracle.rope_attention(q, k, v, w.grid)
    sub = oracle.rope_attention(q, k, v, w.grid, rows=rows)
    assert np.max(np.abs(full[:, rows] - sub)) < 1e-14


def test_pure_python_brute_force_tiny():
    # A third implementation with scalar loops and the math module only, on a
    # 12-token, head_dim 12 (pairs 2/2/2) case.
    grid, d, pairs, base = (3, 2, 2), 12, (2, 2, 2), 10000.0
    n = 12
    q, k, v = _rand(1, n, d), _rand(1, n, d), _rand(1, n, d)

    def rot(x, tok):
        t, h, w = tok // 4, (tok // 2) % 2, tok % 2
        p = (t, h, w)
        y = list(x)
        idx = 0
        for axis in range(3):
            for j in range(pairs[axis]):
                ang = p[axis] * base ** (-j / pairs[axis])
                a, b = x[2 * idx], x[2 * idx + 1]
                y[2 * idx] = a * math.cos(ang) - b * math.sin(ang)
                y[2 * idx + 1] = a * math.sin(ang) + b * math.cos(ang)
                idx += 1
        return y

    qr = [rot(q[0, m], m) for m in range(n)]
    kr = [rot(k[0, m], m) for m in range(n)]
    want = np.zeros((n, d))
    for m in range(n):
        s = [sum(qr[m][c] * kr[j][c] for c in range(d)) / math.sqrt(d) for j in range(n)]
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        den = sum(e)
        for c in range(d):
            want[m, c] = sum(e[j] * v[0, j, c] for j in range(n)) / den
    got = oracle.rope_attention(q, k, v, grid, pairs=pairs, base=base)
    assert np.max(np.abs(got[0] - want)) < 1e-13


def test_golden_closed_form_fixture():
    with open(os.path.join(HERE, "golden", "rope_attention_closed_form.json")) as f:
        g = json.load(f)
    q, k, v, o = (np.array(g[x]) for x in ("q", "k", "v", "o"))
    got_c = oracle.rope_attention(q, k, v, tuple(g["grid"]), pairs=tuple(g["pairs"]),
                                  base=g["base"])
    got_np = oracle.np_rope_attention(q, k, v, tuple(g["grid"]), pairs=tuple(g["pairs"]),
                                      base=g["base"])
    assert np.max(np.abs(got_c - o)) < 1e-13
    assert np.max(np.abs(got_np - o)) < 1e-13


# --------------------------------------------------------------------------
# Log-sum-exp output and the merge of results over disjoint key sets (what
# the Ring half of USP needs to stay exact: blog summary, "Methodology - deep
# read", USP paragraph, and "Technical innovations").
# --------------------------------------------------------------------------

def test_lse_zero_query_is_log_n_exactly():
    # q = 0: every score is 0, so lse = log(n_kv) and o = mean(v).
    n = 37
    q = np.zeros((2, 3, 16))
    k, v = _rand(2, n, 16), _rand(2, n, 16)
    o, lse = oracle.c_attention(q, k, v, return_lse=True)
    assert np.array_equal(lse, np.full((2, 3), math.log(n)))
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape),
                               rtol=0, atol=1e-14)


def test_lse_single_key_is_the_score():
    q, k, v = _rand(1, 4, 8), _rand(1, 1, 8), _rand(1, 1, 8)
    o, lse = oracle.c_attention(q, k, v, scale=0.3, return_lse=True)
    np.testing.assert_allclose(lse, 0.3 * (q @ k.transpose(0, 2, 1))[..., 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(o, np.broadcast_to(v, o.shape), rtol=0, atol=1e-15)


def test_lse_identical_keys():
    # n copies of one key: lse = s + log(n).
    n = 50
    q = _rand(1, 3, 8)
    k = np.broadcast_to(_rand(1, 1, 8), (1, n, 8)).copy()
    _, lse = oracle.c_attention(q, k, _rand(1, n, 8), return_lse=True)
    s = (q @ k[:, :1].transpose(0, 2, 1))[..., 0] / math.sqrt(8)
    np.testing.assert_allclose(lse, s + math.log(n), rtol=0, atol=1e-13)


def test_lse_matches_scipy_logsumexp():
    from scipy.special import logsumexp
    q, k, v = _rand(3, 20, 32, scale=2.0), _rand(3, 45, 32, scale=2.0), _rand(3, 45, 32)
    _, lse = oracle.c_attention(q, k, v, return_lse=True)
    s = (q @ k.transpose(0, 2, 1)) / math.sqrt(32)
    np.testing.assert_allclose(lse, logsumexp(s, axis=-1), rtol=0, atol=1e-12)


def test_lse_large_logits_stay_finite():
    q, k, v = _rand(1, 5, 16, scale=60.0), _rand(1, 30, 16, scale=60.0), _rand(1, 30, 16)
    o, lse = oracle.c_attention(q, k, v, return_lse=True)
    s = (q @ k.transpose(0, 2, 1)) / 4.0
    assert np.all(np.isfinite(lse)) and np.all(np.isfinite(o))
    # lse lies in [max s, max s + log n]
    assert np.all(lse >= s.max(axis=-1) - 1e-9) and np.all(lse <= s.max(axis=-1) + math.log(30) + 1e-9)


@pytest.mark.parametrize("cuts", [[17], [1], [44], [5, 20, 33], [10, 11, 12, 13]])
def test_merge_of_key_chunks_equals_full_attention(cuts):
    # Blockwise softmax: attention over all keys is the merge of attention
    # over any partition of the keys into runs.
    q, k, v = _rand(2, 9, 16), _rand(2, 45, 16), _rand(2, 45, 16)
    o_full, lse_full = oracle.c_attention(q, k, v, return_lse=True)
    edges = [0] + cuts + [45]
    parts = [oracle.c_attention(q, k[:, a:b], v[:, a:b], return_lse=True)
             for a, b in zip(edges[:-1], edges[1:])]
    o, lse = oracle.c_merge([p[0] for p in parts], [p[1] for p in parts])
    np.testing.assert_allclose(o, o_full, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_full, rtol=0, atol=1e-13)


def test_merge_of_non_contiguous_key_sets():
    # Any disjoint split works, not only runs: interleaved keys.
    q, k, v = _rand(1, 6, 8), _rand(1, 30, 8), _rand(1, 30, 8)
    o_full, lse_full = oracle.c_attention(q, k, v, return_lse=True)
    a = oracle.c_attention(q, k[:, 0::2], v[:, 0::2], return_lse=True)
    b = oracle.c_attention(q, k[:, 1::2], v[:, 1::2], return_lse=True)
    o, lse = oracle.c_merge([a[0], b[0]], [a[1], b[1]])
    np.testing.assert_allclose(o, o_full, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, lse_full, rtol=0, atol=1e-13)


def test_merge_special_cases():
    o1, o2 = _rand(4, 8), _rand(4, 8)
    l1, l2 = _rand(4), _rand(4)
    # one part: identity
    o, lse = oracle.c_merge([o1], [l1])
    assert np.array_equal(o, o1) and np.array_equal(lse, l1)
    # equal weights: the mean, lse + log 2
    o, lse = oracle.c_merge([o1, o2], [l1, l1])
    np.testing.assert_allclose(o, (o1 + o2) / 2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, l1 + math.log(2), rtol=0, atol=1e-15)
    # an empty part (lse = -inf) has no weight
    o, lse = oracle.c_merge([o1, o2], [l1, np.full(4, -np.inf)])
    np.testing.assert_allclose(o, o1, rtol=0, atol=0)
    np.testing.assert_allclose(lse, l1, rtol=0, atol=0)
    # order of the parts does not matter
    a = oracle.c_merge([o1, o2], [l1, l2])
    b = oracle.c_merge([o2, o1], [l2, l1])
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-15)
    # a part 40 nats below the other is negligible
    o, _ = oracle.c_merge([o1, o2], [l1, l1 - 40.0])
    np.testing.assert_allclose(o, o1, rtol=0, atol=1e-15)


def test_merge_rejects_all_empty_row():
    with pytest.raises(ValueError):
        oracle.c_merge([_rand(2, 4)], [np.array([0.0, -np.inf])])


def test_c_merge_matches_numpy_merge():
    o_parts = [_rand(3, 5, 16) for _ in range(4)]
    lse_parts = [_rand(3, 5, scale=5.0) for _ in range(4)]
    a = oracle.c_merge(o_parts, lse_parts)
    b = oracle.np_merge(o_parts, lse_parts)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-13)


def test_range_attention_matches_full_grid():
    # Rotating a run of tokens at its own grid places equals slicing the
    # rotation of the whole window: the ranged oracle agrees with the full
    # one on the rows and keys it covers, and merging key halves restores
    # the full result.
    w = synth.WORKLOADS["tiny_1x64_n128"]
    q, k, v = (t.double().numpy() for t in synth.make_qkv(w, 0, 0, device="cpu"))
    o_full, lse_full = oracle.rope_attention(q, k, v, w.grid, return_lse=True)
    qa, qb, ka, kb = 30, 90, 40, 128
    o_r, lse_r = oracle.rope_attention_range(q[:, qa:qb], k[:, ka:kb], v[:, ka:kb], w.grid,
                                             q_begin=qa, kv_begin=ka)
    o_a, lse_a = oracle.rope_attention_range(q[:, qa:qb], k[:, :ka], v[:, :ka], w.grid,
                                             q_begin=qa, kv_begin=0)
    o_m, lse_m = oracle.c_merge([o_r, o_a], [lse_r, lse_a])
    np.testing.assert_allclose(o_m, o_full[:, qa:qb], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse_m, lse_full[:, qa:qb], rtol=0, atol=1e-12)
    # and the NumPy brute force over the same key run
    qr = oracle.np_rope(q, w.grid)[:, qa:qb]
    kr = oracle.np_rope(k, w.grid)[:, ka:kb]
    np.testing.assert_allclose(o_r, oracle.np_attention(qr, kr, v[:, ka:kb]), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# Ulysses layouts (the on-device halves of the all-to-all)
# --------------------------------------------------------------------------

def test_ulysses_pack_unpack_elementwise_brute_force():
    # Every element checked by index arithmetic written out in Python loops.
    nl, h, d, groups = 5, 6, 4, 3
    hg = h // groups
    x = np.arange(nl * h * d).reshape(nl, h, d)
    send = oracle.ulysses_pack(x, groups)
    for g in range(groups):
        for i in range(nl):
            for j in range(hg):
                for c in range(d):
                    assert send[g, i, j, c] == x[i, g * hg + j, c]
    y = oracle.ulysses_unpack(send)
    for i in range(nl):
        for hh in range(h):
            for c in range(d):
                assert y[i, hh, c] == send[hh // hg, i, hh % hg, c]
    assert np.array_equal(y, x)  # unpack undoes pack


@pytest.mark.parametrize("groups", [1, 2, 3, 4, 12])
def test_ulysses_exchange_turns_token_shards_into_head_shards(groups):
    # The defining property: after pack + all-to-all, device g holds all N
    # tokens (in order) of head group g, i.e. X[:, g*Hg:(g+1)*Hg].
    n, h, d = 24, 12, 8
    x = RNG.standard_normal((n, h, d))
    nl, hg = n // groups, h // groups
    sends = [oracle.ulysses_pack(x[s * nl:(s + 1) * nl], groups) for s in range(groups)]
    recvs = oracle.ulysses_exchange(sends)
    for g in range(groups):
        assert np.array_equal(recvs[g].reshape(n, hg, d), x[:, g * hg:(g + 1) * hg])
    # and the reverse path (O in the same layout) restores the token shards
    back = oracle.ulysses_exchange([r.reshape(n, hg, d).reshape(groups, nl, hg, d) for r in recvs])
    for s in range(groups):
        assert np.array_equal(oracle.ulysses_unpack(back[s]), x[s * nl:(s + 1) * nl])


def test_ulysses_attention_equals_full_attention():
    # Attention per head group on the exchanged (token-major) layout, sent
    # back and unpacked, equals attention of the whole tensor.
    w = synth.WORKLOADS["tiny_1x64_n128"]
    groups, heads = 2, 4
    qkv = [RNG.standard_normal((w.tokens, heads, w.head_dim)) for _ in range(3)]
    nl, hg = w.tokens // groups, heads // groups
    full = oracle.rope_attention(*(t.transpose(1, 0, 2) for t in qkv), w.grid)  # [H, N, d]
    recvs = [oracle.ulysses_exchange([oracle.ulysses_pack(t[s * nl:(s + 1) * nl], groups)
                                      for s in range(groups)]) for t in qkv]
    outs = []
    for g in range(groups):
        q, k, v = (r[g].reshape(w.tokens, hg, w.head_dim).transpose(1, 0, 2) for r in recvs)
        outs.append(oracle.rope_attention(q, k, v, w.grid).transpose(1, 0, 2)
                    .reshape(groups, nl, hg, w.head_dim))
    back = oracle.ulysses_exchange(outs)
    got = np.concatenate([oracle.ulysses_unpack(back[s]) for s in range(groups)])  # [N, H, d]
    np.testing.assert_allclose(got, full.transpose(1, 0, 2), rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# Self-attention block with projections
# --------------------------------------------------------------------------

def _block_case(heads=2, d=8, grid=(2, 3, 4)):
    n = grid[0] * grid[1] * grid[2]
    x = RNG.standard_normal((n, heads * d))
    w_qkv = RNG.standard_normal((3 * heads * d, heads * d)) / math.sqrt(heads * d)
    w_o = RNG.standard_normal((heads * d, heads * d)) / math.sqrt(heads * d)
    return x, w_qkv, w_o, grid, heads, d


def test_block_with_identity_projections_is_attention_of_x():
    # W_qkv = [I; I; I], W_o = I: the block is attention(x, x, x) laid out
    # token-major, which pins the Q/K/V column order and the head layout.
    x, _, _, grid, heads, d = _block_case()
    hid = heads * d
    eye = np.eye(hid)
    y = oracle.block_forward(x, np.concatenate([eye, eye, eye], axis=0), eye, grid, heads,
                             pairs=(2, 1, 1))
    xh = x.reshape(-1, heads, d).transpose(1, 0, 2)
    ref = oracle.np_rope_attention(xh, xh, xh, grid, pairs=(2, 1, 1))  # [H, N, d]
    np.testing.assert_allclose(y, ref.transpose(1, 0, 2).reshape(-1, hid), rtol=0, atol=1e-13)


def test_block_column_roles():
    # Zeroing the V rows of W_qkv zeroes Y; scaling W_o scales Y; permuting
    # the rows of W_o permutes the columns of Y.
    x, w_qkv, w_o, grid, heads, d = _block_case()
    hid = heads * d
    w0 = w_qkv.copy()
    w0[2 * hid:, :] = 0.0
    assert np.abs(oracle.block_forward(x, w0, w_o, grid, heads, pairs=(2, 1, 1))).max() == 0.0
    y = oracle.block_forward(x, w_qkv, w_o, grid, heads, pairs=(2, 1, 1))
    np.testing.assert_allclose(oracle.block_forward(x, w_qkv, 3.0 * w_o, grid, heads, pairs=(2, 1, 1)),
                               3.0 * y, rtol=1e-13, atol=1e-14)
    perm = RNG.permutation(hid)
    np.testing.assert_allclose(oracle.block_forward(x, w_qkv, w_o[perm, :], grid, heads,
                                                    pairs=(2, 1, 1)), y[:, perm], rtol=0, atol=1e-14)


def test_block_pure_python_brute_force():
    # Every product written as Python loops over scalars (no matmul, no
    # NumPy attention) on a tiny case.
    x, w_qkv, w_o, grid, heads, d = _block_case(heads=2, d=6, grid=(2, 2, 3))
    n, hid = x.shape
    y = oracle.block_forward(x, w_qkv, w_o, grid, heads)
    P = (1, 1, 1)  # the default split at d = 6
    qkv = [[sum(x[i][c] * w_qkv[j][c] for c in range(hid)) for j in range(3 * hid)] for i in range(n)]
    coords = [(i // (grid[1] * grid[2]), (i // grid[2]) % grid[1], i % grid[2]) for i in range(n)]

    def rot(vec, pos):
        out = list(vec)
        for p_ in range(d // 2):
            axis = 0 if p_ < P[0] else (1 if p_ < P[0] + P[1] else 2)
            j = p_ - (0 if axis == 0 else (P[0] if axis == 1 else P[0] + P[1]))
            ang = pos[axis] * 10000.0 ** (-j / P[axis])
            a, b = vec[2 * p_], vec[2 * p_ + 1]
            out[2 * p_] = a * math.cos(ang) - b * math.sin(ang)
            out[2 * p_ + 1] = a * math.sin(ang) + b * math.cos(ang)
        return out

    o = [[0.0] * hid for _ in range(n)]
    for h in range(heads):
        for i in range(n):
            qi = rot([qkv[i][h * d + c] for c in range(d)], coords[i])
            sc = []
            for j in range(n):
                kj = rot([qkv[j][hid + h * d + c] for c in range(d)], coords[j])
                sc.append(sum(qi[c] * kj[c] for c in range(d)) / math.sqrt(d))
            mx = max(sc)
            e = [math.exp(s - mx) for s in sc]
            z = sum(e)
            for c in range(d):
                o[i][h * d + c] = sum(e[j] * qkv[j][2 * hid + h * d + c] for j in range(n)) / z
    ref = [[sum(o[i][c] * w_o[j][c] for c in range(hid)) for j in range(hid)] for i in range(n)]
    np.testing.assert_allclose(y, np.array(ref), rtol=0, atol=1e-12)
