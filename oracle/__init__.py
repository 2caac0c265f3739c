"""fp64 CPU oracle for the 3D-RoPE exact self-attention of the ReGenVC DiT.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check in
``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py`` may import
this package. The HIP library never imports, links or calls it, and the two
share no code: the only thing both sides see are the seeded inputs.

Two independent implementations live here, both in float64:

* ``c_rope_grid`` / ``c_rope_positions`` / ``c_attention``: the C
  oracle (``regen_oracle.c``, OpenMP over (head, row)), fast enough for row
  samples of the full-window shapes;
* ``np_rope`` / ``np_attention``: NumPy brute force written a second way
  (complex multiplication for the rotation, the explicit N x N probability
  matrix for the softmax), for small shapes.

What the oracle computes (the pages give no equation, so each step cites the
passage it rests on; the readings are listed in ``regen_oracle.c``):

* exact, non-causal softmax attention per head over the whole token sequence
  of one window -- "Technical innovations" of the blog summary (USP keeps
  attention exact and numerically equivalent) and the Methodology paragraph
  on Ulysses/Ring, which reshuffle the sequence into attention heads;
* FlashAttention / FlashAttention-2 (index page, "Builds on") reach this same
  exact result with tiling, which is why the oracle is the plain definition;
* a rotary position embedding over the (t, h, w) latent coordinates applied
  to Q and K before the product (conventions fixed by the readings in
  ``regen_oracle.c``; parity unpinned against the pages, which print no
  rotary values).
"""
import ctypes
import math
import os

import numpy as np

from . import build_oracle

_LIB = None


def load():
    """Load (building first if absent) the C oracle library."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(build_oracle.LIB):
        build_oracle.build()
    lib = ctypes.CDLL(build_oracle.LIB)
    dp = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_rope_grid.argtypes = [dp, dp] + [ctypes.c_int] * 8 + [ctypes.c_double]
    lib.oracle_rope_grid.restype = ctypes.c_int
    lib.oracle_rope_positions.argtypes = [dp, dp, ctypes.c_int64, ctypes.c_int, dp,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double]
    lib.oracle_rope_positions.restype = ctypes.c_int
    lib.oracle_attention.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_int, ctypes.c_double]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_attention_lse.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_double]
    lib.oracle_attention_lse.restype = ctypes.c_int
    lib.oracle_merge.argtypes = [ctypes.POINTER(dp), ctypes.POINTER(dp), ctypes.c_int,
                                 ctypes.c_int64, ctypes.c_int, dp, dp]
    lib.oracle_merge.restype = ctypes.c_int
    lib.oracle_token_coords.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        i64p, i64p, i64p]
    lib.oracle_token_coords.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _LIB = lib
    return lib


def _dptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def default_pairs(head_dim):
    """Rotary pairs per axis: h and w get floor((d/2)/3) each, t the rest.

    Gives 22/21/21 at head_dim 128 (the split the workload names) and
    12/10/10 at head_dim 64, where 22/21/21 cannot fit in 32 pairs.
    """
    half = head_dim // 2
    ph = half // 3
    return (half - 2 * ph, ph, ph)


def num_threads():
    return load().oracle_num_threads()


def token_coords(n, grid):
    """(t, h, w) of token n on grid (T, H, W), via the C oracle."""
    lib = load()
    t, h, w = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    lib.oracle_token_coords(int(n), int(grid[1]), int(grid[2]),
                            ctypes.byref(t), ctypes.byref(h), ctypes.byref(w))
    return t.value, h.value, w.value


def c_rope_grid(x, grid, pairs=None, base=10000.0):
    """Rotate x [heads, T*H*W, d] over the latent grid (C oracle)."""
    x = _f64(x)
    heads, n, d = x.shape
    pairs = tuple(pairs) if pairs is not None else default_pairs(d)
    assert n == grid[0] * grid[1] * grid[2]
    y = np.empty_like(x)
    rc = load().oracle_rope_grid(_dptr(x), _dptr(y), heads, d, grid[0], grid[1], grid[2],
                                 pairs[0], pairs[1], pairs[2], float(base))
    if rc != 0:
        raise ValueError("oracle_rope_grid rejected its arguments (rc=%d)" % rc)
    return y


def c_rope_positions(x, pos, pairs=None, base=10000.0):
    """Rotate rows x [R, d] at explicit positions pos [R, 3] (C oracle)."""
    x = _f64(x)
    pos = _f64(pos)
    r, d = x.shape
    assert pos.shape == (r, 3)
    pairs = tuple(pairs) if pairs is not None else default_pairs(d)
    y = np.empty_like(x)
    rc = load().oracle_rope_positions(_dptr(x), _dptr(y), r, d, _dptr(pos),
                                      pairs[0], pairs[1], pairs[2], float(base))
    if rc != 0:
        raise ValueError("oracle_rope_positions rejected its arguments (rc=%d)" % rc)
    return y


def c_attention(q, k, v, scale=None, return_lse=False):
    """Exact attention of queries q [heads, R, d] against all keys k, v.

    With return_lse, also the log-sum-exp of each row's scores [heads, R]
    (natural log, scores including the scale)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    heads, r, d = q.shape
    n = k.shape[1]
    assert k.shape == (heads, n, d) and v.shape == (heads, n, d)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = np.empty((heads, r, d), dtype=np.float64)
    lse = np.empty((heads, r), dtype=np.float64) if return_lse else None
    rc = load().oracle_attention_lse(_dptr(q), _dptr(k), _dptr(v), _dptr(o),
                                     _dptr(lse) if return_lse else None, heads, r, n, d,
                                     float(scale))
    if rc != 0:
        raise ValueError("oracle_attention_lse failed (rc=%d)" % rc)
    return (o, lse) if return_lse else o


def c_merge(o_parts, lse_parts):
    """Combine attention results over disjoint key sets (C oracle).

    o_parts: list of [..., d] arrays; lse_parts: matching [...] arrays.
    Returns (o, lse) over the union of the key sets."""
    o_parts = [_f64(o) for o in o_parts]
    lse_parts = [_f64(l) for l in lse_parts]
    shape = o_parts[0].shape
    d = shape[-1]
    rows = int(np.prod(shape[:-1]))
    for o, l in zip(o_parts, lse_parts):
        assert o.shape == shape and l.shape == shape[:-1]
    dp = ctypes.POINTER(ctypes.c_double)
    op = (dp * len(o_parts))(*[_dptr(o) for o in o_parts])
    lp = (dp * len(lse_parts))(*[_dptr(l) for l in lse_parts])
    o = np.empty(shape, dtype=np.float64)
    lse = np.empty(shape[:-1], dtype=np.float64)
    rc = load().oracle_merge(op, lp, len(o_parts), rows, d, _dptr(o), _dptr(lse))
    if rc != 0:
        raise ValueError("oracle_merge failed (rc=%d)" % rc)
    return o, lse


def grid_positions(rows, grid):
    """[len(rows), 3] latent positions of the listed tokens (C oracle)."""
    return np.array([token_coords(int(m), grid) for m in rows], dtype=np.float64).reshape(-1, 3)


def rope_attention(q, k, v, grid, pairs=None, base=10000.0, scale=None, rows=None,
                   rope=True, return_lse=False):
    """The whole hot path in fp64: rotate Q and K over the latent grid, then
    exact softmax attention, for the query rows listed (all rows if None).

    Returns [heads, len(rows), d] (or [heads, N, d]), and with return_lse the
    rows' log-sum-exp [heads, len(rows)] too."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    heads, n, d = q.shape
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = np.ascontiguousarray(q[:, rows, :])
    if rope:
        if rows is None:
            q = c_rope_grid(q, grid, pairs, base)
        else:
            pos = np.tile(grid_positions(rows, grid), (heads, 1))
            q = c_rope_positions(q.reshape(-1, d), pos, pairs, base).reshape(q.shape)
        k = c_rope_grid(k, grid, pairs, base)
    return c_attention(q, k, v, scale, return_lse)


def rope_attention_range(q, k, v, grid, q_begin, kv_begin, pairs=None, base=10000.0,
                         scale=None, rows=None, rope=True):
    """Attention of a run of query tokens against a run of key tokens of one
    window, each rotated at its own place on the latent grid.

    q: [heads, nq, d] holds tokens q_begin .. q_begin+nq-1; k, v:
    [heads, nk, d] hold tokens kv_begin .. kv_begin+nk-1. rows (indices into
    q's nq rows) picks a sample of query rows. Returns (o [heads, R, d],
    lse [heads, R])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    heads, nq, d = q.shape
    nk = k.shape[1]
    rows = np.arange(nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    q = np.ascontiguousarray(q[:, rows, :])
    if rope:
        qpos = np.tile(grid_positions(rows + q_begin, grid), (heads, 1))
        q = c_rope_positions(q.reshape(-1, d), qpos, pairs, base).reshape(q.shape)
        kpos = np.tile(grid_positions(np.arange(nk) + kv_begin, grid), (heads, 1))
        k = c_rope_positions(k.reshape(-1, d), kpos, pairs, base).reshape(k.shape)
    return c_attention(q, k, v, scale, return_lse=True)


# ---------------------------------------------------------------------------
# Independent NumPy brute force (small shapes only).
# ---------------------------------------------------------------------------

def np_positions(grid):
    """[T*H*W, 3] positions, row-major with t slowest."""
    t, h, w = np.meshgrid(np.arange(grid[0]), np.arange(grid[1]), np.arange(grid[2]),
                          indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.float64)


def np_angles(pos, head_dim, pairs=None, base=10000.0):
    """[R, d/2] rotation angles: each axis its own ladder base^(-j/P_a)."""
    pairs = tuple(pairs) if pairs is not None else default_pairs(head_dim)
    cols = []
    for axis, p in enumerate(pairs):
        theta = base ** (-np.arange(p, dtype=np.float64) / p)
        cols.append(np.outer(pos[:, axis], theta))
    return np.concatenate(cols, axis=1)


def np_rope(x, grid=None, pairs=None, base=10000.0, pos=None):
    """Rotate x [..., R, d] by complex multiplication of interleaved pairs."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if pos is None:
        pos = np_positions(grid)
    phi = np_angles(np.asarray(pos, dtype=np.float64), d, pairs, base)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    z = z * np.exp(1j * phi)
    y = np.empty_like(x)
    y[..., 0::2] = z.real
    y[..., 1::2] = z.imag
    return y


def np_attention(q, k, v, scale=None, return_probs=False):
    """softmax(q k^T * scale) v with the full probability matrix."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    s = np.matmul(q, np.swapaxes(k, -1, -2)) * scale
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    o = np.matmul(p, v)
    return (o, p) if return_probs else o


def np_merge(o_parts, lse_parts):
    """Combine results over disjoint key sets, written a second way: the
    part weights are a softmax over the stacked LSEs."""
    lse = np.stack([np.asarray(l, dtype=np.float64) for l in lse_parts])  # [P, ...]
    o = np.stack([np.asarray(x, dtype=np.float64) for x in o_parts])      # [P, ..., d]
    top = lse.max(axis=0)
    w = np.exp(lse - top)
    z = w.sum(axis=0)
    merged = (w[..., None] * o).sum(axis=0) / z[..., None]
    return merged, top + np.log(z)


def np_rope_attention(q, k, v, grid, pairs=None, base=10000.0, scale=None, rope=True):
    if rope:
        q = np_rope(q, grid, pairs, base)
        k = np_rope(k, grid, pairs, base)
    return np_attention(q, k, v, scale)


# ---------------------------------------------------------------------------
# Ulysses layouts (blog summary, "Methodology - deep read", USP paragraph:
# Ulysses turns sequence shards into head shards with an all-to-all). Plain
# definitions, element by element in meaning: G devices, device s holding
# tokens s*Nl .. (s+1)*Nl - 1 of all H heads before the exchange, and all N
# tokens of heads g*H/G .. (g+1)*H/G - 1 after it.
# ---------------------------------------------------------------------------

def ulysses_pack(x, groups):
    """x [Nl, H, d] -> send [G, Nl, H/G, d] with send[g, i, j] = x[i, g*H/G + j]."""
    x = np.asarray(x)
    nl, h, d = x.shape
    hg = h // groups
    assert hg * groups == h
    send = np.empty((groups, nl, hg, d), dtype=x.dtype)
    for g in range(groups):
        send[g] = x[:, g * hg:(g + 1) * hg, :]
    return send


def ulysses_exchange(sends):
    """The all-to-all itself, simulated: device dst receives piece dst of
    every device's send buffer, in source order: recv[dst][src] = send[src][dst]."""
    groups = len(sends)
    return [np.stack([sends[src][dst] for src in range(groups)]) for dst in range(groups)]


def ulysses_unpack(recv):
    """recv [G, Nl, Hg, d] -> y [Nl, G*Hg, d] with y[i, g*Hg + j] = recv[g, i, j]."""
    recv = np.asarray(recv)
    groups, nl, hg, d = recv.shape
    y = np.empty((nl, groups * hg, d), dtype=recv.dtype)
    for g in range(groups):
        y[:, g * hg:(g + 1) * hg, :] = recv[g]
    return y


# ---------------------------------------------------------------------------
# One self-attention block of the DiT with synthetic weights (index page,
# "Abstract": the decoder is a diffusion transformer; the blocks' projection
# sizes are not on the pages and follow the 12 heads x 128 workload):
#   [Q | K | V] = X W_qkv^T,  O = attention(R Q, R K, V) per head,  Y = O W_o^T,
# X [N, H*d] token-major, weights in the [out][in] layout of a linear layer:
# W_qkv [3*H*d, H*d] (output rows: Q, then K, then V, head h at rows
# h*d .. h*d + d - 1 of each), W_o [H*d, H*d]; no biases.
# ---------------------------------------------------------------------------

def block_forward(x, w_qkv, w_o, grid, heads, pairs=None, base=10000.0, scale=None, rows=None):
    """fp64 block: returns Y [N, H*d] (or the listed rows of it)."""
    x, w_qkv, w_o = _f64(x), _f64(w_qkv), _f64(w_o)
    n, hidden = x.shape
    d = hidden // heads
    assert heads * d == hidden and w_qkv.shape == (3 * hidden, hidden)
    assert w_o.shape == (hidden, hidden)
    qkv = x @ w_qkv.T  # [N, 3*H*d]

    def head_major(cols):
        return np.ascontiguousarray(cols.reshape(n, heads, d).transpose(1, 0, 2))

    q = head_major(qkv[:, :hidden])
    k = head_major(qkv[:, hidden:2 * hidden])
    v = head_major(qkv[:, 2 * hidden:])
    o = rope_attention(q, k, v, grid, pairs, base, scale, rows=rows)  # [H, R, d]
    o_tok = o.transpose(1, 0, 2).reshape(o.shape[1], hidden)           # [R, H*d]
    return o_tok @ w_o.T
