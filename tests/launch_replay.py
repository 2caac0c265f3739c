"""Host-side replay of the library's launch decisions and of every kernel's
address arithmetic, for checking on the CPU that each access of a launch
configuration stays inside the buffer it belongs to.

Each function below restates, in Python integers, one piece of the library:
the schedule of the persistent attention kernel (regen::Sched, get_segment,
partial_slot, rem_owner in attention.hpp; make_sched in regen_attn.hip), the
choice of GEMM kernel and tiling (gemm() in regen_attn.hip, gemm_nt_kernel /
gemm_nt256_kernel in gemm.hpp), and the byte offsets that rope_k_vt_kernel,
attn_fwd_kernel, merge_kernel and the GEMM kernels read or write. A change to
one of those formulas must be made here too; the tests that use this module
then re-check every launch configuration the library makes.

Accesses are recorded as (buffer, first element, one past the last element)
ranges in bf16 / fp32 elements of the named buffer, or checked on the spot
against a buffer resource's byte extent (loads past it read zero, stores past
it are dropped, so only the extent itself must lie inside the allocation).
"""
import numpy as np

KBM, KBN, KNW = 256, 64, 8          # attention: query rows per tile, keys per block, waves
PREP_KEYS, PREP_BLOCK = 128, 64     # workspace padding unit, keys per rope_k_vt block
TAB_LDS = 3072                      # (cos, sin) entries attn_fwd_kernel keeps in LDS
PIECE_BLOCKS = 6                    # key blocks per claimed leftover piece (at least)
GEMM_TILE, GEMM_BK, GEMM_BIG = 128, 64, 256
LDS_BYTES = 160 * 1024


class OutOfBounds(AssertionError):
    pass


class Buffers:
    """Named allocations (element counts) and a record of the ranges touched."""

    def __init__(self, **sizes):
        self.size = dict(sizes)
        self.touched = {k: [np.iinfo(np.int64).max, -1] for k in sizes}

    def access(self, name, lo, hi, what):
        lo, hi = int(lo), int(hi)
        if lo < 0 or hi > self.size[name]:
            raise OutOfBounds("%s: [%d, %d) outside %s of %d elements" % (what, lo, hi, name, self.size[name]))
        t = self.touched[name]
        t[0], t[1] = min(t[0], lo), max(t[1], hi)

    def rsrc(self, name, base, nbytes, elem_bytes, what):
        """A buffer resource over [base, base + nbytes) (bytes from element `base`)."""
        if nbytes >= 1 << 32:
            raise OutOfBounds("%s: resource extent %d does not fit 32 bits" % (what, nbytes))
        self.access(name, base, base + -(-nbytes // elem_bytes), what + " (resource extent)")


# ---------------------------------------------------------------------------
# attention schedule (attention.hpp Sched and helpers; regen_attn.hip make_sched)
# ---------------------------------------------------------------------------

def make_sched(heads, nq, nk, P):
    n_qtiles, nkv = -(-nq // KBM), -(-nk // KBN)
    tiles = heads * n_qtiles
    if tiles * nkv >= 1 << 31:
        return None
    full = tiles // P
    rem_tiles = tiles - full * P
    rem_units = rem_tiles * nkv
    Prem = (rem_units if rem_units > 0 else 1) if rem_units < P else P
    sc = dict(n_qtiles=n_qtiles, nkv=nkv, P=P, full=full, Prem=Prem, rem_units=rem_units,
              rem_q=rem_units // Prem, rem_r=rem_units % Prem, rem_tiles=rem_tiles, dyn=0, ppt=1, npieces=0)
    # a small leftover after whole-tile passes: pieces claimed at run time
    if full >= 1 and rem_tiles > 0 and rem_units <= 8 * P and nkv >= 16 * PIECE_BLOCKS:
        ppt = min(max(nkv // PIECE_BLOCKS, 1), 2 * P // rem_tiles)
        sc.update(dyn=1, ppt=ppt, npieces=rem_tiles * ppt)
    return sc


def piece_segment(sc, i):
    r, j = divmod(i, sc["ppt"])
    return (i32(sc["full"] * sc["P"] + r), i32(j * sc["nkv"]) // sc["ppt"],
            i32((j + 1) * sc["nkv"]) // sc["ppt"])


def i32(x):
    """The value must fit a signed 32-bit int (the kernels compute in int)."""
    if not -(1 << 31) <= x < (1 << 31):
        raise OutOfBounds("32-bit overflow: %d" % x)
    return x


def rem_begin(sc, p):
    return i32(i32(p * sc["rem_q"]) + i32(p * sc["rem_r"]) // sc["Prem"])


def rem_owner(sc, y):
    return ((y + 1) * sc["Prem"] - 1) // sc["rem_units"]


def partial_slot(sc, p, t):
    x0 = i32(i32(sc["full"] * sc["P"] * sc["nkv"]) + rem_begin(sc, p))
    return 2 * p if t == x0 // sc["nkv"] else 2 * p + 1


def get_segment(sc, p, k):
    if k < sc["full"]:
        return i32(k * sc["P"] + p), 0, sc["nkv"]
    if sc["dyn"] or p >= sc["Prem"]:
        return None
    nkv = sc["nkv"]
    base = i32(sc["full"] * sc["P"] * nkv)
    a, b = base + rem_begin(sc, p), base + rem_begin(sc, p + 1)
    x = a if k == sc["full"] else i32((a // nkv + (k - sc["full"])) * nkv)
    if x >= b:
        return None
    t = x // nkv
    kv0 = x - t * nkv
    left = b - x
    kv1 = kv0 + left if left < nkv - kv0 else nkv
    return t, kv0, kv1


def segments(sc, p):
    out, k = [], 0
    while True:
        s = get_segment(sc, p, k)
        if s is None:
            return out
        out.append(s)
        k += 1


def xcd_remap(b, G):
    per, rem, x, loc = G // 8, G % 8, b % 8, b // 8
    return x * (per + 1) + loc if x < rem else rem * (per + 1) + (x - rem) * per + loc


# ---------------------------------------------------------------------------
# one attention call: rope_k_vt_kernel, attn_fwd_kernel, merge_kernel
# ---------------------------------------------------------------------------

def attention_call(buf, *, heads, D, nq, nk, tokens_pad, P, q_name, q_base, qh, qn, k_name,
                   k_base, v_name, v_base, kh, kn, o_name, o_base, oh, on, lse=False):
    """Replay one call's three kernels against `buf`, which must hold q_name,
    k_name, v_name, o_name, 'kr', 'vt' (heads * tokens_pad * D each), 'part_o'
    (2 P BM D), 'part_ml' (2 P BM 2) and, with lse, 'lse' (heads * nq)."""
    Npad = -(-nk // PREP_KEYS) * PREP_KEYS
    assert Npad <= tokens_pad
    sc = make_sched(heads, nq, nk, P)
    if sc is None:
        raise OutOfBounds("too many units")

    # rope_k_vt_kernel: grid (Npad / 64, heads, D / 64), one 64-key tile and 64
    # head dims per block: reads the keys' chunks 8 z .. 8 z + 7 (16 bytes each)
    # and writes fragments 8 z .. 8 z + 7 of the tile's Kr and of its Vt.
    CPR = 8                            # 16-byte chunks of the 64 dims a block stages
    PER = PREP_BLOCK * CPR // 256
    assert D % 64 == 0
    for hd in range(heads):
        n = np.arange(nk, dtype=np.int64)  # keys read (n < N)
        for z in range(D // 64):
            for name, base in ((k_name, k_base), (v_name, v_base)):
                off = base + hd * kh + n * kn + z * 64
                buf.access(name, off.min(), off.max() + 64, "rope_k_vt read")
            # write: (hd Npad + n0) D + 8 z 512 + F 512 + lane 8 + 8, F < 4 PER
            last_tile = Npad // PREP_BLOCK - 1
            for tile in (0, last_tile):
                base_t = (hd * Npad + tile * PREP_BLOCK) * D + z * 8 * 512
                buf.access("kr", base_t, base_t + (4 * PER - 1) * 512 + 63 * 8 + 8, "rope_k_vt Kr write")
                buf.access("vt", base_t, base_t + (4 * PER - 1) * 512 + 63 * 8 + 8, "rope_k_vt Vt write")
    assert 2 * PREP_BLOCK * CPR * 16 <= LDS_BYTES
    # every tile's fragments are written exactly once over the z blocks
    assert (D // 64) * 4 * PER * 512 == PREP_BLOCK * D

    # attn_fwd_kernel: persistent grid of P workgroups.
    KBYTES = KBN * D * 2
    BM = KBM
    # K / Vt double buffer, the Q rows of the next tile, the (cos, sin) table
    assert 2 * (2 * KBYTES) + BM * D * 2 + TAB_LDS * 8 <= LDS_BYTES, "LDS of attn_fwd_kernel"
    head_bytes = Npad * D * 2
    covered = np.zeros((heads * sc["n_qtiles"], sc["nkv"]), dtype=np.int32)
    slots = {}
    q_lds = qn * 2 * BM < (1 << 31)
    remapped = sorted(xcd_remap(b, P) for b in range(P))
    assert remapped == list(range(P)), "xcd_remap is not a permutation"
    for pid in range(P):
        for (t, kv0, kv1) in segments(sc, pid):
            h, qt = t // sc["n_qtiles"], t % sc["n_qtiles"]
            assert 0 <= h < heads and 0 <= kv0 < kv1 <= sc["nkv"]
            covered[t, kv0:kv1] += 1
            # Kr / Vt resources of head h, tile copies of blocks kv0..kv1-1.
            buf.rsrc("kr", h * Npad * D, head_bytes, 2, "attn Kr resource")
            buf.rsrc("vt", h * Npad * D, head_bytes, 2, "attn Vt resource")
            if (kv1 - 1) * KBYTES + KBYTES > head_bytes:
                raise OutOfBounds("key block past the head's Kr rows")
            rows = min(BM, nq - qt * BM)
            assert rows >= 1
            if q_lds:
                qb = q_base + h * qh + qt * BM * qn
                buf.rsrc(q_name, qb, ((rows - 1) * qn + D) * 2, 2, "attn Q LDS copy")
            # direct Q loads and O stores of the rows below nq
            r = np.arange(qt * BM, qt * BM + rows, dtype=np.int64)
            qoff = q_base + h * qh + r * qn
            buf.access(q_name, qoff.min(), qoff.max() + D, "attn Q load")
            if kv0 == 0 and kv1 == sc["nkv"]:
                ooff = o_base + h * oh + r * on
                buf.access(o_name, ooff.min(), ooff.max() + D, "attn O store")
                if lse:
                    buf.access("lse", h * nq + r.min(), h * nq + r.max() + 1, "attn lse store")
            else:
                slot = partial_slot(sc, pid, t)
                key = (pid, slot)
                assert key not in slots, "partial slot written twice"
                slots[key] = t
                buf.access("part_o", slot * BM * D, (slot * BM + BM) * D, "attn partial O")
                buf.access("part_ml", slot * BM * 2, (slot * BM + BM) * 2, "attn partial (m, l)")
    # Claimed pieces (any workgroup may take any piece; each writes slot i).
    for i in range(sc["npieces"]):
        t, kv0, kv1 = piece_segment(sc, i)
        assert 0 <= kv0 < kv1 <= sc["nkv"] and kv1 - kv0 >= min(PIECE_BLOCKS, sc["nkv"])
        covered[t, kv0:kv1] += 1
        if not i < 2 * P:
            raise OutOfBounds("piece %d has no partial slot (2P = %d)" % (i, 2 * P))
        if not (kv0 == 0 and kv1 == sc["nkv"]):
            buf.access("part_o", i * BM * D, (i * BM + BM) * D, "attn partial O (piece)")
            buf.access("part_ml", i * BM * 2, (i * BM + BM) * 2, "attn partial (m, l) (piece)")
            slots[("piece", i)] = t
    if not np.all(covered == 1):
        raise OutOfBounds("schedule does not cover every (tile, key block) exactly once")

    # merge_kernel: grid (rem tiles, rows); reads the slots the attention
    # kernel wrote, writes O (and lse) of split tiles.
    for bx in range(sc["rem_tiles"]):
        t = sc["full"] * P + bx
        if sc["dyn"]:
            if sc["ppt"] == 1:
                continue
            for i in range(bx * sc["ppt"], (bx + 1) * sc["ppt"]):
                if slots.get(("piece", i)) != t:
                    raise OutOfBounds("merge reads piece slot %d, which holds no part of tile %d" % (i, t))
            h, qt = t // sc["n_qtiles"], t % sc["n_qtiles"]
            rows = min(BM, nq - qt * BM)
            r = np.arange(qt * BM, qt * BM + rows, dtype=np.int64)
            ooff = o_base + h * oh + r * on
            buf.access(o_name, ooff.min(), ooff.max() + D, "merge O store")
            if lse:
                buf.access("lse", h * nq + r.min(), h * nq + r.max() + 1, "merge lse store")
            continue
        y0 = bx * sc["nkv"]
        p0, p1 = rem_owner(sc, y0), rem_owner(sc, y0 + sc["nkv"] - 1)
        if p0 == p1:
            assert segments(sc, p0) and any(s[0] == t and s[1] == 0 and s[2] == sc["nkv"]
                                            for s in segments(sc, p0))
            continue
        h, qt = t // sc["n_qtiles"], t % sc["n_qtiles"]
        for p in range(p0, p1 + 1):
            slot = partial_slot(sc, p0, t) if p == p0 else 2 * p
            if slots.get((p, slot)) != t:
                raise OutOfBounds("merge reads slot %d of workgroup %d, which holds no part of tile %d"
                                  % (slot, p, t))
        # every workgroup that wrote a part of t is in [p0, p1]
        writers = {p for (p, s), tt in slots.items() if tt == t}
        assert writers == set(range(p0, p1 + 1)), (writers, p0, p1)
        rows = min(BM, nq - qt * BM)
        r = np.arange(qt * BM, qt * BM + rows, dtype=np.int64)
        ooff = o_base + h * oh + r * on
        buf.access(o_name, ooff.min(), ooff.max() + D, "merge O store")
        if lse:
            buf.access("lse", h * nq + r.min(), h * nq + r.max() + 1, "merge lse store")
    return sc


# ---------------------------------------------------------------------------
# GEMM: C[M][N] = A[M][K] B[N][K]^T (gemm() in regen_attn.hip, gemm.hpp)
# ---------------------------------------------------------------------------

def gemm_call(buf, *, a_name, a_base, lda, b_name, b_base, ldb, c_name, c_base, ldc, M, N, K,
              big_slots=256, small_slots=512, written=None):
    """Replay one GEMM launch; `written` (optional bool [M, N]) counts the
    output elements each tile stores."""
    assert K % GEMM_BK == 0
    cover = np.zeros((M, N), dtype=np.int16) if written is None else written

    def tile(m0, n0, TM, TN):
        # copies: rows m0 .. m0 + TM - 1 of A and n0 .. of B, k < K, through
        # resources of extent M lda 2 and N ldb 2 (rows past the end read 0)
        buf.rsrc(a_name, a_base, M * lda * 2, 2, "gemm A resource")
        buf.rsrc(b_name, b_base, N * ldb * 2, 2, "gemm B resource")
        if ((m0 + TM - 1) * lda + K) * 2 >= 1 << 32 or ((n0 + TN - 1) * ldb + K) * 2 >= 1 << 32:
            raise OutOfBounds("gemm copy offset does not fit 32 bits")
        # stores: m < M, n < N only
        m1, n1 = min(m0 + TM, M), min(n0 + TN, N)
        if m0 < M and n0 < N:
            buf.access(c_name, c_base + m0 * ldc + n0, c_base + (m1 - 1) * ldc + n1, "gemm C store")
            cover[m0:m1, n0:n1] += 1

    big_tiles = -(-M // GEMM_BIG) * -(-N // GEMM_BIG)
    if big_tiles >= big_slots:
        G, GM = big_slots, 4
        mt, nt = -(-M // GEMM_BIG), -(-N // GEMM_BIG)
        rounds = big_tiles // G

        def origin(t):
            first = (t // (GM * nt)) * GM
            gm = min(mt - first, GM)
            r = t - first * nt
            return (first + r % gm) * GEMM_BIG, (r // gm) * GEMM_BIG

        assert 2 * 2 * GEMM_BIG * GEMM_BK * 2 <= LDS_BYTES
        for blk in range(G):
            pid = xcd_remap(blk, G)
            for k in range(rounds):
                m0, n0 = origin(k * G + pid)
                tile(m0, n0, 256, 256)
            done = rounds * G
            left = big_tiles - done
            if left * 8 <= G:
                if pid < left * 8:
                    m0, n0 = origin(done + pid // 8)
                    tile(m0 + ((pid & 7) >> 2) * 128, n0 + (pid & 3) * 64, 128, 64)
            else:
                for qd in range(pid, left * 4, G):
                    m0, n0 = origin(done + qd // 4)
                    tile(m0 + ((qd & 3) >> 1) * 128, n0 + (qd & 1) * 128, 128, 128)
    else:
        GM = 8
        mt, nt = -(-M // GEMM_TILE), -(-N // GEMM_TILE)
        tiles = mt * nt
        full = tiles // small_slots * small_slots
        rem = tiles - full
        nfull = full if (full > 0 and rem > 0 and rem * 4 <= small_slots) else tiles
        blocks = nfull + (tiles - nfull) * 4
        for bid in range(blocks):
            t = xcd_remap(bid, nfull) if bid < nfull else nfull + (bid - nfull) // 4
            first = (t // (GM * nt)) * GM
            gm = min(mt - first, GM)
            r = t - first * nt
            m0, n0 = (first + r % gm) * GEMM_TILE, (r // gm) * GEMM_TILE
            if bid < nfull:
                tile(m0, n0, 128, 128)
            else:
                qd = (bid - nfull) & 3
                tile(m0 + (qd >> 1) * 64, n0 + (qd & 1) * 64, 64, 64)
    if written is None and not np.all(cover == 1):
        raise OutOfBounds("GEMM output not covered exactly once")
    return cover


# ---------------------------------------------------------------------------
# whole entry points
# ---------------------------------------------------------------------------

def attention_forward(heads, D, tokens, P, token_major=False, q_begin=0, nq=None, kv_begin=0,
                      nk=None, lse=False):
    """regen_attn_forward / _range on a handle of `tokens` tokens (caller's
    buffers exactly as large as the header requires)."""
    nq = tokens if nq is None else nq
    nk = tokens if nk is None else nk
    tokens_pad = -(-tokens // PREP_KEYS) * PREP_KEYS
    Pcall = P
    buf = Buffers(q=heads * nq * D, k=heads * nk * D, v=heads * nk * D, o=heads * nq * D,
                  kr=heads * tokens_pad * D, vt=heads * tokens_pad * D,
                  part_o=2 * Pcall * KBM * D, part_ml=2 * Pcall * KBM * 2, lse=heads * nq)
    if token_major:
        qh, qn, kh, kn = D, heads * D, D, heads * D
    else:
        qh, qn, kh, kn = nq * D, D, nk * D, D
    attention_call(buf, heads=heads, D=D, nq=nq, nk=nk, tokens_pad=tokens_pad, P=Pcall,
                   q_name="q", q_base=0, qh=qh, qn=qn, k_name="k", k_base=0, v_name="v", v_base=0,
                   kh=kh, kn=kn, o_name="o", o_base=0, oh=qh, on=qn, lse=lse)
    return buf


def block_forward(heads, D, tokens, P, big_slots=256, small_slots=512):
    """regen_block_forward: QKV GEMM into qkv [N][3 hidden], attention on the
    strided views, output GEMM from attn_out [N][hidden] into y."""
    hid = heads * D
    tokens_pad = -(-tokens // PREP_KEYS) * PREP_KEYS
    buf = Buffers(x=tokens * hid, w_qkv=3 * hid * hid, w_o=hid * hid, qkv=tokens * 3 * hid,
                  attn_out=tokens * hid, y=tokens * hid, kr=heads * tokens_pad * D,
                  vt=heads * tokens_pad * D, part_o=2 * P * KBM * D, part_ml=2 * P * KBM * 2)
    gemm_call(buf, a_name="x", a_base=0, lda=hid, b_name="w_qkv", b_base=0, ldb=hid, c_name="qkv",
              c_base=0, ldc=3 * hid, M=tokens, N=3 * hid, K=hid, big_slots=big_slots,
              small_slots=small_slots)
    # Q, K, V are column blocks of qkv: token stride 3 hidden, head stride D.
    attention_call(buf, heads=heads, D=D, nq=tokens, nk=tokens, tokens_pad=tokens_pad, P=P,
                   q_name="qkv", q_base=0, qh=D, qn=3 * hid, k_name="qkv", k_base=hid,
                   v_name="qkv", v_base=2 * hid, kh=D, kn=3 * hid, o_name="attn_out", o_base=0, oh=D, on=hid)
    gemm_call(buf, a_name="attn_out", a_base=0, lda=hid, b_name="w_o", b_base=0, ldb=hid,
              c_name="y", c_base=0, ldc=hid, M=tokens, N=hid, K=hid, big_slots=big_slots,
              small_slots=small_slots)
    return buf
