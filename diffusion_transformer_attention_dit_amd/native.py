"""ctypes binding of the C ABI in include/regen_attn.h (argument marshalling only).

Every computation happens in the HIP library ``libregen_attn.so``; there is
no fallback. If the library is missing, loading fails loudly with the build
command to run.
"""
import ctypes
import os

from . import build as _build

REGEN_OK = 0
REGEN_ERR_INVALID_ARGUMENT = 1
REGEN_ERR_UNSUPPORTED = 2
REGEN_ERR_NO_DEVICE = 3
REGEN_ERR_OUT_OF_MEMORY = 4
REGEN_ERR_HIP = 5

REGEN_ATTN_NO_ROPE = 0x1
REGEN_ATTN_PROFILE = 0x2
REGEN_ATTN_TOKEN_MAJOR = 0x4

# Names the header declares; the CPU tests check the library exports each.
EXPORTS = (
    "regen_attn_create",
    "regen_attn_forward",
    "regen_attn_forward_range",
    "regen_attn_forward_cross",
    "regen_attn_merge",
    "regen_ulysses_pack",
    "regen_ulysses_unpack",
    "regen_linear",
    "regen_block_create",
    "regen_block_forward",
    "regen_block_destroy",
    "regen_attn_destroy",
    "regen_attn_status_string",
    "regen_attn_last_error",
    "regen_attn_workspace_size",
    "regen_attn_profile_read",
    "regen_attn_forward_noalloc",
    "regen_clock_probe",
)

# Size of the static device scratch behind regen_attn_forward_noalloc.
REGEN_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


class regen_attn_desc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("grid_t", ctypes.c_int32),
        ("grid_h", ctypes.c_int32),
        ("grid_w", ctypes.c_int32),
        ("pairs_t", ctypes.c_int32),
        ("pairs_h", ctypes.c_int32),
        ("pairs_w", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("sm_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


def make_desc(heads, head_dim, grid, pairs=(0, 0, 0), rope_base=0.0, sm_scale=0.0, flags=0):
    d = regen_attn_desc()
    d.struct_size = ctypes.sizeof(regen_attn_desc)
    d.heads, d.head_dim = int(heads), int(head_dim)
    d.grid_t, d.grid_h, d.grid_w = (int(x) for x in grid)
    d.pairs_t, d.pairs_h, d.pairs_w = (int(x) for x in pairs)
    d.rope_base, d.sm_scale, d.flags = float(rope_base), float(sm_scale), int(flags)
    return d


_LIB = None


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_build.LIB):
        raise RuntimeError(
            "libregen_attn.so is not built; run `python -m diffusion_transformer_attention_dit_amd.build`"
            " (or __graft_entry__.build())")
    L = ctypes.CDLL(_build.LIB)
    vp = ctypes.c_void_p
    L.regen_attn_create.argtypes = [ctypes.POINTER(regen_attn_desc), ctypes.POINTER(vp)]
    L.regen_attn_create.restype = ctypes.c_int
    L.regen_attn_forward.argtypes = [vp, vp, vp, vp, vp, vp]
    L.regen_attn_forward.restype = ctypes.c_int
    i64 = ctypes.c_int64
    L.regen_attn_forward_range.argtypes = [vp, vp, i64, i64, vp, vp, i64, i64, vp, vp, vp]
    L.regen_attn_forward_range.restype = ctypes.c_int
    L.regen_attn_forward_cross.argtypes = [vp, vp, vp, vp, i64, vp, vp, vp]
    L.regen_attn_forward_cross.restype = ctypes.c_int
    L.regen_attn_merge.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.c_int,
                                   ctypes.c_int, i64, ctypes.c_int, vp, vp, vp]
    L.regen_attn_merge.restype = ctypes.c_int
    for name in ("regen_ulysses_pack", "regen_ulysses_unpack"):
        f = getattr(L, name)
        f.argtypes = [vp, vp, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
        f.restype = ctypes.c_int
    L.regen_linear.argtypes = [vp, vp, vp, i64, ctypes.c_int, ctypes.c_int, vp]
    L.regen_linear.restype = ctypes.c_int
    L.regen_block_create.argtypes = [ctypes.POINTER(regen_attn_desc), ctypes.POINTER(vp)]
    L.regen_block_create.restype = ctypes.c_int
    L.regen_block_forward.argtypes = [vp] * 6
    L.regen_block_forward.restype = ctypes.c_int
    L.regen_block_destroy.argtypes = [vp]
    L.regen_block_destroy.restype = ctypes.c_int
    L.regen_attn_destroy.argtypes = [vp]
    L.regen_attn_destroy.restype = ctypes.c_int
    L.regen_attn_status_string.argtypes = [ctypes.c_int]
    L.regen_attn_status_string.restype = ctypes.c_char_p
    L.regen_attn_last_error.argtypes = []
    L.regen_attn_last_error.restype = ctypes.c_char_p
    L.regen_attn_workspace_size.argtypes = [ctypes.POINTER(regen_attn_desc)]
    L.regen_attn_workspace_size.restype = ctypes.c_size_t
    L.regen_attn_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64)]
    L.regen_attn_profile_read.restype = ctypes.c_int
    L.regen_attn_forward_noalloc.argtypes = [ctypes.POINTER(regen_attn_desc), vp, vp, vp, vp, vp]
    L.regen_attn_forward_noalloc.restype = ctypes.c_int
    L.regen_clock_probe.argtypes = [ctypes.c_int, vp, ctypes.POINTER(ctypes.c_double), vp]
    L.regen_clock_probe.restype = ctypes.c_int
    _LIB = L
    return L


class RegenAttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = "%s failed: %s (%s)" % (where, regen_attn_status_string(status), regen_attn_last_error())
        super().__init__(msg)


# ---- the C functions, same names -------------------------------------------

def regen_attn_create(desc):
    """Returns (status, handle); handle is None on failure."""
    h = ctypes.c_void_p()
    s = lib().regen_attn_create(ctypes.byref(desc) if desc is not None else None, ctypes.byref(h))
    return s, (h.value if s == REGEN_OK else None)


def regen_attn_forward(handle, q, k, v, o, stream):
    """q, k, v, o, stream are integer device addresses / a hipStream_t value."""
    return lib().regen_attn_forward(handle, q, k, v, o, stream)


def regen_attn_forward_noalloc(desc, q, k, v, o, stream):
    """Handle-free, allocation-free forward; q, k, v, o, stream are integer
    device addresses / a hipStream_t value."""
    return lib().regen_attn_forward_noalloc(ctypes.byref(desc) if desc is not None else None, q, k, v, o,
                                            stream)


def regen_attn_forward_range(handle, q, q_begin, q_count, k, v, kv_begin, kv_count, o, lse,
                             stream):
    """Pointers are integer device addresses (lse may be 0 / None)."""
    return lib().regen_attn_forward_range(handle, q, q_begin, q_count, k, v, kv_begin, kv_count,
                                          o, lse or None, stream)


def regen_attn_forward_cross(handle, q, k_ctx, v_ctx, ctx_len, o, lse, stream):
    return lib().regen_attn_forward_cross(handle, q, k_ctx, v_ctx, ctx_len, o, lse or None, stream)


def regen_attn_merge(o_parts, lse_parts, heads, rows, head_dim, o, lse, stream):
    """o_parts, lse_parts: sequences of integer device addresses."""
    n = len(o_parts)
    vp = ctypes.c_void_p
    op = (vp * max(n, 1))(*[vp(a) for a in o_parts])
    lp = (vp * max(len(lse_parts), 1))(*[vp(a) for a in lse_parts])
    return lib().regen_attn_merge(op if o_parts is not None else None,
                                  lp if lse_parts is not None else None, n, heads, rows,
                                  head_dim, o, lse or None, stream)


def regen_ulysses_pack(x, send, tokens_local, heads, head_dim, groups, stream):
    return lib().regen_ulysses_pack(x, send, tokens_local, heads, head_dim, groups, stream)


def regen_ulysses_unpack(recv, y, tokens_local, heads, head_dim, groups, stream):
    return lib().regen_ulysses_unpack(recv, y, tokens_local, heads, head_dim, groups, stream)


def regen_linear(x, w, y, rows, in_features, out_features, stream):
    return lib().regen_linear(x, w, y, rows, in_features, out_features, stream)


def regen_block_create(desc):
    """Returns (status, block); block is None on failure."""
    b = ctypes.c_void_p()
    s = lib().regen_block_create(ctypes.byref(desc) if desc is not None else None, ctypes.byref(b))
    return s, (b.value if s == REGEN_OK else None)


def regen_block_forward(block, x, w_qkv, w_o, y, stream):
    return lib().regen_block_forward(block, x, w_qkv, w_o, y, stream)


def regen_block_destroy(block):
    return lib().regen_block_destroy(block)


def regen_attn_destroy(handle):
    return lib().regen_attn_destroy(handle)


def regen_attn_status_string(status):
    return lib().regen_attn_status_string(int(status)).decode()


def regen_attn_last_error():
    return lib().regen_attn_last_error().decode()


def regen_attn_workspace_size(desc):
    return lib().regen_attn_workspace_size(ctypes.byref(desc) if desc is not None else None)


def regen_attn_profile_read(handle):
    """Returns (status, prep_ms, attn_ms, merge_ms, calls) accumulated since the last read."""
    a, b, c, n = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0), ctypes.c_int64(0)
    s = lib().regen_attn_profile_read(handle, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c),
                                      ctypes.byref(n))
    return s, a.value, b.value, c.value, n.value


def regen_clock_probe(iters, counters, stream):
    """Returns (status, wall_clock_khz); counters is an integer device address."""
    khz = ctypes.c_double(0)
    s = lib().regen_clock_probe(int(iters), counters, ctypes.byref(khz), stream)
    return s, khz.value


# ---- small convenience wrappers over torch tensors --------------------------


def clock_probe(iters=150000, stream=None):
    """GPU core clock (GHz) under a pure bf16 MFMA load, and that load's
    TFLOP/s: (ghz, tflops, seconds)."""
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    c = torch.zeros(5, dtype=torch.int64, device="cuda")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    s, khz = regen_clock_probe(iters, c.data_ptr(), stream.cuda_stream)
    b.record(stream)
    if s != REGEN_OK:
        raise RegenAttnError(s, "regen_clock_probe")
    torch.cuda.synchronize()
    t0, t1, w0, w1 = (int(x) for x in c[:4].tolist())
    wall_s = (w1 - w0) / (khz * 1e3)
    ghz = (t1 - t0) / wall_s / 1e9
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    flops = cus * 8 * iters * 4 * 2 * 32 * 32 * 16
    secs = a.elapsed_time(b) * 1e-3
    return ghz, flops / secs / 1e12, secs

def ulysses_pack(x, groups, out=None, stream=None):
    """x [tokens_local, heads, d] bf16 -> [groups, tokens_local, heads/groups, d]."""
    import torch
    nl, heads, d = (int(a) for a in x.shape)
    if out is None:
        out = torch.empty((groups, nl, heads // groups, d), dtype=x.dtype, device=x.device)
    _ulysses_call(regen_ulysses_pack, x, out, nl, heads, d, groups, stream, "regen_ulysses_pack")
    return out


def ulysses_unpack(recv, out=None, stream=None):
    """recv [groups, tokens_local, heads/groups, d] bf16 -> [tokens_local, heads, d]."""
    import torch
    groups, nl, hg, d = (int(a) for a in recv.shape)
    if out is None:
        out = torch.empty((nl, groups * hg, d), dtype=recv.dtype, device=recv.device)
    _ulysses_call(regen_ulysses_unpack, recv, out, nl, groups * hg, d, groups, stream,
                  "regen_ulysses_unpack")
    return out


def _ulysses_call(fn, src, dst, nl, heads, d, groups, stream, name):
    import torch
    for t in (src, dst):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("%s: tensors must be contiguous bf16 device tensors" % name)
    if src.numel() != nl * heads * d or dst.numel() != src.numel():
        raise ValueError("%s: sizes do not match" % name)
    if stream is None:
        stream = torch.cuda.current_stream(src.device)
    s = fn(src.data_ptr(), dst.data_ptr(), nl, heads, d, groups, stream.cuda_stream)
    if s != REGEN_OK:
        raise RegenAttnError(s, name)

def merge(o_parts, lse_parts, out=None, lse=None, stream=None):
    """Combine results over disjoint key sets: o_parts bf16 [heads, rows, d],
    lse_parts fp32 [heads, rows] (torch device tensors). Returns (o, lse)."""
    import torch
    if len(o_parts) != len(lse_parts) or not o_parts:
        raise ValueError("need as many lse parts as o parts, at least one")
    heads, rows, d = (int(x) for x in o_parts[0].shape)
    for o_, l_ in zip(o_parts, lse_parts):
        if o_.dtype != torch.bfloat16 or not o_.is_contiguous() or tuple(o_.shape) != (heads, rows, d):
            raise ValueError("o parts must be contiguous bf16 [heads, rows, d] tensors of one shape")
        if l_.dtype != torch.float32 or not l_.is_contiguous() or tuple(l_.shape) != (heads, rows):
            raise ValueError("lse parts must be contiguous fp32 [heads, rows] tensors")
    if out is None:
        out = torch.empty_like(o_parts[0])
    if lse is None:
        lse = torch.empty_like(lse_parts[0])
    if stream is None:
        stream = torch.cuda.current_stream(o_parts[0].device)
    s = regen_attn_merge([t.data_ptr() for t in o_parts], [t.data_ptr() for t in lse_parts],
                         heads, rows, d, out.data_ptr(), lse.data_ptr() if lse is not False else None,
                         stream.cuda_stream)
    if s != REGEN_OK:
        raise RegenAttnError(s, "regen_attn_merge")
    return out, (lse if lse is not False else None)


class Attention:
    """One problem shape on the current device. torch supplies memory and the
    stream only; the call enqueues the library's kernels."""

    def __init__(self, heads, head_dim, grid, pairs=(0, 0, 0), rope_base=0.0, sm_scale=0.0,
                 flags=0):
        self.heads, self.head_dim, self.grid = int(heads), int(head_dim), tuple(grid)
        self.tokens = self.grid[0] * self.grid[1] * self.grid[2]
        self.desc = make_desc(heads, head_dim, grid, pairs, rope_base, sm_scale, flags)
        s, h = regen_attn_create(self.desc)
        if s != REGEN_OK:
            raise RegenAttnError(s, "regen_attn_create")
        self.handle = h

    def _shape(self, n):
        if self.desc.flags & REGEN_ATTN_TOKEN_MAJOR:
            return (n, self.heads, self.head_dim)
        return (self.heads, n, self.head_dim)

    def _check(self, t, name):
        import torch
        shape = self._shape(self.tokens)
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bf16 device tensor" % name)
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))

    def forward(self, q, k, v, out=None, stream=None):
        import torch
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            self._check(t, n)
        if out is None:
            out = torch.empty_like(q)
        self._check(out, "out")
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        s = regen_attn_forward(self.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                               out.data_ptr(), stream.cuda_stream)
        if s != REGEN_OK:
            raise RegenAttnError(s, "regen_attn_forward")
        return out

    __call__ = forward

    def forward_range(self, q, q_begin, k, v, kv_begin, out=None, lse=None, stream=None):
        """Query tokens q_begin.. (q: [heads, nq, d]) against key tokens
        kv_begin.. (k, v: [heads, nk, d]). Returns (o, lse); lse=False skips
        the log-sum-exp."""
        import torch
        tm = bool(self.desc.flags & REGEN_ATTN_TOKEN_MAJOR)
        nq, nk = (int(q.shape[0]), int(k.shape[0])) if tm else (int(q.shape[1]), int(k.shape[1]))
        for t, n, name in ((q, nq, "q"), (k, nk, "k"), (v, nk, "v")):
            self._check_rows(t, n, name)
        if out is None:
            out = torch.empty_like(q)
        self._check_rows(out, nq, "out")
        if lse is None:
            lse = torch.empty((self.heads, nq), dtype=torch.float32, device=q.device)
        if lse is not False:
            if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != (self.heads, nq):
                raise ValueError("lse must be a contiguous fp32 [heads, q_count] tensor")
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        s = regen_attn_forward_range(self.handle, q.data_ptr(), int(q_begin), nq, k.data_ptr(),
                                     v.data_ptr(), int(kv_begin), nk, out.data_ptr(),
                                     lse.data_ptr() if lse is not False else None,
                                     stream.cuda_stream)
        if s != REGEN_OK:
            raise RegenAttnError(s, "regen_attn_forward_range")
        return out, (lse if lse is not False else None)

    def forward_cross(self, q, k_ctx, v_ctx, out=None, lse=False, stream=None):
        """All window tokens q against context keys/values (no rotation).
        Returns (o, lse or None); pass lse=None to have it allocated."""
        import torch
        tm = bool(self.desc.flags & REGEN_ATTN_TOKEN_MAJOR)
        nc = int(k_ctx.shape[0] if tm else k_ctx.shape[1])
        self._check(q, "q")
        self._check_rows(k_ctx, nc, "k_ctx")
        self._check_rows(v_ctx, nc, "v_ctx")
        if out is None:
            out = torch.empty_like(q)
        self._check(out, "out")
        if lse is None:
            lse = torch.empty((self.heads, self.tokens), dtype=torch.float32, device=q.device)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        s = regen_attn_forward_cross(self.handle, q.data_ptr(), k_ctx.data_ptr(), v_ctx.data_ptr(),
                                     nc, out.data_ptr(),
                                     lse.data_ptr() if lse is not False else None,
                                     stream.cuda_stream)
        if s != REGEN_OK:
            raise RegenAttnError(s, "regen_attn_forward_cross")
        return out, (lse if lse is not False else None)

    def _check_rows(self, t, n, name):
        import torch
        shape = self._shape(n)
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bf16 device tensor" % name)
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))

    def profile_read(self):
        """(prep_ms, attn_ms, merge_ms, calls) since the last read; needs REGEN_ATTN_PROFILE."""
        s, a, b, c, n = regen_attn_profile_read(self.handle)
        if s != REGEN_OK:
            raise RegenAttnError(s, "regen_attn_profile_read")
        return a, b, c, n

    def close(self):
        if self.handle is not None:
            s = regen_attn_destroy(self.handle)
            self.handle = None
            if s != REGEN_OK:
                raise RegenAttnError(s, "regen_attn_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def linear(x, w, out=None, stream=None):
    """y = x w^T for bf16 device tensors x [rows, in], w [out, in]."""
    import torch
    rows, fin = (int(a) for a in x.shape)
    fout = int(w.shape[0])
    for t, name in ((x, "x"), (w, "w")):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("%s must be a contiguous bf16 device tensor" % name)
    if tuple(w.shape) != (fout, fin):
        raise ValueError("w must be [out_features, in_features]")
    if out is None:
        out = torch.empty((rows, fout), dtype=torch.bfloat16, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    s = regen_linear(x.data_ptr(), w.data_ptr(), out.data_ptr(), rows, fin, fout, stream.cuda_stream)
    if s != REGEN_OK:
        raise RegenAttnError(s, "regen_linear")
    return out


class Block:
    """Self-attention block [Q|K|V] = X W_qkv, attention, Y = O W_o on the
    current device; torch supplies memory and the stream only."""

    def __init__(self, heads, head_dim, grid, pairs=(0, 0, 0), rope_base=0.0, sm_scale=0.0,
                 flags=0):
        self.heads, self.head_dim, self.grid = int(heads), int(head_dim), tuple(grid)
        self.hidden = self.heads * self.head_dim
        self.tokens = self.grid[0] * self.grid[1] * self.grid[2]
        self.desc = make_desc(heads, head_dim, grid, pairs, rope_base, sm_scale, flags)
        s, b = regen_block_create(self.desc)
        if s != REGEN_OK:
            raise RegenAttnError(s, "regen_block_create")
        self.handle = b

    def forward(self, x, w_qkv, w_o, out=None, stream=None):
        import torch
        shapes = ((x, (self.tokens, self.hidden), "x"), (w_qkv, (3 * self.hidden, self.hidden), "w_qkv"),
                  (w_o, (self.hidden, self.hidden), "w_o"))
        for t, shape, name in shapes:
            if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError("%s must be a contiguous bf16 device tensor of shape %s" % (name, shape))
        if out is None:
            out = torch.empty_like(x)
        if stream is None:
            stream = torch.cuda.current_stream(x.device)
        s = regen_block_forward(self.handle, x.data_ptr(), w_qkv.data_ptr(), w_o.data_ptr(),
                                out.data_ptr(), stream.cuda_stream)
        if s != REGEN_OK:
            raise RegenAttnError(s, "regen_block_forward")
        return out

    __call__ = forward

    def close(self):
        if self.handle is not None:
            s = regen_block_destroy(self.handle)
            self.handle = None
            if s != REGEN_OK:
                raise RegenAttnError(s, "regen_block_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
