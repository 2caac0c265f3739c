"""The C-ABI library on a host without a GPU: it loads, exports every symbol
the header declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re
import sys

import pytest
import torch

from diffusion_transformer_attention_dit_amd import build, native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if build.is_stale():
        build.build()
    native.lib()


def header_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(regen_\w+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == set(native.EXPORTS)
    L = ctypes.CDLL(build.LIB)
    for n in names:
        assert hasattr(L, n), n


def test_desc_layout_matches_header():
    # 11 x 4-byte fields + flags: no padding in the C struct.
    assert ctypes.sizeof(native.regen_attn_desc) == 48


def test_status_strings():
    for s, name in [(0, "REGEN_OK"), (1, "REGEN_ERR_INVALID_ARGUMENT"), (2, "REGEN_ERR_UNSUPPORTED"),
                    (3, "REGEN_ERR_NO_DEVICE"), (4, "REGEN_ERR_OUT_OF_MEMORY"), (5, "REGEN_ERR_HIP")]:
        assert native.regen_attn_status_string(s) == name
    assert native.regen_attn_status_string(99) == "REGEN_ERR_UNKNOWN"


def good_desc(**kw):
    args = dict(heads=12, head_dim=128, grid=(7, 30, 52))
    args.update(kw)
    return native.make_desc(**args)


@pytest.mark.parametrize("mutate,expect", [
    (lambda d: setattr(d, "struct_size", 12), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "heads", 0), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "grid_t", 0), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "grid_w", -3), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "head_dim", 96), native.REGEN_ERR_UNSUPPORTED),
    (lambda d: setattr(d, "head_dim", 63), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "pairs_t", 22), native.REGEN_ERR_INVALID_ARGUMENT),  # 22/0/0
    (lambda d: (setattr(d, "pairs_t", 22), setattr(d, "pairs_h", 22), setattr(d, "pairs_w", 21)),
     native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "rope_base", -1.0), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "rope_base", float("nan")), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "sm_scale", float("inf")), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: setattr(d, "flags", 0x80), native.REGEN_ERR_INVALID_ARGUMENT),
    (lambda d: (setattr(d, "grid_t", 2048), setattr(d, "grid_h", 1024), setattr(d, "grid_w", 1024)),
     native.REGEN_ERR_INVALID_ARGUMENT),
])
def test_create_rejects_bad_descriptions(mutate, expect):
    d = good_desc()
    mutate(d)
    s, h = native.regen_attn_create(d)
    assert s == expect and h is None
    assert native.regen_attn_last_error() != ""
    assert native.regen_attn_workspace_size(d) == 0


def test_one_head_key_workspace_limit():
    # 2^31 bytes of rotated K for one head is one past the limit; just below
    # it the description is valid (its workspace size is reported).
    over = good_desc(heads=1, grid=(128, 256, 256))  # 8388608 tokens x 128 x 2 B = 2^31
    assert native.regen_attn_workspace_size(over) == 0
    s, h = native.regen_attn_create(over)
    assert s == native.REGEN_ERR_INVALID_ARGUMENT and h is None
    assert "one head" in native.regen_attn_last_error()
    # Below it, the schedule's 31-bit numbering of (query tile, key block)
    # pairs is the binding limit: heads * ceil(N/256) * ceil(N/64) < 2^31.
    under = good_desc(heads=1, grid=(90, 256, 256))  # 23040 x 92160 pairs
    assert native.regen_attn_workspace_size(under) == 2 * 90 * 256 * 256 * 128 * 2
    pairs_over = good_desc(heads=1, grid=(91, 256, 256))  # 23296 x 93184 >= 2^31
    assert native.regen_attn_workspace_size(pairs_over) == 0
    s, h = native.regen_attn_create(pairs_over)
    assert s == native.REGEN_ERR_INVALID_ARGUMENT and h is None
    assert "pairs" in native.regen_attn_last_error()


def test_create_rejects_null_desc():
    s, h = native.regen_attn_create(None)
    assert s == native.REGEN_ERR_INVALID_ARGUMENT and h is None


@pytest.mark.skipif(torch.cuda.is_available(), reason="host has a GPU")
def test_create_without_device_reports_no_device():
    s, h = native.regen_attn_create(good_desc())
    assert s == native.REGEN_ERR_NO_DEVICE and h is None


def test_workspace_size():
    # Kr + Vt, bf16, tokens padded to a multiple of 128.
    assert native.regen_attn_workspace_size(good_desc()) == 2 * 12 * 11008 * 128 * 2
    assert native.regen_attn_workspace_size(good_desc(heads=1, head_dim=64, grid=(2, 8, 8))) == \
        2 * 1 * 128 * 64 * 2
    assert native.regen_attn_workspace_size(None) == 0


def test_forward_and_destroy_reject_non_live_handles():
    assert native.regen_attn_forward(None, 16, 32, 48, 64, None) == native.REGEN_ERR_INVALID_ARGUMENT
    bogus = ctypes.addressof(ctypes.c_int64(0))  # never created: must not be dereferenced
    assert native.regen_attn_forward(bogus, 16, 32, 48, 64, None) == native.REGEN_ERR_INVALID_ARGUMENT
    assert native.regen_attn_destroy(bogus) == native.REGEN_ERR_INVALID_ARGUMENT
    assert native.regen_attn_destroy(None) == native.REGEN_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(native, "_LIB", None)
    monkeypatch.setattr(native._build, "LIB", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        native.lib()


def test_forward_range_rejects_non_live_handle():
    fake = ctypes.c_void_p(0x1000)
    s = native.regen_attn_forward_range(fake.value, 16, 0, 1, 16, 16, 0, 1, 32, None, None)
    assert s == native.REGEN_ERR_INVALID_ARGUMENT
    assert native.regen_attn_forward_range(None, 16, 0, 1, 16, 16, 0, 1, 32, None, None) == \
        native.REGEN_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("kw,expect", [
    (dict(nparts=0), native.REGEN_ERR_INVALID_ARGUMENT),
    (dict(nparts=9), native.REGEN_ERR_INVALID_ARGUMENT),
    (dict(heads=0), native.REGEN_ERR_INVALID_ARGUMENT),
    (dict(rows=0), native.REGEN_ERR_INVALID_ARGUMENT),
    (dict(head_dim=96), native.REGEN_ERR_UNSUPPORTED),
    (dict(o=0), native.REGEN_ERR_INVALID_ARGUMENT),
    (dict(o=0x10008), native.REGEN_ERR_INVALID_ARGUMENT),            # misaligned
    (dict(null_part=True), native.REGEN_ERR_INVALID_ARGUMENT),
    (dict(o=0x100000 + 64), native.REGEN_ERR_INVALID_ARGUMENT),      # overlaps part 0
    (dict(), native.REGEN_ERR_NO_DEVICE),                            # valid, but no GPU here
])
def test_merge_argument_checks_before_the_device(kw, expect):
    # Addresses are never dereferenced: every one of these fails before a
    # kernel could be launched.
    if expect == native.REGEN_ERR_NO_DEVICE and torch.cuda.is_available():
        pytest.skip("host has a GPU: valid arguments would launch on these fake addresses")
    n = kw.get("nparts", 2)
    parts = [0x100000 + i * 0x100000 for i in range(max(n, 0))]
    lses = [0x4000000 + i * 0x100000 for i in range(max(n, 0))]
    if kw.get("null_part"):
        parts[1] = 0
    s = native.regen_attn_merge(parts, lses, kw.get("heads", 2), kw.get("rows", 8),
                                kw.get("head_dim", 128), kw.get("o", 0x8000000), None, None)
    assert s == expect, native.regen_attn_last_error()


def test_block_entry_points_without_device():
    assert native.regen_block_forward(None, 16, 16, 16, 32, None) == native.REGEN_ERR_INVALID_ARGUMENT
    assert native.regen_block_destroy(None) == native.REGEN_OK
    bogus = ctypes.addressof(ctypes.c_int64(0))
    assert native.regen_block_destroy(bogus) == native.REGEN_ERR_INVALID_ARGUMENT
    s, b = native.regen_block_create(good_desc(flags=native.REGEN_ATTN_TOKEN_MAJOR))
    assert s == native.REGEN_ERR_INVALID_ARGUMENT and b is None
    if not torch.cuda.is_available():
        s, b = native.regen_block_create(good_desc())
        assert s == native.REGEN_ERR_NO_DEVICE and b is None


def test_linear_argument_checks_before_the_device():
    E = native.REGEN_ERR_INVALID_ARGUMENT
    assert native.regen_linear(0, 16, 32, 4, 64, 8, None) == E
    assert native.regen_linear(16, 32, 48, 0, 64, 8, None) == E
    assert native.regen_linear(16, 32, 48, 4, 96, 8, None) == native.REGEN_ERR_UNSUPPORTED
    assert native.regen_linear(16 + 2, 0x100000, 0x200000, 4, 64, 8, None) == E   # misaligned
    assert native.regen_linear(0x100000, 0x200000, 0x100000, 4, 64, 8, None) == E  # y overlaps x
    if not torch.cuda.is_available():
        assert native.regen_linear(0x100000, 0x200000, 0x300000, 4, 64, 8, None) == \
            native.REGEN_ERR_NO_DEVICE


def test_bench_refuses_more_than_one_gpu():
    # The library has no multi-GPU path: bench.py says so and exits non-zero
    # before touching any device.
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_build_tracks_every_kernel_source():
    # A library older than any of its sources is rebuilt before use, so the
    # dependency list must name every file under csrc/ and the header.
    csrc = os.path.join(ROOT, "diffusion_transformer_attention_dit_amd", "csrc")
    on_disk = {os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".hpp"))}
    assert on_disk <= set(build.DEPENDS), sorted(on_disk - set(build.DEPENDS))
    assert os.path.join(ROOT, "include", "regen_attn.h") in build.DEPENDS
    # Packed FP32 instructions stay out of the generated code.
    assert "-packed-fp32-ops" in build.HIPCC_FLAGS
