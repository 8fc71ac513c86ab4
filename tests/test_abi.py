"""The C-ABI library loads, exports every entry point include/ssd.h
declares, and rejects every invalid argument on the host with the right
status before any launch (CPU only: no kernel is ever started here)."""
import ctypes
import os
import re

import pytest

import ssd_chunked_scan_amd as ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "ssd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ssd.load_library()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ssd.h but not exported"
    assert sorted(ssd.EXPORTS) == names
    assert lib.ssd_version().startswith(b"ssd-mi355x")


def test_status_strings():
    lib = ssd.load_library()
    for code, name in ssd.STATUS.items():
        assert lib.ssd_status_str(code).decode() == name


FAKE = 0x100000  # aligned, never dereferenced: every call below fails validation


def _fwd(shape, io=1, chunk=256, x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, y=FAKE, fs=None,
         h0=None, ws=None, ws_bytes=0, opts=None, seq=None, D=None):
    lib = ssd.load_library()
    o = None if opts is None else ctypes.byref(opts)
    shp = None if shape is None else ctypes.byref(shape)
    return lib.ssd_fwd_ex(shp, io, x, dt, A, B, C, D, seq, chunk, h0, y, fs, ws, ws_bytes, o, None)


def good_shape():
    return ssd.Shape(2, 1000, 8, 64, 128, 2)


@pytest.mark.parametrize("mutate,status", [
    (lambda s: setattr(s, "batch", 0), 2),
    (lambda s: setattr(s, "seqlen", 0), 2),
    (lambda s: setattr(s, "nheads", -1), 2),
    (lambda s: setattr(s, "ngroups", 3), 2),      # 8 % 3 != 0
    (lambda s: setattr(s, "headdim", 48), 3),
    (lambda s: setattr(s, "headdim", 256), 3),
    (lambda s: setattr(s, "dstate", 8), 3),
    (lambda s: setattr(s, "dstate", 256), 3),
])
def test_shape_errors(mutate, status):
    s = good_shape()
    mutate(s)
    assert _fwd(s) == status
    assert ssd.load_library().ssd_last_error() != b""


def test_argument_errors():
    s = good_shape()
    assert _fwd(None) == 1
    assert _fwd(s, chunk=32) == 3
    assert _fwd(s, chunk=512) == 3
    assert _fwd(s, io=5) == 3
    assert _fwd(s, x=None) == 1
    assert _fwd(s, y=None) == 1
    assert _fwd(s, C=None) == 1
    assert _fwd(s, x=FAKE + 2) == 4
    assert _fwd(s, B=FAKE + 8) == 4
    assert _fwd(s, dt=FAKE + 2) == 4
    assert _fwd(s, fs=FAKE + 4) == 4
    assert _fwd(s, h0=FAKE + 8) == 4
    o = ssd.Options(100)              # not a multiple of the chunk size
    assert _fwd(s, opts=o) == 3
    o = ssd.Options(256)
    o.reserved[3] = 1
    assert _fwd(s, opts=o) == 3
    o = ssd.Options(0, 8)             # unknown flag bit
    assert _fwd(s, opts=o) == 3
    assert b"flags" in ssd.load_library().ssd_last_error()
    # segsum variants of the forward mask: one at a time; bf16 io only at
    # chunk 256, dstate 64 or 128 and headdim blocks of 32 or 64
    assert _fwd(s, io=0, opts=ssd.Options(0, 6)) == 3
    assert _fwd(s, io=0, opts=ssd.Options(0, 4)) == 5   # accepted: reaches the workspace check
    assert _fwd(s, io=1, opts=ssd.Options(0, 2)) == 5   # bf16, chunk 256, dstate 128: accepted
    assert _fwd(s, io=1, chunk=128, opts=ssd.Options(0, 2)) == 3
    assert b"segsum" in ssd.load_library().ssd_last_error()
    assert _fwd(ssd.Shape(2, 1000, 8, 64, 32, 2), io=1, opts=ssd.Options(0, 4)) == 3
    o = ssd.Options(0, 4)
    o.headdim_block = 16
    assert _fwd(s, io=1, opts=o) == 3
    assert b"headdim blocks of 32 or 64" in ssd.load_library().ssd_last_error()
    o = ssd.Options(256)              # 4 splits -> workspace required
    assert _fwd(s, opts=o) == 5
    assert b"workspace" in ssd.load_library().ssd_last_error()
    need = ssd.ssd_fwd_workspace_bytes(s, 256, 1, split_len=256)
    assert _fwd(s, opts=o, ws=FAKE, ws_bytes=need - 1) == 5
    assert _fwd(s, opts=o, ws=FAKE + 4, ws_bytes=need) == 4


def _ru(v):
    return (v + 255) // 256 * 256


def _bf16_group_bytes(b, G, nchunks, Q, N):
    """Per-group C B^T blocks, token-transposed B and C in operand order, as
    documented in ssd.h."""
    return (_ru(b * G * nchunks * 1024 * (Q // 32) * (Q // 32 + 1)) + _ru(b * G * nchunks * 2 * Q * N)
            + _ru(b * G * nchunks * 2 * Q * max(N, 32)))


def test_workspace_and_plan():
    s = good_shape()
    # forced split: 1000 tokens, chunk 256 -> 4 chunks; split 256 -> 4 splits
    need = ssd.ssd_fwd_workspace_bytes(s, 256, 1, split_len=256)
    assert need == _ru((2 * 8 * 4 * (64 * 128 + 1)) * 4) + _bf16_group_bytes(2, 2, 4, 256, 128)
    # fp32 io keeps no per-group operands
    assert ssd.ssd_fwd_workspace_bytes(s, 256, 0, split_len=256) == _ru((2 * 8 * 4 * (64 * 128 + 1)) * 4)
    assert ssd.ssd_fwd_workspace_bytes(s, 256, 0, split_len=1024) == 0
    assert ssd.ssd_fwd_workspace_bytes(s, 256, 1, split_len=1024) == _bf16_group_bytes(2, 2, 4, 256, 128)
    assert ssd.ssd_fwd_workspace_bytes(s, 64, 1, split_len=1024) == _bf16_group_bytes(2, 2, 16, 64, 128)
    # planner: plenty of (batch, head) pairs -> one split per row
    big = ssd.Shape(8, 2048, 80, 64, 128, 1)
    assert ssd.ssd_plan_split_len(big, 256, 1) == 2048
    assert ssd.ssd_fwd_workspace_bytes(big, 256, 1) == _bf16_group_bytes(8, 1, 8, 256, 128)
    assert ssd.ssd_fwd_workspace_bytes(big, 256, 0) == 0
    # few long rows -> sequence-parallel splits, chosen independently of the chunk
    long = ssd.Shape(1, 65536, 16, 64, 64, 1)
    sl = ssd.ssd_plan_split_len(long, 256, 1)
    assert sl % 256 == 0 and 256 <= sl < 65536
    assert ssd.ssd_plan_split_len(long, 64, 1) == sl
    assert ssd.ssd_fwd_workspace_bytes(long, 256, 0) > 0
    assert ssd.ssd_fwd_workspace_bytes(ssd.Shape(0, 1, 1, 16, 16, 1), 256, 1) == 0


def test_mask_errors():
    lib = ssd.load_library()
    s = ssd.Shape(1, 1000, 2, 16, 16, 1)
    f = lib.ssd_debug_chunk_mask
    assert f(ctypes.byref(s), FAKE, FAKE, None, 256, 0, 5, FAKE, None) == 2   # only 4 chunks
    assert f(ctypes.byref(s), FAKE, FAKE, None, 256, -1, 1, FAKE, None) == 2
    assert f(ctypes.byref(s), FAKE, FAKE, None, 256, 0, 0, FAKE, None) == 2
    assert f(ctypes.byref(s), None, FAKE, None, 256, 0, 1, FAKE, None) == 1
    assert f(ctypes.byref(s), FAKE, FAKE, None, 256, 0, 1, FAKE + 4, None) == 4
    assert f(ctypes.byref(s), FAKE, FAKE, None, 100, 0, 1, FAKE, None) == 3


def test_product_path_has_no_cpu_fallback(monkeypatch):
    """Without libssd.so the binding raises instead of computing anything."""
    monkeypatch.setattr(ssd, "_lib", None)
    monkeypatch.setattr(ssd, "_LIB_PATH", os.path.join(ROOT, "no_such_libssd.so"))
    with pytest.raises(ImportError):
        ssd.load_library()


def test_binding_does_not_import_oracle():
    import ast
    for fn in os.listdir(os.path.join(ROOT, "ssd_chunked_scan_amd")):
        if fn.endswith(".py"):
            tree = ast.parse(open(os.path.join(ROOT, "ssd_chunked_scan_amd", fn)).read())
            for node in ast.walk(tree):
                if isinstance(node, (ast.Import, ast.ImportFrom)):
                    mods = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module or ""]
                    assert not any(m.split(".")[0] == "oracle" for m in mods), fn


def test_mask_ex_host_validation():
    """Argument errors of ssd_debug_chunk_mask_ex are reported before any HIP
    call (fake but aligned device pointers; nothing is dereferenced)."""
    lib = ssd.load_library()
    s = ssd.Shape(1, 256, 2, 16, 16, 1)
    p = ctypes.c_void_p(1 << 20)
    # both outputs missing
    st = lib.ssd_debug_chunk_mask_ex(ctypes.byref(s), p, p, None, 64, 0, 1, 0, None, None, None)
    assert st == 1 and b"at least one" in lib.ssd_last_error()
    # unknown variant
    st = lib.ssd_debug_chunk_mask_ex(ctypes.byref(s), p, p, None, 64, 0, 1, 7, p, None, None)
    assert st == 3 and b"variant" in lib.ssd_last_error()
    # chunk range outside the sequence
    st = lib.ssd_debug_chunk_mask_ex(ctypes.byref(s), p, p, None, 64, 3, 2, 1, None, p, None)
    assert st == 2


def test_decode_step_host_validation():
    """ssd_decode_step reports argument errors before any HIP call."""
    lib = ssd.load_library()
    p = ctypes.c_void_p(1 << 20)
    one = ssd.Shape(2, 1, 4, 64, 128, 1)
    # more than one token
    st = lib.ssd_decode_step(ctypes.byref(ssd.Shape(2, 5, 4, 64, 128, 1)), 1, p, p, p, p, p, None, p, p, None)
    assert st == 2 and b"one token" in lib.ssd_last_error()
    # missing state
    st = lib.ssd_decode_step(ctypes.byref(one), 1, p, p, p, p, p, None, None, p, None)
    assert st == 1
    # unknown io dtype
    st = lib.ssd_decode_step(ctypes.byref(one), 9, p, p, p, p, p, None, p, p, None)
    assert st == 3
    # unsupported dstate
    st = lib.ssd_decode_step(ctypes.byref(ssd.Shape(2, 1, 4, 64, 48, 1)), 1, p, p, p, p, p, None, p, p, None)
    assert st == 3
    # misaligned state
    st = lib.ssd_decode_step(ctypes.byref(one), 1, p, p, p, p, p, None, ctypes.c_void_p((1 << 20) + 4), p, None)
    assert st == 4


def _fused_call(fused, ws=FAKE, ws_bytes=1 << 40):
    lib = ssd.load_library()
    s = good_shape()
    f = None if fused is None else ctypes.byref(fused)
    return lib.ssd_fwd_fused(ctypes.byref(s), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 256,
                             None, FAKE, None, f, ws, ws_bytes, None, None)


def test_fused_argument_errors():
    """ssd_fwd_fused validates its prologue/epilogue block on the host."""
    F = ssd.Fused
    bad = F()
    bad.reserved[2] = 1
    assert _fused_call(bad) == 3
    assert _fused_call(F(None, None, 0, 1, 0.5, 0.1)) == 3            # dt_min > dt_max
    assert _fused_call(F(None, None, 0, 1, 0.0, float("inf"))) == 3   # unbounded clamp
    assert _fused_call(F(None, None, 0, 1, float("nan"), 1.0)) == 3
    assert _fused_call(F(FAKE + 2, None, 1, 0, 0.0, 0.0)) == 4        # dt_bias misaligned
    assert _fused_call(F(None, FAKE + 8, 1, 0, 0.0, 0.0)) == 4        # z misaligned
    # a valid block reaches the workspace check (the last host check)
    assert _fused_call(F(FAKE, FAKE, 1, 1, 0.001, 0.1), ws=None, ws_bytes=0) == 5
    assert _fused_call(None, ws=None, ws_bytes=0) == 5


def test_headdim_block_option_errors():
    """headdim_block: 0 or a power of two >= 16 dividing headdim whose tiles
    fit the LDS (bf16); fp32 takes only 0 or headdim."""
    s = good_shape()                                   # headdim 64, dstate 128
    for hb, io, chunk in [(48, 1, 256), (8, 1, 256), (128, 1, 256), (-16, 1, 256),
                          (32, 0, 256), (16, 0, 64)]:
        o = ssd.Options(0, 0, hb)
        assert _fwd(s, io=io, chunk=chunk, opts=o) == 3, (hb, io)
    # accepted values reach the workspace check
    for hb, io in [(16, 1), (32, 1), (64, 1), (64, 0)]:
        assert _fwd(s, io=io, opts=ssd.Options(0, 0, hb)) == 5, (hb, io)


def test_plan_queries():
    lib = ssd.load_library()
    s = ssd.Shape(8, 2048, 80, 64, 128, 1)
    assert ssd.ssd_plan_headdim_block(s, 256, 1) == 64
    assert ssd.ssd_plan_split_len(s, 256, 1) == 2048
    assert ssd.ssd_plan_headdim_block(s, 256, 0) == 64
    assert lib.ssd_plan_headdim_block(None, 256, 1) == 0


def test_binding_argument_counts_match_the_header():
    """Every function the binding declares takes as many arguments as ssd.h
    gives it (a short argtypes list would pass trailing pointers as 32-bit
    ints)."""
    src = open(os.path.join(ROOT, "include", "ssd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lib = ssd.load_library()
    for name, params in re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", src):
        n = 0 if params.strip() in ("", "void") else params.count(",") + 1
        argtypes = getattr(lib, name).argtypes
        assert argtypes is not None, name
        assert len(argtypes) == n, f"{name}: header {n} parameters, binding {len(argtypes)}"


def test_debug_export_host_validation():
    lib = ssd.load_library()
    s = good_shape()
    assert lib.ssd_segsum_record_words(256) == 4 * 256 + 2 * 16 + 8
    assert lib.ssd_segsum_record_words(64) == 4 * 64 + 2 * 4 + 2
    assert lib.ssd_segsum_record_words(100) == 0
    assert lib.ssd_debug_segsum_factors(ctypes.byref(s), FAKE, FAKE, None, 256, None, None) == 1
    assert lib.ssd_debug_segsum_factors(ctypes.byref(s), FAKE, FAKE, None, 96, FAKE, None) == 3
    assert lib.ssd_debug_segsum_factors(ctypes.byref(s), FAKE + 2, FAKE, None, 256, FAKE, None) == 4
    o = ssd.Options()
    # the head kernel's factor export is a bf16-path aid
    assert lib.ssd_debug_fwd_segsum_factors(ctypes.byref(s), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                            256, None, FAKE, None, None, 0, ctypes.byref(o), FAKE,
                                            None) == 3
    assert lib.ssd_debug_fwd_segsum_factors(ctypes.byref(s), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                            256, None, FAKE, None, None, 0, ctypes.byref(o), None,
                                            None) == 1
    # without a workspace the bf16 call stops at the workspace check
    assert lib.ssd_debug_fwd_segsum_factors(ctypes.byref(s), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, None,
                                            256, None, FAKE, None, None, 0, ctypes.byref(o), FAKE,
                                            None) == 5
    # exp2 probe: non-positive patterns only, -0 .. -inf
    assert lib.ssd_debug_exp2_probe(0, 16, FAKE, 64, None) == 3
    assert lib.ssd_debug_exp2_probe(0xFF800000, 2, FAKE, 64, None) == 3
    assert lib.ssd_debug_exp2_probe(0x80000000, 0, FAKE, 64, None) == 3
    assert lib.ssd_debug_exp2_probe(0x80000000, 16, None, 64, None) == 1
    assert lib.ssd_debug_exp2_probe(0x80000000, 16, FAKE, 0, None) == 3
    assert lib.ssd_debug_exp2_probe(0x80000000, 16, FAKE + 2, 64, None) == 4


def test_launch_limits_are_checked_on_the_host():
    """Shapes whose work units or grids would not fit a launch (or an int) are
    refused before anything is launched."""
    huge = ssd.Shape(1 << 20, 1, 65536, 16, 16, 1)      # 2^36 (batch row, head) units
    assert ssd.ssd_fwd_workspace_bytes(huge, 64, 1) == 0
    assert _fwd(huge, chunk=64, ws=FAKE, ws_bytes=1 << 40) == 3
    assert _fwd(huge, io=0, chunk=64, ws=FAKE, ws_bytes=1 << 40) == 3
    lib = ssd.load_library()
    dec = ssd.Shape(1 << 20, 1, 65536, 16, 16, 1)
    assert lib.ssd_decode_step(ctypes.byref(dec), 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE,
                               None) == 3


def test_unknown_dtype_is_rejected():
    s = good_shape()
    for io in (2, 7, 1 << 20):
        assert _fwd(s, io=io) == 3
