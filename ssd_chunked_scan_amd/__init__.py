"""MI355X (gfx950) SSD chunked forward pass: thin Python binding of libssd.so.

Every step of the forward pass runs in the HIP kernels behind the C ABI in
include/ssd.h; this module only marshals torch tensors (device memory and the
current HIP stream) into that ABI.  There is no CPU or PyTorch fallback: if
libssd.so is missing or fails to load, every call raises.

    y, final_states = ssd_fwd(x, dt, A, B, C, D, seq_idx=None, chunk_size=256)

Shapes (dense, contiguous): x [b, L, H, P]; dt [b, L, H] fp32; A [H] fp32;
B, C [b, L, G, N]; D [H] fp32 or None; seq_idx [b, L] int32 or None;
init_states [b, H, P, N] fp32 or None.  x, B, C share one dtype, bf16 or
fp32; y has that dtype; final_states is fp32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = [
    "ssd_fwd", "prepare_fwd", "ssd_bwd", "ssd_fwd_workspace_bytes", "ssd_plan_split_len", "ssd_debug_chunk_mask",
    "ssd_decode_step",
    "SsdError", "library_path", "load_library", "STATUS", "EXPORTS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_UNSUPPORTED",
          4: "SSD_ERR_ALIGN", 5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_HIP"}
EXPORTS = ["ssd_fwd_workspace_bytes", "ssd_fwd", "ssd_fwd_ex_workspace_bytes", "ssd_fwd_ex",
           "ssd_fwd_fused",
           "ssd_plan_split_len", "ssd_plan_headdim_block", "ssd_debug_chunk_mask",
           "ssd_debug_chunk_mask_ex",
           "ssd_decode_step", "ssd_decode_step_fused", "ssd_bwd_workspace_bytes", "ssd_bwd",
           "ssd_segsum_record_words", "ssd_debug_segsum_factors", "ssd_debug_fwd_segsum_factors",
           "ssd_debug_exp2_probe", "ssd_fwd_noalloc",
           "ssd_status_str", "ssd_last_error", "ssd_version"]
# segsum evaluations of the mask export (ssd.h SSD_SEGSUM_*)
SEGSUM = {"hierarchy": 0, "direct": 1, "diff": 2}


class SsdError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64)]


class Options(ctypes.Structure):
    _fields_ = [("split_len", ctypes.c_int64), ("flags", ctypes.c_int64),
                ("headdim_block", ctypes.c_int64), ("reserved", ctypes.c_int64 * 5)]


SSD_OPT_REUSE_GROUP_OPERANDS = 1
SSD_OPT_SEGSUM = {"hierarchy": 0, "direct": 2, "diff": 4}   # forward mask evaluation


class Fused(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("z", ctypes.c_void_p),
                ("dt_softplus", ctypes.c_int32), ("dt_clamp", ctypes.c_int32),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float),
                ("reserved", ctypes.c_int64 * 4)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m ssd_chunked_scan_amd._build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz, i64, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int
    shp, opt = ctypes.POINTER(Shape), ctypes.POINTER(Options)
    lib.ssd_fwd_workspace_bytes.argtypes = [shp, i64, i32]
    lib.ssd_fwd_workspace_bytes.restype = sz
    lib.ssd_fwd_ex_workspace_bytes.argtypes = [shp, i64, i32, opt]
    lib.ssd_fwd_ex_workspace_bytes.restype = sz
    lib.ssd_plan_split_len.argtypes = [shp, i64, i32]
    lib.ssd_plan_split_len.restype = i64
    lib.ssd_plan_headdim_block.argtypes = [shp, i64, i32]
    lib.ssd_plan_headdim_block.restype = i64
    fwd_args = [shp, i32, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz]
    lib.ssd_fwd.argtypes = fwd_args + [vp]
    lib.ssd_fwd.restype = i32
    lib.ssd_fwd_ex.argtypes = fwd_args + [opt, vp]
    lib.ssd_fwd_ex.restype = i32
    lib.ssd_fwd_fused.argtypes = fwd_args[:13] + [ctypes.POINTER(Fused)] + fwd_args[13:] + [opt, vp]
    lib.ssd_fwd_fused.restype = i32
    lib.ssd_debug_chunk_mask.argtypes = [shp, vp, vp, vp, i64, i64, i64, vp, vp]
    lib.ssd_debug_chunk_mask.restype = i32
    lib.ssd_debug_chunk_mask_ex.argtypes = [shp, vp, vp, vp, i64, i64, i64, i32, vp, vp, vp]
    lib.ssd_debug_chunk_mask_ex.restype = i32
    lib.ssd_decode_step.argtypes = [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ssd_decode_step.restype = i32
    lib.ssd_decode_step_fused.argtypes = [shp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.POINTER(Fused), vp]
    lib.ssd_decode_step_fused.restype = i32
    lib.ssd_bwd_workspace_bytes.argtypes = [shp, i32]
    lib.ssd_bwd_workspace_bytes.restype = sz
    lib.ssd_bwd.argtypes = [shp, i32] + [vp] * 18 + [sz, vp]
    lib.ssd_bwd.restype = i32
    lib.ssd_segsum_record_words.argtypes = [i64]
    lib.ssd_segsum_record_words.restype = i64
    lib.ssd_debug_segsum_factors.argtypes = [shp, vp, vp, vp, i64, vp, vp]
    lib.ssd_debug_segsum_factors.restype = i32
    lib.ssd_debug_fwd_segsum_factors.argtypes = fwd_args + [opt, vp, vp]
    lib.ssd_debug_fwd_segsum_factors.restype = i32
    u32 = ctypes.c_uint32
    lib.ssd_debug_exp2_probe.argtypes = [u32, u32, vp, u32, vp]
    lib.ssd_debug_exp2_probe.restype = i32
    lib.ssd_fwd_noalloc.argtypes = fwd_args[:13] + [vp]
    lib.ssd_fwd_noalloc.restype = i32
    lib.ssd_status_str.argtypes = [i32]
    lib.ssd_status_str.restype = ctypes.c_char_p
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_version.argtypes = []
    lib.ssd_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise SsdError(status, load_library().ssd_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _io_code(dtype) -> int:
    import torch
    if dtype == torch.bfloat16:
        return SSD_BF16
    if dtype == torch.float32:
        return SSD_F32
    raise TypeError(f"x/B/C dtype must be bfloat16 or float32, got {dtype}")


def _need(t, name, shape, dtype, device):
    if t.shape != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def make_shape(batch, seqlen, nheads, headdim, dstate, ngroups) -> Shape:
    return Shape(batch, seqlen, nheads, headdim, dstate, ngroups)


def ssd_fwd_workspace_bytes(shape: Shape, chunk_size: int, io: int, split_len: int = 0) -> int:
    lib = load_library()
    if split_len:
        return int(lib.ssd_fwd_ex_workspace_bytes(ctypes.byref(shape), chunk_size, io,
                                                  ctypes.byref(Options(split_len))))
    return int(lib.ssd_fwd_workspace_bytes(ctypes.byref(shape), chunk_size, io))


def ssd_plan_split_len(shape: Shape, chunk_size: int, io: int) -> int:
    return int(load_library().ssd_plan_split_len(ctypes.byref(shape), chunk_size, io))


def ssd_plan_headdim_block(shape: Shape, chunk_size: int, io: int) -> int:
    return int(load_library().ssd_plan_headdim_block(ctypes.byref(shape), chunk_size, io))


def ssd_fwd(x, dt, A, B, C, D=None, seq_idx=None, chunk_size: int = 256, init_states=None,
            return_final_states: bool = True, split_len: int = 0, y=None, final_states=None,
            workspace=None, stream=None, reuse_group_operands: bool = False,
            dt_bias=None, dt_softplus: bool = False, dt_limit=None, z=None,
            headdim_block: int = 0, segsum: str = "hierarchy") -> Tuple[object, Optional[object]]:
    """Run the forward pass on x.device.  Returns (y, final_states or None).
    Arguments as for prepare_fwd, which this calls once."""
    call, y, final_states = _marshal_fwd(
        x, dt, A, B, C, D, seq_idx, chunk_size, init_states, return_final_states, split_len, y,
        final_states, workspace, stream, reuse_group_operands, dt_bias, dt_softplus, dt_limit, z,
        headdim_block, segsum)
    call()
    return y, (final_states if return_final_states else None)


def prepare_fwd(x, dt, A, B, C, D=None, seq_idx=None, chunk_size: int = 256, init_states=None,
                return_final_states: bool = True, split_len: int = 0, y=None,
                final_states=None, workspace=None, stream=None,
                reuse_group_operands: bool = False, dt_bias=None, dt_softplus: bool = False,
                dt_limit=None, z=None, headdim_block: int = 0, segsum: str = "hierarchy"):
    """Check and marshal the arguments of ssd_fwd once and return
    (launch, y, final_states): each launch() call runs the forward pass again
    on the same buffers and stream, with no per-call Python checks (for
    loops over fixed buffers, e.g. timing).  The caller keeps the tensors
    alive and unchanged in shape while it uses launch()."""
    return _marshal_fwd(x, dt, A, B, C, D, seq_idx, chunk_size, init_states, return_final_states,
                        split_len, y, final_states, workspace, stream, reuse_group_operands,
                        dt_bias, dt_softplus, dt_limit, z, headdim_block, segsum)


def _marshal_fwd(x, dt, A, B, C, D, seq_idx, chunk_size, init_states, return_final_states,
                 split_len, y, final_states, workspace, stream, reuse_group_operands, dt_bias,
                 dt_softplus, dt_limit, z, headdim_block=0, segsum="hierarchy"):
    """Argument checks and marshalling of ssd_fwd / prepare_fwd.
    ``split_len`` forces the sequence-parallel split length (0 = planner);
    ``headdim_block`` the headdim columns per workgroup (0 = planner);
    ``segsum`` ("hierarchy", "direct" or "diff") how the intra-chunk decay
    mask is evaluated (an ablation for tests and benchmarks; bf16 io: chunk
    256, dstate 64 or 128, headdim blocks of 32 or 64).
    Preallocated ``y`` / ``final_states`` / ``workspace`` (uint8) may be given.
    ``reuse_group_operands`` (bf16) skips the per-group C B^T / B^T kernel: the
    given ``workspace`` must hold them from an earlier call with the same B, C.
    Fused prologue/epilogue (ssd_fwd_fused): ``dt`` holds raw values mapped to
    clamp(softplus(dt + dt_bias)) per enabled step (``dt_bias`` [H] fp32,
    ``dt_softplus``, ``dt_limit`` = (lo, hi)); ``z`` [b, L, H, P] in x's dtype
    gates the output, y * silu(z)."""
    import torch
    lib = load_library()
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b, L, H, P] and B, C [b, L, G, N]")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_fwd runs on the GPU only (x is on %s)" % dev)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x.dtype)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if seq_idx is not None:
        _need(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", (H,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (b, L, H, P), x.dtype, dev)
    fused = Fused(_ptr(dt_bias), _ptr(z), 1 if dt_softplus else 0,
                  0 if dt_limit is None else 1,
                  0.0 if dt_limit is None else float(dt_limit[0]),
                  0.0 if dt_limit is None else float(dt_limit[1]))
    shape = Shape(b, L, H, P, N, G)
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", (b, L, H, P), x.dtype, dev)
    if return_final_states and final_states is None:
        final_states = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    elif final_states is not None:
        _need(final_states, "final_states", (b, H, P, N), torch.float32, dev)
    if reuse_group_operands and workspace is None:
        raise ValueError("reuse_group_operands needs the workspace of the earlier call")
    flags = (SSD_OPT_REUSE_GROUP_OPERANDS if reuse_group_operands else 0) | SSD_OPT_SEGSUM[segsum]
    opts = Options(split_len, flags, headdim_block)
    with torch.cuda.device(dev):
        ws_bytes = int(lib.ssd_fwd_ex_workspace_bytes(ctypes.byref(shape), chunk_size, io,
                                                      ctypes.byref(opts)))
        if ws_bytes and (workspace is None or workspace.numel() < ws_bytes):
            if reuse_group_operands:
                raise ValueError(f"reuse_group_operands: the workspace holds {workspace.numel()} "
                                 f"bytes, {ws_bytes} needed")
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
    args = (ctypes.byref(shape), io, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(seq_idx), chunk_size, _ptr(init_states), _ptr(y), _ptr(final_states),
            ctypes.byref(fused), _ptr(workspace) if ws_bytes else None, ws_bytes,
            ctypes.byref(opts), stream)
    keep = (shape, fused, opts, workspace)   # the byref targets live as long as the closure
    fn = lib.ssd_fwd_fused

    def launch():
        _check(fn(*args))
        return keep

    return launch, y, final_states


def ssd_debug_chunk_mask(dt, A, seq_idx=None, chunk_size: int = 256, chunk_begin: int = 0,
                         chunk_count: Optional[int] = None, variant: str = "hierarchy",
                         sums_only: bool = False):
    """The decay mask of chunks [chunk_begin, chunk_begin + chunk_count) as the
    forward kernels build it (variant "hierarchy"), or by the dense direct or
    the prefix-difference segsum: fp32 [b, H, chunk_count, Q, Q].  With
    sums_only, only each chunk's sum of mask entries, fp32 [b, H, chunk_count]
    (the mask is evaluated but not written)."""
    import torch
    lib = load_library()
    if variant not in SEGSUM:
        raise ValueError(f"variant must be one of {sorted(SEGSUM)}")
    b, L, H = dt.shape
    dev = dt.device
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    if seq_idx is not None:
        _need(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    nchunks = (L + chunk_size - 1) // chunk_size
    if chunk_count is None:
        chunk_count = nchunks - chunk_begin
    out = None if sums_only else torch.empty((b, H, chunk_count, chunk_size, chunk_size),
                                             dtype=torch.float32, device=dev)
    sums = torch.empty((b, H, chunk_count), dtype=torch.float32, device=dev) if sums_only else None
    shape = Shape(b, L, H, 16, 16, 1)
    with torch.cuda.device(dev):
        st = lib.ssd_debug_chunk_mask_ex(ctypes.byref(shape), _ptr(dt), _ptr(A), _ptr(seq_idx),
                                         chunk_size, chunk_begin, chunk_count, SEGSUM[variant],
                                         _ptr(out), _ptr(sums), torch.cuda.current_stream(dev).cuda_stream)
    _check(st)
    return sums if sums_only else out


def ssd_debug_segsum_factors(dt, A, seq_idx=None, chunk_size: int = 256):
    """Segsum factor records (ssd.h) of every chunk as the mask export builds
    them: int32 view [b, H, nchunks, ssd_segsum_record_words(chunk_size)]
    (the words are fp32 values except last1 and blast1, which are int32)."""
    import torch
    lib = load_library()
    b, L, H = dt.shape
    dev = dt.device
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    if seq_idx is not None:
        _need(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    words = int(lib.ssd_segsum_record_words(chunk_size))
    nchunks = (L + chunk_size - 1) // chunk_size
    out = torch.empty((b, H, nchunks, max(words, 1)), dtype=torch.int32, device=dev)
    shape = Shape(b, L, H, 16, 16, 1)
    with torch.cuda.device(dev):
        st = lib.ssd_debug_segsum_factors(ctypes.byref(shape), _ptr(dt), _ptr(A), _ptr(seq_idx),
                                          chunk_size, _ptr(out), torch.cuda.current_stream(dev).cuda_stream)
    _check(st)
    return out


def ssd_debug_fwd_segsum_factors(x, dt, A, B, C, D=None, seq_idx=None, chunk_size: int = 256,
                                 init_states=None, split_len: int = 0, headdim_block: int = 0):
    """The bf16 forward pass with the head kernel's own segsum factor records:
    returns (y, final_states, records), records as ssd_debug_segsum_factors."""
    import torch
    lib = load_library()
    dev = x.device
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if x.dtype != torch.bfloat16:
        raise TypeError("the head kernel's segsum factor export is a bf16-path debug aid")
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if seq_idx is not None:
        _need(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    words = int(lib.ssd_segsum_record_words(chunk_size))
    nchunks = (L + chunk_size - 1) // chunk_size
    rec = torch.empty((b, H, nchunks, max(words, 1)), dtype=torch.int32, device=dev)
    y = torch.empty_like(x)
    fs = torch.empty((b, H, P, N), dtype=torch.float32, device=dev)
    shape = Shape(b, L, H, P, N, G)
    opts = Options(split_len, 0, headdim_block)
    with torch.cuda.device(dev):
        ws_bytes = int(lib.ssd_fwd_ex_workspace_bytes(ctypes.byref(shape), chunk_size, SSD_BF16,
                                                      ctypes.byref(opts)))
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        st = lib.ssd_debug_fwd_segsum_factors(
            ctypes.byref(shape), SSD_BF16, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
            _ptr(seq_idx), chunk_size, _ptr(init_states), _ptr(y), _ptr(fs), _ptr(ws), ws_bytes,
            ctypes.byref(opts), _ptr(rec), torch.cuda.current_stream(dev).cuda_stream)
    _check(st)
    return y, fs, rec


def ssd_debug_exp2_probe(first_bits: int, count: int, nthreads: int = 1 << 18, device="cuda"):
    """Run the device exp2 probe (ssd.h) over fp32 bit patterns [first_bits,
    first_bits + count); returns the summed counts (increases as the argument
    decreases, values above 1, values below 0 or NaN)."""
    import torch
    lib = load_library()
    counts = torch.zeros(3 * nthreads, dtype=torch.int32, device=device)
    dev = counts.device
    with torch.cuda.device(dev):
        st = lib.ssd_debug_exp2_probe(first_bits, count, _ptr(counts), nthreads,
                                      torch.cuda.current_stream(dev).cuda_stream)
    _check(st)
    c = counts.view(nthreads, 3).to(torch.int64).sum(0).cpu().tolist()
    return {"increases": c[0], "above_one": c[1], "negative_or_nan": c[2]}


def ssd_decode_step(x, dt, A, B, C, D, state, y=None, stream=None, dt_bias=None,
                    dt_softplus: bool = False, dt_limit=None, z=None):
    """One decode step: x [b, H, P], dt [b, H], B, C [b, G, N], A, D [H] (D may
    be None), state [b, H, P, N] fp32 updated in place.  Returns y [b, H, P].
    Fused dt map and output gate as in ssd_fwd (z [b, H, P] in x's dtype)."""
    import torch
    lib = load_library()
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [b, H, P] and B, C [b, G, N]")
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_decode_step runs on the GPU only (x is on %s)" % dev)
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    io = _io_code(x.dtype)
    _need(x, "x", (b, H, P), x.dtype, dev)
    _need(dt, "dt", (b, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, G, N), x.dtype, dev)
    _need(C, "C", (b, G, N), x.dtype, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    _need(state, "state", (b, H, P, N), torch.float32, dev)
    if dt_bias is not None:
        _need(dt_bias, "dt_bias", (H,), torch.float32, dev)
    if z is not None:
        _need(z, "z", (b, H, P), x.dtype, dev)
    fused = Fused(_ptr(dt_bias), _ptr(z), 1 if dt_softplus else 0,
                  0 if dt_limit is None else 1,
                  0.0 if dt_limit is None else float(dt_limit[0]),
                  0.0 if dt_limit is None else float(dt_limit[1]))
    if y is None:
        y = torch.empty_like(x)
    else:
        _need(y, "y", (b, H, P), x.dtype, dev)
    shape = Shape(b, 1, H, P, N, G)
    with torch.cuda.device(dev):
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.ssd_decode_step_fused(ctypes.byref(shape), io, _ptr(x), _ptr(dt), _ptr(A),
                                       _ptr(B), _ptr(C), _ptr(D), _ptr(state), _ptr(y),
                                       ctypes.byref(fused), stream)
    _check(st)
    return y


def ssd_bwd(x, dt, A, B, C, D, dy, seq_idx=None, init_states=None, dfinal=None, stream=None,
            workspace=None, out=None):
    """Gradients of J = <dy, y> + <dfinal, final_states> for y, final_states =
    ssd_fwd(x, dt, A, B, C, D, seq_idx, init_states=init_states): returns a
    dict of fp32 tensors dx, ddt, dA, dB, dC, dD (None if D is None) and
    dinit (None if init_states is None).  dy has x's dtype; dfinal is fp32
    [b, H, P, N] or None.  workspace: a uint8 device tensor of at least
    ssd_bwd_workspace_bytes (allocated per call when None); out: a dict of
    the output tensors to write (every gradient the call returns, each of the
    shape and fp32 dtype above), allocated per call when None."""
    import torch
    lib = load_library()
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("ssd_bwd runs on the GPU only (x is on %s)" % dev)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = _io_code(x.dtype)
    _need(x, "x", (b, L, H, P), x.dtype, dev)
    _need(dy, "dy", (b, L, H, P), x.dtype, dev)
    _need(dt, "dt", (b, L, H), torch.float32, dev)
    _need(A, "A", (H,), torch.float32, dev)
    _need(B, "B", (b, L, G, N), x.dtype, dev)
    _need(C, "C", (b, L, G, N), x.dtype, dev)
    if D is not None:
        _need(D, "D", (H,), torch.float32, dev)
    if seq_idx is not None:
        _need(seq_idx, "seq_idx", (b, L), torch.int32, dev)
    if init_states is not None:
        _need(init_states, "init_states", (b, H, P, N), torch.float32, dev)
    if dfinal is not None:
        _need(dfinal, "dfinal", (b, H, P, N), torch.float32, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    shapes = {"dx": (b, L, H, P), "ddt": (b, L, H), "dA": (H,), "dB": (b, L, G, N),
              "dC": (b, L, G, N), "dD": None if D is None else (H,),
              "dinit": None if init_states is None else (b, H, P, N)}
    if out is None:
        out = {k: None if v is None else torch.empty(v, **f32) for k, v in shapes.items()}
    else:
        out = dict(out)
        for k, v in shapes.items():
            if v is None:
                out[k] = None
            else:
                _need(out[k], k, v, torch.float32, dev)
    shape = Shape(b, L, H, P, N, G)
    with torch.cuda.device(dev):
        ws_bytes = int(lib.ssd_bwd_workspace_bytes(ctypes.byref(shape), io))
        if workspace is None:
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        else:
            if workspace.dtype != torch.uint8 or workspace.device != dev or not workspace.is_contiguous():
                raise ValueError("workspace: a contiguous uint8 tensor on %s" % dev)
            if workspace.numel() < ws_bytes:
                raise ValueError(f"workspace: {workspace.numel()} bytes, {ws_bytes} needed")
            ws = workspace
            ws_bytes = workspace.numel()
        if stream is None:
            stream = torch.cuda.current_stream(dev).cuda_stream
        st = lib.ssd_bwd(ctypes.byref(shape), io, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                         _ptr(D), _ptr(seq_idx), _ptr(init_states), _ptr(dy), _ptr(dfinal),
                         _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]),
                         _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]), _ptr(ws), ws_bytes,
                         stream)
    _check(st)
    return out
