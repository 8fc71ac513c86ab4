"""The allocation-free entry point ssd_fwd_noalloc against ssd_fwd, through
the C ABI (needs an MI355X).  Both run the same kernels on the same inputs,
so the outputs must agree bit for bit; ssd_fwd_noalloc takes its workspace
from the library's fixed per-GPU array instead of the caller's.  Two calls in
a row, the second on a smaller problem (the array keeps the first call's
contents), and a problem whose workspace exceeds the array (refused, nothing
launched)."""
import ctypes

import numpy as np
import pytest

import workloads
from ssd_testlib import to_device

pytestmark = pytest.mark.gpu


def _noalloc(t, inp, chunk_size, D=True, h0=None):
    import torch
    import ssd_chunked_scan_amd as ssd
    lib = ssd.load_library()
    b, L, H, P = inp.x.shape
    G, N = inp.B.shape[2], inp.B.shape[3]
    io = 1 if inp.wl.io == "bf16" else 0
    y = torch.full_like(t["x"], float("nan"))
    fs = torch.full((b, H, P, N), float("nan"), dtype=torch.float32, device="cuda")
    shape = ssd.Shape(b, L, H, P, N, G)
    p = lambda v: None if v is None else v.data_ptr()
    st = lib.ssd_fwd_noalloc(ctypes.byref(shape), io, p(t["x"]), p(t["dt"]), p(t["A"]), p(t["B"]),
                             p(t["C"]), p(t["D"]) if D else None, p(t["seq_idx"]), chunk_size, p(h0),
                             p(y), p(fs), torch.cuda.current_stream().cuda_stream)
    return st, y, fs


def _reference(t, chunk_size, D=True, h0=None):
    import ssd_chunked_scan_amd as ssd
    return ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"] if D else None, t["seq_idx"],
                       chunk_size=chunk_size, init_states=h0)


def test_noalloc_matches_ssd_fwd_on_two_calls_in_a_row():
    import torch
    big = workloads.custom_workload(name="noalloc_big", batch=2, seqlen=1100, nheads=16, headdim=64,
                                    dstate=128, ngroups=2, chunk_size=256, io="bf16", packed=True,
                                    doc_range=(50, 700), doc_count=(2, 64))
    small = workloads.custom_workload(name="noalloc_small", batch=1, seqlen=300, nheads=4, headdim=32,
                                      dstate=64, ngroups=1, chunk_size=128, io="bf16")
    for k, wl in enumerate((big, small)):
        inp = workloads.make_inputs(wl, seed=40 + k)
        t = to_device(inp)
        h0 = torch.from_numpy(np.random.default_rng(50 + k).standard_normal(
            (wl.batch, wl.nheads, wl.headdim, wl.dstate)).astype(np.float32)).cuda()
        st, y, fs = _noalloc(t, inp, wl.chunk_size, h0=h0)
        assert st == 0, st
        yr, fsr = _reference(t, wl.chunk_size, h0=h0)
        torch.cuda.synchronize()
        assert torch.equal(y, yr) and torch.equal(fs, fsr), wl.name


def test_noalloc_fp32_and_without_skip():
    import torch
    wl = workloads.custom_workload(name="noalloc_f32", batch=2, seqlen=500, nheads=4, headdim=32,
                                   dstate=32, ngroups=2, chunk_size=64, io="f32")
    inp = workloads.make_inputs(wl, seed=43)
    t = to_device(inp)
    st, y, fs = _noalloc(t, inp, 64, D=False)
    assert st == 0, st
    yr, fsr = _reference(t, 64, D=False)
    torch.cuda.synchronize()
    assert torch.equal(y, yr) and torch.equal(fs, fsr)


def test_noalloc_refuses_a_workspace_above_its_array():
    """The packed-document workload (1 x 32768 tokens, 32 heads, 8 groups,
    chunk 128) needs more per-group workspace than the array holds."""
    import torch
    import ssd_chunked_scan_amd as ssd
    wl = workloads.WORKLOADS["packed"]
    shape = ssd.Shape(wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups)
    assert ssd.ssd_fwd_workspace_bytes(shape, wl.chunk_size, 1) > (64 << 20)
    inp = workloads.make_inputs(wl, seed=0)
    t = to_device(inp)
    st, y, fs = _noalloc(t, inp, wl.chunk_size)
    torch.cuda.synchronize()
    assert st == 5
    assert b"ssd_fwd_noalloc" in ssd.load_library().ssd_last_error()
    assert torch.isnan(fs).all()      # nothing was launched
