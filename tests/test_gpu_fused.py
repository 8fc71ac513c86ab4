"""Fused prologue/epilogue of the HIP path (ssd_fwd_fused) vs the fp64
oracle's ssd_forward_fused, through the C ABI (needs an MI355X).

dt = clamp(softplus(dt_raw + dt_bias)) and out = (y + D x) * silu(z)
(page "NVIDIA Accelerates Mamba-2 Forward Kernel with CUDA Tile": the
element-wise gating around the scan, fused into its kernels).  Same parity
bar as the plain path: max|out_gpu - out_ref| / max|out_ref| <= 1e-2 for
bf16 inputs and <= 1e-4 for fp32, final_states to the same bound.
"""
import numpy as np
import pytest

import oracle
import workloads
from ssd_testlib import TOL, max_rel, to_device

pytestmark = pytest.mark.gpu


def _run(inp, fz, *, bias=True, softplus=True, limit=None, gate=True, split_len=0,
         init_states=None, chunk_size=None):
    import torch
    import ssd_chunked_scan_amd as ssd
    t = to_device(inp)
    io = torch.bfloat16 if inp.wl.io == "bf16" else torch.float32
    dt_raw = torch.from_numpy(fz.dt_raw).cuda().contiguous()
    kw = dict(dt_softplus=softplus, dt_limit=limit)
    if bias:
        kw["dt_bias"] = torch.from_numpy(fz.dt_bias).cuda().contiguous()
    if gate:
        kw["z"] = torch.from_numpy(fz.z).cuda().to(io).contiguous()
    h0 = None if init_states is None else torch.from_numpy(init_states.astype(np.float32)).cuda()
    y, fs = ssd.ssd_fwd(t["x"], dt_raw, t["A"], t["B"], t["C"], t["D"], t["seq_idx"],
                        chunk_size=chunk_size or inp.wl.chunk_size, init_states=h0,
                        split_len=split_len, **kw)
    torch.cuda.synchronize()
    yo, fso = oracle.ssd_forward_fused(
        inp.x, fz.dt_raw, inp.A, inp.B, inp.C, inp.D, inp.seq_idx, init_states,
        dt_bias=fz.dt_bias if bias else None, dt_softplus=softplus, dt_limit=limit,
        z=fz.z if gate else None)
    return (y.float().cpu().numpy().astype(np.float64), fs.cpu().numpy().astype(np.float64),
            yo, fso)


def _check(inp, y, fs, yo, fso):
    tol = TOL[inp.wl.io]
    ey, ef = max_rel(y, yo), max_rel(fs, fso)
    assert ey <= tol and ef <= tol, f"{inp.wl.name}: y err {ey:.3e}, final_states err {ef:.3e}"


SHAPES = [
    # (io, Q, N, P, G, H, L)   ragged tails, several tiles
    ("bf16", 64, 64, 64, 2, 4, 333),
    ("bf16", 128, 64, 128, 4, 8, 517),
    ("bf16", 256, 128, 64, 1, 4, 1000),
    ("bf16", 256, 32, 16, 1, 2, 300),
    ("bf16", 256, 128, 128, 2, 4, 600),     # two headdim blocks per head (tiles of 256 x 64)
    ("bf16", 64, 16, 32, 1, 2, 1),          # a single token
    ("f32", 64, 16, 16, 1, 2, 190),
    ("f32", 256, 128, 128, 1, 2, 300),
]


@pytest.mark.parametrize("io,Q,N,P,G,H,L", SHAPES, ids=lambda v: str(v))
def test_fused_shapes(io, Q, N, P, G, H, L):
    wl = workloads.custom_workload(name=f"fused_{io}_{Q}_{N}_{P}", batch=2, seqlen=L, nheads=H,
                                   headdim=P, dstate=N, ngroups=G, chunk_size=Q, io=io)
    inp = workloads.make_inputs(wl, seed=3)
    fz = workloads.make_fused_inputs(inp, seed=3)
    _check(inp, *_run(inp, fz, limit=(1e-3, 0.1)))


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("parts", ["bias_only", "softplus_only", "gate_only", "clamp_only"])
def test_fused_each_part_alone(io, parts):
    wl = workloads.custom_workload(name=f"fused_part_{io}", batch=2, seqlen=400, nheads=4,
                                   headdim=64, dstate=64, ngroups=2, chunk_size=128, io=io)
    inp = workloads.make_inputs(wl, seed=4)
    fz = workloads.make_fused_inputs(inp, seed=4)
    if parts != "softplus_only":
        # without softplus the raw values must already be positive step sizes
        fz = workloads.FusedInputs(inp.dt, np.abs(fz.dt_bias) * 1e-3, fz.z)
    kw = dict(bias=parts == "bias_only", softplus=parts == "softplus_only",
              gate=parts == "gate_only",
              limit=(0.01, 0.05) if parts == "clamp_only" else None)
    _check(inp, *_run(inp, fz, **kw))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_fused_with_resets_splits_and_init_state(io):
    """Packed documents, forced sequence splits and an entering state: the
    prologue must reach the split-local pass and the gate the full pass."""
    wl = workloads.custom_workload(name=f"fused_packed_{io}", batch=1, seqlen=2000, nheads=4,
                                   headdim=64, dstate=64, ngroups=2, chunk_size=128, io=io)
    inp = workloads.make_inputs(wl, seed=5)
    seq = np.zeros((1, 2000), dtype=np.int32)
    for k, cut in enumerate([130, 131, 700, 1500, 1999]):
        seq[0, cut:] = k + 1
    inp.seq_idx = seq
    fz = workloads.make_fused_inputs(inp, seed=5)
    h0 = np.random.default_rng(6).standard_normal((1, 4, 64, 64))
    _check(inp, *_run(inp, fz, split_len=512, init_states=h0, limit=(1e-3, 0.1)))


def test_fused_off_is_bitwise_plain_path():
    """No bias, no softplus, no clamp, no gate: exactly the plain call."""
    import torch
    import ssd_chunked_scan_amd as ssd
    wl = workloads.custom_workload(name="fused_off", batch=2, seqlen=700, nheads=4, headdim=64,
                                   dstate=128, ngroups=1, chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=7)
    t = to_device(inp)
    y1, f1 = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None, chunk_size=256)
    y2, f2 = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None, chunk_size=256,
                         dt_bias=torch.zeros(4, device="cuda"), dt_softplus=False, z=None)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_fused_zero_gate_gives_zero_and_keeps_state():
    import torch
    import ssd_chunked_scan_amd as ssd
    wl = workloads.custom_workload(name="fused_zero_gate", batch=1, seqlen=600, nheads=2,
                                   headdim=64, dstate=64, ngroups=1, chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=8)
    t = to_device(inp)
    z0 = torch.zeros_like(t["x"])
    y1, f1 = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None, chunk_size=256, z=z0)
    _, f2 = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None, chunk_size=256)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y1.float()) == 0
    assert torch.equal(f1, f2)


def test_fused_layer27b_full_size():
    """The benchmark layer (batch 8, seqlen 2048, 80 heads, headdim 64,
    dstate 128, chunk 256, bf16) with the prologue and the gate, every
    output against the oracle, in the launch configuration of the bench."""
    inp = workloads.make_inputs(workloads.WORKLOADS["layer27b"], seed=0)
    fz = workloads.make_fused_inputs(inp, seed=0)
    _check(inp, *_run(inp, fz))
