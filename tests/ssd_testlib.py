"""Helpers shared by the GPU tests: move seeded inputs to the device, run
the HIP path through the C ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np

import oracle
import workloads


def to_device(inp: workloads.Inputs, device="cuda"):
    import torch
    io = torch.bfloat16 if inp.wl.io == "bf16" else torch.float32
    t = {
        "x": torch.from_numpy(inp.x).to(device).to(io).contiguous(),
        "dt": torch.from_numpy(inp.dt).to(device).contiguous(),
        "A": torch.from_numpy(inp.A).to(device).contiguous(),
        "B": torch.from_numpy(inp.B).to(device).to(io).contiguous(),
        "C": torch.from_numpy(inp.C).to(device).to(io).contiguous(),
        "D": torch.from_numpy(inp.D).to(device).contiguous(),
        "seq_idx": None if inp.seq_idx is None else torch.from_numpy(inp.seq_idx).to(device).contiguous(),
    }
    return t


def run_gpu(inp: workloads.Inputs, init_states=None, split_len=0, chunk_size=None, skip=True,
            **kw):
    """Run the HIP path; skip=False drops the D x term (D = None).  y and
    final_states start out NaN, so any element the kernels leave unwritten
    fails every comparison."""
    import ssd_chunked_scan_amd as ssd
    import torch
    t = to_device(inp)
    h0 = None if init_states is None else torch.from_numpy(np.asarray(init_states, np.float32)).cuda()
    b, L, H, P = inp.x.shape
    N = inp.B.shape[3]
    y = torch.full_like(t["x"], float("nan"))
    fs = torch.full((b, H, P, N), float("nan"), dtype=torch.float32, device=t["x"].device)
    y, fs = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"] if skip else None, t["seq_idx"],
                        chunk_size=chunk_size or inp.wl.chunk_size, init_states=h0,
                        split_len=split_len, y=y, final_states=fs, **kw)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), fs.cpu().numpy().astype(np.float64)


def oracle_slice(inp: workloads.Inputs, batches, heads, init_states=None, skip=True):
    """fp64 oracle on a subset of (batch rows, heads); B/C groups follow the
    heads.  Returns y [nb, L, nh, P] and final_states [nb, nh, P, N]."""
    H, G = inp.wl.nheads, inp.wl.ngroups
    hpg = H // G
    batches = list(batches)
    heads = list(heads)
    groups = [h // hpg for h in heads]
    x = inp.x[batches][:, :, heads]
    dt = inp.dt[batches][:, :, heads]
    A = inp.A[heads]
    D = inp.D[heads] if skip else None
    # one group per selected head keeps the head -> group map exact
    B = inp.B[batches][:, :, groups]
    C = inp.C[batches][:, :, groups]
    si = None if inp.seq_idx is None else inp.seq_idx[batches]
    h0 = None if init_states is None else np.asarray(init_states)[batches][:, heads]
    return oracle.ssd_forward(x, dt, A, B, C, D, si, h0)


def max_rel(a, ref):
    """max |a - ref| / max |ref| over the whole array; inf if a holds a
    non-finite value (an unwritten, NaN-poisoned element included)."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    if a.shape != ref.shape:
        raise ValueError(f"shape {a.shape} vs reference {ref.shape}")
    if not np.isfinite(a).all():
        return float("inf")
    return float(np.abs(a - ref).max() / max(np.abs(ref).max(), 1e-30))


# Measured worst-case relative errors of the whole-tensor parity tests,
# printed in the terminal summary (tests/conftest.py) so that the margin to
# the tolerance is visible in the test output.
ERRORS = []


def record_error(label, ey, ef, tol):
    ERRORS.append((label, ey, ef, tol))


TOL = {"bf16": 1e-2, "f32": 1e-4}
