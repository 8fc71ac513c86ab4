"""Single-token decode step (the recurrence of page "State Space Duality and
Mamba-2", "The Mathematical Bridge", one token at a time) through the C ABI,
against the fp64 oracle run over the same tokens with the state as its
initial state, and as the continuation of the chunked forward pass."""
import numpy as np
import pytest

import oracle
import workloads
from ssd_testlib import TOL, max_rel, run_gpu

pytestmark = pytest.mark.gpu


def _dev(a, io="f32"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if io == "bf16" and t.dtype == torch.float32 else t


def _decode(inp, t, state, io, skip=True):
    """Decode token t of inp from `state` (numpy fp32); returns (y [b, H, P], state)."""
    import torch
    import ssd_chunked_scan_amd as ssd
    st = _dev(state.astype(np.float32))
    y = ssd.ssd_decode_step(_dev(inp.x[:, t], io), _dev(inp.dt[:, t]), _dev(inp.A),
                            _dev(inp.B[:, t], io), _dev(inp.C[:, t], io),
                            _dev(inp.D) if skip else None, st)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), st.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("P,N,G,H", [(64, 128, 1, 8), (16, 16, 2, 4), (128, 64, 4, 8), (32, 32, 1, 3)])
def test_decode_one_token_vs_oracle(io, P, N, G, H):
    wl = workloads.custom_workload(name="decode", batch=3, seqlen=1, nheads=H, headdim=P, dstate=N,
                                   ngroups=G, io=io)
    inp = workloads.make_inputs(wl, seed=21)
    h0 = np.random.default_rng(22).standard_normal((3, H, P, N)).astype(np.float32)
    y, st = _decode(inp, 0, h0, io)
    yr, fr = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, init_states=h0)
    ey, es = max_rel(y, yr[:, 0]), max_rel(st, fr)
    assert ey <= TOL[io] and es <= TOL[io], f"y {ey:.3e} state {es:.3e}"


def test_decode_sixteen_steps_from_zero_vs_oracle():
    """16 steps from a zero state (no D term) reproduce the oracle's forward
    pass over those 16 tokens, output by output and the final state."""
    wl = workloads.custom_workload(name="decode16", batch=2, seqlen=16, nheads=4, headdim=32,
                                   dstate=64, ngroups=2, io="f32")
    inp = workloads.make_inputs(wl, seed=23)
    yr, fr = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, None)
    state = np.zeros((2, 4, 32, 64), np.float32)
    for t in range(16):
        y, state = _decode(inp, t, state, "f32", skip=False)
        assert max_rel(y, yr[:, t]) <= TOL["f32"], f"token {t}"
        state = state.astype(np.float32)
    assert max_rel(state, fr) <= TOL["f32"]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_continues_the_forward_pass(io):
    """Chunked forward over 299 tokens, then one decode step with token 299,
    equals the oracle over all 300 tokens at the last output and final state."""
    L = 300
    wl = workloads.custom_workload(name="decode_cont", batch=2, seqlen=L, nheads=4, headdim=64,
                                   dstate=128, ngroups=1, chunk_size=128, io=io)
    inp = workloads.make_inputs(wl, seed=24)
    head = workloads.Inputs(**{**inp.__dict__, "x": inp.x[:, :L - 1], "dt": inp.dt[:, :L - 1],
                               "B": inp.B[:, :L - 1], "C": inp.C[:, :L - 1]})
    _, fs = run_gpu(head)
    y, st = _decode(inp, L - 1, fs.astype(np.float32), io)
    yr, fr = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D)
    ey, es = max_rel(y, yr[:, L - 1]), max_rel(st, fr)
    assert ey <= TOL[io] and es <= TOL[io], f"y {ey:.3e} state {es:.3e}"


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_decode_fused_continues_the_fused_forward(io):
    """The fused forward (raw dt through bias + softplus, silu(z) gate) over
    299 tokens, then one fused decode step with token 299, equals the
    oracle's fused forward over all 300 tokens at the last output and the
    final state."""
    import torch
    import ssd_chunked_scan_amd as ssd
    L = 300
    wl = workloads.custom_workload(name="decode_fused", batch=2, seqlen=L, nheads=4, headdim=64,
                                   dstate=64, ngroups=2, chunk_size=128, io=io)
    inp = workloads.make_inputs(wl, seed=25)
    fz = workloads.make_fused_inputs(inp, seed=25)
    t = lambda a, conv=False: _dev(np.ascontiguousarray(a), io if conv else "f32")
    bias = t(fz.dt_bias)
    _, fs = ssd.ssd_fwd(t(inp.x[:, :L - 1], True), t(fz.dt_raw[:, :L - 1]), t(inp.A),
                        t(inp.B[:, :L - 1], True), t(inp.C[:, :L - 1], True), t(inp.D),
                        chunk_size=128, dt_bias=bias, dt_softplus=True, dt_limit=(1e-3, 0.1),
                        z=t(fz.z[:, :L - 1], True))
    y = ssd.ssd_decode_step(t(inp.x[:, L - 1], True), t(fz.dt_raw[:, L - 1]), t(inp.A),
                            t(inp.B[:, L - 1], True), t(inp.C[:, L - 1], True), t(inp.D), fs,
                            dt_bias=bias, dt_softplus=True, dt_limit=(1e-3, 0.1),
                            z=t(fz.z[:, L - 1], True))
    torch.cuda.synchronize()
    yr, fr = oracle.ssd_forward_fused(inp.x, fz.dt_raw, inp.A, inp.B, inp.C, inp.D,
                                      dt_bias=fz.dt_bias, dt_softplus=True, dt_limit=(1e-3, 0.1),
                                      z=fz.z)
    ey = max_rel(y.float().cpu().numpy(), yr[:, L - 1])
    es = max_rel(fs.cpu().numpy(), fr)
    assert ey <= TOL[io] and es <= TOL[io], f"y {ey:.3e} state {es:.3e}"
