"""Edge cases of the HIP path vs the fp64 oracle, through the C ABI (needs an
MI355X): rows shorter than one chunk (down to a single token), rows that end
one token into a chunk, no decay at all (A = 0: unnormalised causal linear
attention, page "State Space Duality and Mamba-2", "The Duality Revealed")
and total decay (a_t underflows to 0 within a token: only the diagonal of
the quadratic form survives).  Same parity bar as the other GPU tests."""
import numpy as np
import pytest

import workloads
from ssd_testlib import TOL, max_rel, oracle_slice, run_gpu

pytestmark = pytest.mark.gpu


def _check(inp, y, fs, init_states=None):
    tol = TOL[inp.wl.io]
    b, H = inp.wl.batch, inp.wl.nheads
    yr, fsr = oracle_slice(inp, range(b), range(H), init_states)
    ey, ef = max_rel(y, yr), max_rel(fs, fsr)
    assert ey <= tol and ef <= tol, f"{inp.wl.name}: y err {ey:.3e}, final_states err {ef:.3e}"


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("Q", [64, 256])
@pytest.mark.parametrize("L", [1, 2, 15, 16, 17, 63, 64, 65, 257])
def test_short_and_ragged_rows(io, Q, L):
    """Rows of L tokens with an entering state (so that even one token has a
    state-projection term) and, from three tokens on, a document boundary."""
    wl = workloads.custom_workload(name=f"edge_{io}_{Q}_{L}", batch=2, seqlen=L, nheads=4,
                                   headdim=64, dstate=64, ngroups=2, chunk_size=Q, io=io)
    inp = workloads.make_inputs(wl, seed=L)
    if L >= 3:
        seq = np.zeros((2, L), dtype=np.int32)
        seq[1, L // 2:] = 1
        inp.seq_idx = seq
    h0 = np.random.default_rng(L + 1).standard_normal((2, 4, 64, 64))
    y, fs = run_gpu(inp, init_states=h0)
    _check(inp, y, fs, h0)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_no_decay_is_linear_attention(io):
    """A = 0: every decay is exactly 1, the mask is all ones on the lower
    triangle and the state only accumulates."""
    wl = workloads.custom_workload(name=f"edge_a0_{io}", batch=2, seqlen=700, nheads=4,
                                   headdim=64, dstate=128, ngroups=1, chunk_size=256, io=io)
    inp = workloads.make_inputs(wl, seed=21)
    inp.A = np.zeros_like(inp.A)
    y, fs = run_gpu(inp)
    _check(inp, y, fs)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_total_decay_keeps_only_the_diagonal(io):
    """A = -1e4 with dt >= 1e-2: a_t = exp(dt A) underflows to 0 (fp32) at
    every token, so y_t = (C_t . B_t) dt_t x_t + D x_t and the final state
    is the last token's own dt x B^T (the fp64 oracle agrees to far below
    the tolerance)."""
    wl = workloads.custom_workload(name=f"edge_ainf_{io}", batch=2, seqlen=600, nheads=4,
                                   headdim=64, dstate=64, ngroups=2, chunk_size=128, io=io,
                                   dt_range=(1e-2, 1.0))
    inp = workloads.make_inputs(wl, seed=22)
    inp.A = np.full_like(inp.A, -1e4)
    y, fs = run_gpu(inp)
    _check(inp, y, fs)
    cb = np.einsum("blgn,blgn->blg", inp.B.astype(np.float64), inp.C.astype(np.float64))
    g = np.arange(4) // 2
    diag = (cb[:, :, g] * inp.dt)[..., None] * inp.x + inp.D[None, None, :, None] * inp.x
    assert max_rel(y, diag) <= TOL[io]
