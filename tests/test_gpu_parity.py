"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Parity bar: max|y_gpu - y_ref| / max|y_ref| <= 1e-2 for bf16 inputs and
<= 1e-4 for fp32 inputs, final_states held to the same bound, on identical
seeded inputs.  Every test compares every element of y and final_states
with one oracle run over the whole call (the full-size workloads included,
in the launch configuration the benchmark times); the outputs start out NaN,
so an element the kernels never write fails.  The measured errors are listed
in the terminal summary.
"""
import numpy as np
import pytest

import workloads
from ssd_testlib import TOL, max_rel, oracle_slice, record_error, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    return workloads.custom_workload(name=name, **kw)


def _check_full(inp, y, fs, tol, init_states=None, skip=True, label=None):
    """Every element of y and final_states against the oracle over the whole
    call."""
    import oracle
    h0 = None if init_states is None else np.asarray(init_states, np.float64)
    yr, fsr = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D if skip else None,
                                 inp.seq_idx, h0)
    ey, ef = max_rel(y, yr), max_rel(fs, fsr)
    if label is not None:
        record_error(label, ey, ef, tol)
    assert ey <= tol and ef <= tol, f"{inp.wl.name}: y err {ey:.3e}, final_states err {ef:.3e}"
    return ey, ef


def test_tiny_fp32_workload():
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"], seed=0)
    y, fs = run_gpu(inp)
    _check_full(inp, y, fs, TOL["f32"], label="tiny fp32")


SHAPES = [
    # (Q, N, P, G, H, L)   ragged tails and several tiles everywhere
    (64, 16, 16, 1, 2, 200),
    (64, 64, 64, 2, 4, 333),
    (64, 128, 128, 1, 2, 150),
    (128, 32, 64, 1, 3, 300),
    (128, 64, 128, 4, 8, 517),
    (128, 128, 32, 2, 4, 260),
    (256, 16, 64, 1, 2, 700),
    (256, 64, 128, 2, 4, 600),
    (256, 128, 64, 1, 4, 1000),
    (256, 128, 128, 1, 2, 530),
    (256, 32, 16, 1, 2, 256),
]


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
@pytest.mark.parametrize("Q,N,P,G,H,L", SHAPES, ids=lambda v: str(v))
def test_bf16_shapes(Q, N, P, G, H, L, skip):
    """Without the D x skip (D = None) the error bound applies to the state-space
    part alone, which the skip term would otherwise dominate."""
    wl = _case(f"bf16_{Q}_{N}_{P}", batch=2, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G,
               chunk_size=Q, io="bf16")
    inp = workloads.make_inputs(wl, seed=1)
    y, fs = run_gpu(inp, skip=skip)
    _check_full(inp, y, fs, TOL["bf16"], skip=skip)


@pytest.mark.parametrize("Q,N,P,G,H,L", [(64, 16, 16, 1, 2, 190), (128, 64, 32, 2, 4, 300),
                                         (256, 128, 128, 1, 2, 300), (256, 32, 64, 1, 2, 513)],
                         ids=lambda v: str(v))
def test_fp32_shapes(Q, N, P, G, H, L):
    wl = _case(f"f32_{Q}_{N}_{P}", batch=2, seqlen=L, nheads=H, headdim=P, dstate=N, ngroups=G,
               chunk_size=Q, io="f32")
    inp = workloads.make_inputs(wl, seed=2)
    y, fs = run_gpu(inp)
    _check_full(inp, y, fs, TOL["f32"])


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("split_chunks", [1, 2, 3])
def test_forced_splits_with_init_state(io, split_chunks):
    Q = 64
    wl = _case(f"split_{io}", batch=2, seqlen=7 * Q - 5, nheads=4, headdim=32, dstate=64,
               ngroups=2, chunk_size=Q, io=io)
    inp = workloads.make_inputs(wl, seed=3)
    h0 = np.random.default_rng(4).standard_normal((2, 4, 32, 64)).astype(np.float32) * 0.5
    y, fs = run_gpu(inp, init_states=h0, split_len=split_chunks * Q)
    _check_full(inp, y, fs, TOL[io], init_states=h0)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_packed_documents_small(io):
    Q = 64
    wl = _case(f"packed_{io}", batch=2, seqlen=900, nheads=4, headdim=64, dstate=32, ngroups=2,
               chunk_size=Q, io=io, packed=True, doc_range=(1, 200), doc_count=(3, 64))
    inp = workloads.make_inputs(wl, seed=5)
    # also put boundaries exactly at a chunk start and at token 1
    si = inp.seq_idx.copy()
    si[0, 128:] += 100
    si[1, 1:] += 100
    inp.seq_idx[:] = si
    h0 = np.random.default_rng(6).standard_normal((2, 4, 64, 32)).astype(np.float32)
    y, fs = run_gpu(inp, init_states=h0)
    _check_full(inp, y, fs, TOL[io], init_states=h0)
    y2, fs2 = run_gpu(inp, init_states=h0, split_len=2 * Q)
    _check_full(inp, y2, fs2, TOL[io], init_states=h0)


# ----------------------------------------------------------- full-size workloads
# Each full-size call is compared element by element with one oracle run over
# the whole call (every batch row and head; the fp64 recurrence takes well
# under a second per workload on the host cores).

@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_layer27b_full_size(skip):
    """The benchmarked call: 8 x 2048 tokens, 80 heads, headdim 64, dstate 128,
    chunk 256, bf16, every unit of the launch (whole-headdim workgroups and the
    last round's half-headdim ones)."""
    inp = workloads.make_inputs(workloads.WORKLOADS["layer27b"], seed=0)
    y, fs = run_gpu(inp, skip=skip)
    _check_full(inp, y, fs, TOL["bf16"], skip=skip, label=f"layer27b {'skip' if skip else 'no skip'}")


def test_layer27b_bitwise_determinism():
    """Two calls of the benchmarked launch give identical bits."""
    inp = workloads.make_inputs(workloads.WORKLOADS["layer27b"], seed=0)
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_partial_last_round_half_blocks(skip):
    """288 (batch row, head) units of one workgroup each on a 256-CU device: the
    last 32 units (batch row 1, heads 112..143) run as two workgroups of half
    the headdim block each.  Ragged tail chunk, two groups."""
    wl = _case("half_blocks", batch=2, seqlen=600, nheads=144, headdim=64, dstate=128, ngroups=2,
               chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=3)
    y, fs = run_gpu(inp, skip=skip)
    _check_full(inp, y, fs, TOL["bf16"], skip=skip, label=f"half blocks {'skip' if skip else 'no skip'}")


def test_partial_last_round_half_blocks_uneven():
    """276 units on a 256-CU device: the last 20 run as half-headdim
    workgroups.  20 does not divide by the 8 XCDs, so the blocks take the
    other unit order (whole and half units each dealt in contiguous ranges);
    the 288-unit shapes above take the one-range-per-XCD order."""
    wl = _case("half_blocks_uneven", batch=2, seqlen=600, nheads=138, headdim=64, dstate=128,
               ngroups=2, chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=11)
    y, fs = run_gpu(inp)
    _check_full(inp, y, fs, TOL["bf16"], label="half blocks, 20 of 276 units")


def test_half_blocks_with_forced_splits_and_init_state():
    """The 288-unit shape in three sequence splits: 864 units, of which the last
    96 (batch row 1, heads 112..143, every split) run as half-headdim
    workgroups on a 256-CU device, through the split-local pass, the split
    scan and the full pass, with an entering state."""
    wl = _case("half_blocks_split", batch=2, seqlen=600, nheads=144, headdim=64, dstate=128,
               ngroups=2, chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=5)
    h0 = np.random.default_rng(6).standard_normal((2, 144, 64, 128)).astype(np.float32) * 0.5
    y, fs = run_gpu(inp, init_states=h0, split_len=256)
    _check_full(inp, y, fs, TOL["bf16"], init_states=h0, label="half blocks, 3 splits, h0")


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_decay_stress_full_size(skip):
    inp = workloads.make_inputs(workloads.WORKLOADS["decay"], seed=0)
    y, fs = run_gpu(inp, skip=skip)
    _check_full(inp, y, fs, TOL["bf16"], skip=skip, label=f"decay {'skip' if skip else 'no skip'}")


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_packed_full_size_and_per_document(skip):
    import oracle
    inp = workloads.make_inputs(workloads.WORKLOADS["packed"], seed=0)
    y, fs = run_gpu(inp, skip=skip)
    _check_full(inp, y, fs, TOL["bf16"], skip=skip, label=f"packed {'skip' if skip else 'no skip'}")
    # independent per-document oracle runs from a zero state, head 5 (group 1)
    lens = inp.doc_lens
    starts = np.concatenate([[0], np.cumsum(lens)])
    h, g = 5, 5 // 4
    for d in [0, len(lens) // 2, len(lens) - 1]:
        s0, s1 = starts[d], starts[d + 1]
        yd, fd = oracle.ssd_forward(inp.x[:, s0:s1, h:h + 1], inp.dt[:, s0:s1, h:h + 1],
                                    inp.A[h:h + 1], inp.B[:, s0:s1, g:g + 1],
                                    inp.C[:, s0:s1, g:g + 1], inp.D[h:h + 1] if skip else None)
        e = max_rel(y[:, s0:s1, h:h + 1], yd)
        assert e <= TOL["bf16"], f"document {d}: {e:.3e}"
        if d == len(lens) - 1:
            assert max_rel(fs[:, h:h + 1], fd) <= TOL["bf16"]


@pytest.mark.parametrize("b,L", workloads.SWEEP_SHAPES)
@pytest.mark.parametrize("Q", [128, 256])
def test_sweep_full_size(b, L, Q):
    """Every element, with the skip and without it (D = None)."""
    inp = workloads.make_inputs(workloads.WORKLOADS[f"sweep_b{b}_L{L}_q{Q}"], seed=0)
    y, fs = run_gpu(inp)
    _check_full(inp, y, fs, TOL["bf16"], label=f"sweep b{b} L{L} Q{Q} skip")
    y, fs = run_gpu(inp, skip=False)
    _check_full(inp, y, fs, TOL["bf16"], skip=False, label=f"sweep b{b} L{L} Q{Q} no skip")
