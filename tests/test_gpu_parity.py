"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Parity bar: max|y_gpu - y_ref| / max|y_ref| <= 1e-2 for bf16 inputs and
<= 1e-4 for fp32 inputs, final_states held to the same bound, on identical
seeded inputs.  Small cases compare every element; the full-size workloads
compare every output of a sample of (batch row, head) pairs that the oracle
computes independently.
"""
import numpy as np
import pytest

import workloads
from ssd_testlib import TOL, max_rel, oracle_slice, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _case(name, **kw):
    return workloads.custom_workload(name=name, **kw)


def _check_full(inp, y, fs, tol, init_states=None, skip=True):
    b, H = inp.wl.batch, inp.wl.nheads
    yr, fsr = oracle_slice(inp, range(b), range(H), init_states, skip=skip)
    ey, ef = max_rel(y, yr), max_rel(fs, fsr)
    assert ey <= tol and ef <= tol, f"{inp.wl.name}: y err {ey:.3e}, final_states err {ef:.3e}"
    return ey, ef


def test_tiny_fp32_workload():
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"], seed=0)
    y, fs = run_gpu(inp)
    _check_full(inp, y, fs, TOL["f32"])


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

def _sampled(inp, pairs, y, fs, tol, label, skip=True):
    worst = 0.0
    for b, h in pairs:
        yr, fsr = oracle_slice(inp, [b], [h], skip=skip)
        ey = max_rel(y[b:b + 1, :, h:h + 1], yr)
        ef = max_rel(fs[b:b + 1, h:h + 1], fsr)
        worst = max(worst, ey, ef)
        assert ey <= tol and ef <= tol, f"{label} (b={b}, h={h}): y {ey:.3e} fs {ef:.3e}"
    return worst


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_layer27b_full_size_sampled(skip):
    inp = workloads.make_inputs(workloads.WORKLOADS["layer27b"], seed=0)
    y, fs = run_gpu(inp, skip=skip)
    assert np.isfinite(y).all() and np.isfinite(fs).all()
    pairs = [(0, 0), (3, 41), (7, 79), (5, 17)]
    _sampled(inp, pairs, y, fs, TOL["bf16"], "layer27b", skip=skip)


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_partial_last_round_half_blocks(skip):
    """288 (batch row, head) units of one workgroup each on a 256-CU device: the
    last 32 units (batch row 1, heads 112..143) run as two workgroups of half
    the headdim block each.  Samples on both sides of that boundary, ragged
    tail chunk, two groups."""
    wl = _case("half_blocks", batch=2, seqlen=600, nheads=144, headdim=64, dstate=128, ngroups=2,
               chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=3)
    y, fs = run_gpu(inp, skip=skip)
    assert np.isfinite(y).all() and np.isfinite(fs).all()
    _sampled(inp, [(0, 5), (1, 111), (1, 112), (1, 127), (1, 143)], y, fs, TOL["bf16"],
             "half blocks", skip=skip)


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
    assert np.isfinite(y).all() and np.isfinite(fs).all()
    for b, h in [(0, 0), (1, 111), (1, 112), (1, 143)]:
        yr, fsr = oracle_slice(inp, [b], [h], init_states=h0)
        ey = max_rel(y[b:b + 1, :, h:h + 1], yr)
        ef = max_rel(fs[b:b + 1, h:h + 1], fsr)
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"], f"(b={b}, h={h}): y {ey:.3e} fs {ef:.3e}"


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_decay_stress_full_size_sampled(skip):
    inp = workloads.make_inputs(workloads.WORKLOADS["decay"], seed=0)
    y, fs = run_gpu(inp, skip=skip)
    assert np.isfinite(y).all() and np.isfinite(fs).all()
    _sampled(inp, [(0, 0), (0, 9)], y, fs, TOL["bf16"], "decay", skip=skip)


@pytest.mark.parametrize("skip", [True, False], ids=["with_skip", "no_skip"])
def test_packed_full_size_sampled_and_per_document(skip):
    import oracle
    inp = workloads.make_inputs(workloads.WORKLOADS["packed"], seed=0)
    y, fs = run_gpu(inp, skip=skip)
    assert np.isfinite(y).all()
    _sampled(inp, [(0, 0), (0, 13), (0, 31)], y, fs, TOL["bf16"], "packed", skip=skip)
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
def test_sweep_sampled(b, L, Q):
    """Sampled with the skip for one head and without it (D = None) for another."""
    inp = workloads.make_inputs(workloads.WORKLOADS[f"sweep_b{b}_L{L}_q{Q}"], seed=0)
    y, fs = run_gpu(inp)
    _sampled(inp, [(b - 1, 31), (0, 7)], y, fs, TOL["bf16"], f"sweep b{b} L{L} Q{Q}")
    y, fs = run_gpu(inp, skip=False)
    _sampled(inp, [(0, 3)], y, fs, TOL["bf16"], f"sweep b{b} L{L} Q{Q} no skip", skip=False)
