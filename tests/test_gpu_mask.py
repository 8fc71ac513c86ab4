"""The decay mask exactly as the kernels build it (debug export through the C
ABI) against the fp64 mask oracle and against the invariants the pages fix:
entries in [0, 1], ones on the diagonal, zeros above it and across document
boundaries, and non-increasing along each row away from the diagonal (page
"GPU Hierarchy Meets Structured Matrices", abstract: stable segsum without
monotonicity violations)."""
import numpy as np
import pytest

import oracle
import workloads
from mask_invariants import check_mask_invariants as _invariants

pytestmark = pytest.mark.gpu


def _mask(inp, Q, begin=0, count=None, seq_idx=None):
    import torch
    import ssd_chunked_scan_amd as ssd
    dt = torch.from_numpy(inp.dt).cuda()
    A = torch.from_numpy(inp.A).cuda()
    si = None if seq_idx is None else torch.from_numpy(seq_idx).cuda()
    m = ssd.ssd_debug_chunk_mask(dt, A, si, chunk_size=Q, chunk_begin=begin, chunk_count=count)
    torch.cuda.synchronize()
    return m.cpu().numpy()


def test_mask_tiny_vs_oracle():
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"], seed=0)
    m = _mask(inp, 64)
    ref = oracle.decay_mask(inp.dt, inp.A, chunk_size=64)
    assert m.shape == ref.shape
    assert np.abs(m - ref).max() <= 2e-6
    assert np.all(np.diagonal(m, axis1=-2, axis2=-1) == 1.0)
    _invariants(m)


@pytest.mark.parametrize("Q", [64, 128, 256])
def test_mask_ragged_tail_and_resets(Q):
    wl = workloads.custom_workload(seqlen=3 * Q - 29, nheads=3, chunk_size=Q, packed=True,
                                   doc_range=(1, 90), doc_count=(2, 400),
                                   dt_range=(1e-3, 1.0), a_range=(0.5, 20.0))
    inp = workloads.make_inputs(wl, seed=7)
    m = _mask(inp, Q, seq_idx=inp.seq_idx)
    ref = oracle.decay_mask(inp.dt, inp.A, inp.seq_idx, chunk_size=Q)
    assert np.abs(m - ref).max() <= 1e-5
    # exact zeros across documents and past the end of the row
    assert np.all(m[ref == 0] == 0.0)
    _invariants(m)


def test_mask_linear_attention_exact_ones():
    wl = workloads.custom_workload(seqlen=300, nheads=2, chunk_size=128)
    inp = workloads.make_inputs(wl, seed=8)
    inp.A[:] = 0.0
    m = _mask(inp, 128)
    Q = 128
    tri = np.tril(np.ones((Q, Q), dtype=np.float32))
    assert np.array_equal(m[0, :, 0], np.broadcast_to(tri, (2, Q, Q)))
    tail = 300 - 2 * Q
    assert np.array_equal(m[0, :, 2, :tail, :tail], np.broadcast_to(tri[:tail, :tail], (2, tail, tail)))
    assert np.all(m[0, :, 2, tail:, :] == 0) and np.all(m[0, :, 2, :, tail:] == 0)


def test_mask_decay_stress_slices():
    """Decay-stress workload (dt in [1e-2, 1], A in -[4, 64]): most entries
    underflow to exactly 0; the rest must keep the invariants.  Checked on
    slices of chunks across the 65536-token row."""
    wl = workloads.WORKLOADS["decay"]
    inp = workloads.make_inputs(wl, seed=0)
    for begin in (0, 97, 255):
        m = _mask(inp, 256, begin=begin, count=1)
        _invariants(m)
        ref = oracle.decay_mask(inp.dt, inp.A, chunk_size=256, chunk_begin=begin, chunk_count=1)
        assert np.abs(m - ref).max() <= 1e-5


def test_mask_tiny_decay_steps_stay_monotone():
    """Decays so close to 1 that adjacent mask values differ by less than an
    fp32 ulp: the nested construction still never increases along a row."""
    wl = workloads.custom_workload(seqlen=512, nheads=2, chunk_size=256, dt_range=(1e-9, 1e-7),
                                   a_range=(1e-3, 1e-2))
    inp = workloads.make_inputs(wl, seed=9)
    m = _mask(inp, 256)
    _invariants(m)
    assert np.all(np.diagonal(m, axis1=-2, axis2=-1) == 1.0)
