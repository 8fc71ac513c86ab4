"""The bf16 head kernel's own segsum factors against the mask export's, bit
for bit (needs an MI355X).

The hierarchy-aware segsum (page "GPU Hierarchy Meets Structured Matrices",
abstract) is built twice in the library: the bf16 head kernel sums each
16-token sub-block with row shifts across the lanes of a wave (its producer
waves, as it streams the chunk), and the mask export -- whose values the mask
tests hold to the fp64 mask oracle and to the [0, 1] / monotone invariants --
sums them with sequential per-token loops.  Both add the same terms in the
same order, so every factor (d, dt, W dt, Tb, Tp and the reset positions)
must agree exactly; then everything the mask tests prove of the export's
factors holds for the factors the forward pass multiplies with.  The forward
pass that writes the records must also return exactly what it returns
without them."""
import numpy as np
import pytest

import workloads
from ssd_testlib import to_device

pytestmark = pytest.mark.gpu


def _compare(inp, chunk_size=None, split_len=0, headdim_block=0):
    import torch
    import ssd_chunked_scan_amd as ssd
    Q = chunk_size or inp.wl.chunk_size
    t = to_device(inp)
    y, fs, rec = ssd.ssd_debug_fwd_segsum_factors(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"],
                                                  t["seq_idx"], chunk_size=Q, split_len=split_len,
                                                  headdim_block=headdim_block)
    ref = ssd.ssd_debug_segsum_factors(t["dt"], t["A"], t["seq_idx"], chunk_size=Q)
    y0, f0 = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["seq_idx"], chunk_size=Q,
                         split_len=split_len, headdim_block=headdim_block)
    torch.cuda.synchronize()
    assert rec.shape == ref.shape
    diff = (rec != ref)
    if diff.any():
        where = torch.nonzero(diff)[:5].tolist()
        raise AssertionError(f"{int(diff.sum())} factor words differ, first at {where}")
    assert torch.equal(y, y0) and torch.equal(fs, f0), "the factor export changed the outputs"
    return rec.cpu().numpy()


@pytest.mark.parametrize("Q", [64, 128, 256])
def test_factors_with_resets_and_ragged_tail(Q):
    wl = workloads.custom_workload(name=f"seg_{Q}", batch=2, seqlen=3 * Q - 29, nheads=3, headdim=32,
                                   dstate=32, chunk_size=Q, io="bf16", packed=True,
                                   doc_range=(1, 90), doc_count=(2, 400), dt_range=(1e-3, 1.0),
                                   a_range=(0.5, 20.0))
    inp = workloads.make_inputs(wl, seed=31)
    rec = _compare(inp)
    # the resets really are exercised: some last1 words are nonzero
    import ssd_chunked_scan_amd as ssd
    words = int(ssd.load_library().ssd_segsum_record_words(Q))
    assert rec.shape[-1] == words
    assert (rec[..., 3 * Q:4 * Q] != 0).any()


def test_factors_forced_splits_and_half_headdim_blocks():
    wl = workloads.custom_workload(name="seg_split", batch=2, seqlen=1000, nheads=4, headdim=64,
                                   dstate=64, chunk_size=128, io="bf16")
    inp = workloads.make_inputs(wl, seed=32)
    _compare(inp, split_len=256)
    _compare(inp, headdim_block=32)


def test_factors_decay_stress_full_size():
    """The decay-stress workload (1 x 65536, 16 heads, dt in [1e-2, 1], A in
    -[4, 64]): a 16-token sub-block decays by e^-74 on average, so many
    sub-block decays underflow to exactly 0 (measured: 30%) and the pair
    decays Tp, products of two of them, more often still."""
    inp = workloads.make_inputs(workloads.WORKLOADS["decay"], seed=0)
    rec = _compare(inp)
    tb = rec[..., 4 * 256:4 * 256 + 16].view(np.float32)
    tp = rec[..., 4 * 256 + 32:4 * 256 + 40].view(np.float32)
    assert (tb == 0).mean() > 0.1 and (tb >= 0).all() and (tb <= 1).all()
    assert (tp == 0).mean() >= (tb == 0).mean() and (tp >= 0).all() and (tp <= 1).all()


def test_factors_packed_full_size():
    """The packed workload (1 x 32768, 32 heads, 8 groups, chunk 128, 8..64
    documents): resets inside and at the start of sub-blocks."""
    inp = workloads.make_inputs(workloads.WORKLOADS["packed"], seed=0)
    _compare(inp)
