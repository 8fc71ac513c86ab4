"""Segsum ablation (page "GPU Hierarchy Meets Structured Matrices", abstract):
the same chunk decay mask by the hierarchy-aware segsum the forward kernels
use, by the dense direct segsum and by the prefix-difference ("diff") segsum,
through the C ABI's mask export, against the fp64 mask oracle.  The page's
claims checked here: direct and hierarchy-aware are both accurate and the
hierarchy-aware mask keeps the invariants (entries in [0, 1], non-increasing
along a row away from the diagonal); the diff segsum loses accuracy to
cancellation and breaks the invariants once the chunk's prefix sums are large
next to the decays that follow.  The same three evaluations also run inside
the fp32 forward pass and on the output path of the bf16 head kernel at
chunk 256 (option flags of ssd_fwd_ex), against the fp64 recurrence; there a
constructed chunk shows the prefix differences' cancellation in y."""
import numpy as np
import pytest

import oracle
import workloads
from mask_invariants import check_mask_invariants

pytestmark = pytest.mark.gpu

VARIANTS = ("hierarchy", "direct", "diff")


def _mask(dt, A, Q, variant, seq_idx=None, sums_only=False, begin=0, count=None):
    import torch
    import ssd_chunked_scan_amd as ssd
    si = None if seq_idx is None else torch.from_numpy(seq_idx).cuda()
    m = ssd.ssd_debug_chunk_mask(torch.from_numpy(dt).cuda(), torch.from_numpy(A).cuda(), si,
                                 chunk_size=Q, chunk_begin=begin, chunk_count=count,
                                 variant=variant, sums_only=sums_only)
    torch.cuda.synchronize()
    return m.cpu().numpy()


@pytest.mark.parametrize("Q", [64, 256])
def test_variants_match_oracle_with_resets_and_ragged_tail(Q):
    wl = workloads.custom_workload(seqlen=3 * Q - 29, nheads=3, chunk_size=Q, packed=True,
                                   doc_range=(1, 90), doc_count=(2, 400),
                                   dt_range=(1e-3, 1.0), a_range=(0.5, 20.0))
    inp = workloads.make_inputs(wl, seed=7)
    ref = oracle.decay_mask(inp.dt, inp.A, inp.seq_idx, chunk_size=Q)
    tol = {"hierarchy": 1e-5, "direct": 1e-5, "diff": 1e-3}
    for v in VARIANTS:
        m = _mask(inp.dt, inp.A, Q, v, inp.seq_idx)
        assert m.shape == ref.shape
        err = np.abs(m - ref).max()
        assert err <= tol[v], f"{v}: {err:.3e}"
        # exact zeros above the diagonal, across documents and past the row end
        assert np.all(m[ref == 0] == 0.0), v
    check_mask_invariants(_mask(inp.dt, inp.A, Q, "hierarchy", inp.seq_idx))


def _strong_then_tiny(Q=256, heads=2):
    """One chunk: strong decays on its first half (d = dt A log2 e ~ -58 per
    token), decays of ~6e-5 on its second half.  The prefix sums reach ~-7400,
    where an fp32 ulp (~5e-4) exceeds the later decays."""
    dt = np.full((1, Q, heads), 1e-6, np.float32)
    dt[:, :Q // 2] = 1.0
    A = np.full(heads, -40.0, np.float32)
    return dt, A


def test_diff_segsum_breaks_invariants_hierarchy_keeps_them():
    Q = 256
    dt, A = _strong_then_tiny(Q)
    ref = oracle.decay_mask(dt, A, chunk_size=Q)
    mh = _mask(dt, A, Q, "hierarchy")
    md = _mask(dt, A, Q, "direct")
    mf = _mask(dt, A, Q, "diff")
    eh, ed, ef = (np.abs(m - ref).max() for m in (mh, md, mf))
    assert eh <= 1e-6 and ed <= 1e-6, (eh, ed)
    check_mask_invariants(mh)
    # the diff segsum: cancellation error far above the other two, entries
    # above 1 and increases along rows (a monotonicity violation)
    assert ef >= 1e-4 and ef >= 100 * max(eh, ed), (ef, eh, ed)
    assert (mf > 1.0).any()
    lower = np.tril(np.ones((Q, Q - 1), dtype=bool), -1)
    rises = (mf[..., :, :-1] - mf[..., :, 1:])[..., lower] > 0     # L[i, j-1] > L[i, j]
    assert rises.any()
    with pytest.raises(AssertionError):
        check_mask_invariants(mf)


@pytest.mark.parametrize("variant", VARIANTS)
def test_sums_only_is_the_sum_of_the_mask(variant):
    Q = 128
    wl = workloads.custom_workload(seqlen=2 * Q + 40, nheads=3, chunk_size=Q)
    inp = workloads.make_inputs(wl, seed=11)
    m = _mask(inp.dt, inp.A, Q, variant).astype(np.float64)
    sums = _mask(inp.dt, inp.A, Q, variant, sums_only=True)
    assert sums.shape == m.shape[:3]
    np.testing.assert_allclose(sums, m.sum(axis=(-1, -2)), rtol=1e-5)


# --------------------------------------------------------------------------
# The same three evaluations inside the forward pass (fp32 path, ssd_fwd_ex
# option flags): only the intra-chunk mask changes.

def _fwd_variant(inp, variant, init_states=None, **kw):
    from ssd_testlib import run_gpu
    return run_gpu(inp, init_states=init_states, segsum=variant, **kw)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("Q", [64, 256])
def test_forward_variants_match_oracle(variant, Q):
    """Moderate decays, document resets, a ragged tail and an entering state:
    each evaluation meets the fp32 bound against the fp64 oracle."""
    from ssd_testlib import TOL, max_rel, oracle_slice
    wl = workloads.custom_workload(name=f"fwd_seg_{variant}", batch=2, seqlen=3 * Q - 29,
                                   nheads=3, headdim=32, dstate=32, chunk_size=Q, packed=True,
                                   doc_range=(20, 300), doc_count=(2, 400))
    inp = workloads.make_inputs(wl, seed=9)
    h0 = np.random.default_rng(10).standard_normal((2, 3, 32, 32))
    y, fs = _fwd_variant(inp, variant, h0)
    yr, fsr = oracle_slice(inp, range(2), range(3), h0)
    ey, ef = max_rel(y, yr), max_rel(fs, fsr)
    assert ey <= TOL["f32"] and ef <= TOL["f32"], f"{variant}: y {ey:.2e} fs {ef:.2e}"


def test_forward_deep_decay_variants():
    """The decay-stress distribution (dt in [1e-2, 1], A in -[4, 64]) at chunk
    256, fp32: hierarchy-aware and direct stay at the fp32 bound; the diff
    segsum, whose prefix sums reach thousands before decays of a few units,
    is less accurate (its error is reported)."""
    from ssd_testlib import TOL, max_rel, oracle_slice
    wl = workloads.custom_workload(name="fwd_seg_deep", batch=1, seqlen=2048, nheads=4,
                                   headdim=32, dstate=32, chunk_size=256,
                                   dt_range=(1e-2, 1.0), a_range=(4.0, 64.0))
    inp = workloads.make_inputs(wl, seed=11)
    yr, fsr = oracle_slice(inp, range(1), range(4))
    errs = {}
    for v in VARIANTS:
        y, fs = _fwd_variant(inp, v)
        errs[v] = (max_rel(y, yr), max_rel(fs, fsr))
        assert np.isfinite(y).all()
    print("deep-decay forward errors (y, final_states):", errs)
    for v in ("hierarchy", "direct"):
        assert max(errs[v]) <= TOL["f32"], f"{v}: {errs[v]}"
    # measured on gfx950: hierarchy and direct 6.3e-8, diff 6.8e-6 on y (the
    # final state does not go through the intra-chunk mask)
    assert errs["diff"][0] > 10 * errs["hierarchy"][0], errs


# --------------------------------------------------------------------------
# The bf16 head kernel at chunk 256 with each evaluation on its output path:
# the hierarchy's rank-one factors, or every C B^T block masked element by
# element (direct running sums, prefix differences).  The states are the
# hierarchy's in all three.

BF16_SHAPES = [
    # (dstate, headdim, headdim_block, split_len)
    (128, 64, 0, 0),       # whole headdim per workgroup, one split
    (64, 128, 64, 256),    # two headdim blocks, a split per chunk (split-local
                           # pass and split scan before the variant's full pass)
    (128, 64, 32, 512),    # blocks of 32, two chunks per split
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("N,P,hb,split", BF16_SHAPES,
                         ids=[f"N{n}_P{p}_pb{b}_split{s}" for n, p, b, s in BF16_SHAPES])
def test_bf16_forward_variants_match_oracle(variant, N, P, hb, split):
    """Document resets inside and across chunks, a ragged tail, two groups and
    an entering state: every element of y and final_states within the bf16
    bound of the fp64 oracle."""
    from ssd_testlib import TOL, max_rel, record_error
    wl = workloads.custom_workload(name=f"bf16_seg_{variant}", batch=2, seqlen=4 * 256 - 29,
                                   nheads=4, headdim=P, dstate=N, ngroups=2, chunk_size=256,
                                   io="bf16", packed=True, doc_range=(20, 400), doc_count=(2, 400))
    inp = workloads.make_inputs(wl, seed=13)
    h0 = np.random.default_rng(14).standard_normal((2, 4, P, N)).astype(np.float32) * 0.5
    y, fs = _fwd_variant(inp, variant, h0, split_len=split, headdim_block=hb)
    yr, fsr = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.seq_idx,
                                 h0.astype(np.float64))
    ey, ef = max_rel(y, yr), max_rel(fs, fsr)
    record_error(f"bf16 {variant} N{N} P{P} pb{hb} split{split}", ey, ef, TOL["bf16"])
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], f"{variant}: y {ey:.2e} fs {ef:.2e}"


@pytest.mark.parametrize("variant", ("direct", "diff"))
def test_bf16_variants_half_headdim_units(variant):
    """288 (batch row, head) units on a 256-CU device: the last round runs as
    half-headdim workgroups, the variant's half-unit kernel among them."""
    from ssd_testlib import TOL, max_rel, record_error
    wl = workloads.custom_workload(name="bf16_seg_half", batch=2, seqlen=600, nheads=144,
                                   headdim=64, dstate=128, ngroups=2, chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=3)
    y, fs = _fwd_variant(inp, variant)
    yr, fsr = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.seq_idx)
    ey, ef = max_rel(y, yr), max_rel(fs, fsr)
    record_error(f"bf16 {variant} half units", ey, ef, TOL["bf16"])
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], f"{variant}: y {ey:.2e} fs {ef:.2e}"


@pytest.mark.parametrize("variant", ("direct", "diff"))
@pytest.mark.parametrize("name", ("layer27b", "decay"))
def test_bf16_variants_full_size(variant, name):
    """The 2.7B-shaped layer and the decay-stress workload at full size, every
    element against the fp64 oracle."""
    from ssd_testlib import TOL, max_rel, record_error
    inp = workloads.make_inputs(workloads.WORKLOADS[name], seed=0)
    y, fs = _fwd_variant(inp, variant)
    yr, fsr = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.seq_idx)
    ey, ef = max_rel(y, yr), max_rel(fs, fsr)
    record_error(f"bf16 {variant} {name}", ey, ef, TOL["bf16"])
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"], f"{variant} {name}: y {ey:.2e} fs {ef:.2e}"


def test_bf16_diff_segsum_cancellation_in_the_forward_pass():
    """One chunk whose first half decays by ~1.4e4 (log2) per token and whose
    second half by 0.14: the prefix sums reach -1.8e6, where an fp32 ulp is
    0.125, comparable with the second half's decays.  Rows of the second half
    (no D term): the direct and hierarchy-aware evaluations stay within the
    bf16 bound, the prefix differences lose several percent."""
    from ssd_testlib import TOL, max_rel
    wl = workloads.custom_workload(name="bf16_cancel", batch=1, seqlen=256, nheads=2, headdim=64,
                                   dstate=64, chunk_size=256, io="bf16")
    inp = workloads.make_inputs(wl, seed=17)
    inp.dt = np.full_like(inp.dt, 1e-5)
    inp.dt[:, :128] = 1.0
    inp.A = np.full_like(inp.A, -1.0e4)
    yr, _ = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, None)
    err = {}
    for v in VARIANTS:
        y, _ = _fwd_variant(inp, v, skip=False)
        err[v] = max_rel(y[:, 128:], yr[:, 128:])
    print("second-half errors:", err)
    assert err["hierarchy"] <= TOL["bf16"] and err["direct"] <= TOL["bf16"], err
    assert err["diff"] > 2 * TOL["bf16"], err


@pytest.mark.parametrize("variant", ("direct", "diff"))
def test_bf16_variants_change_only_the_mask(variant):
    """The mask variants share the hierarchy kernel's state path, so the final
    states are bit-identical to the hierarchy-aware kernel's; y differs only by
    the mask's rounding (a bf16 ulp at most where a rounding flips)."""
    from ssd_testlib import TOL, max_rel
    wl = workloads.custom_workload(name="bf16_seg_state", batch=2, seqlen=3 * 256 + 77, nheads=4,
                                   headdim=64, dstate=128, ngroups=2, chunk_size=256, io="bf16",
                                   packed=True, doc_range=(30, 500), doc_count=(2, 400))
    inp = workloads.make_inputs(wl, seed=23)
    h0 = np.random.default_rng(24).standard_normal((2, 4, 64, 128)).astype(np.float32)
    yh, fh = _fwd_variant(inp, "hierarchy", h0)
    yv, fv = _fwd_variant(inp, variant, h0)
    assert np.array_equal(fh, fv)
    assert max_rel(yv, yh) <= TOL["bf16"]
