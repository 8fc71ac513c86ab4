"""Properties of the HIP path that hold at any size (needs an MI355X):
chunk-size and split-length invariance, composition of two calls through the
carried state, bitwise determinism, zero leakage across documents (bit for
bit), batch-row independence and the trivial-input identities."""
import numpy as np
import pytest

import workloads
from ssd_testlib import TOL, max_rel, oracle_slice, run_gpu, to_device

pytestmark = pytest.mark.gpu


def _wl(**kw):
    base = dict(batch=2, seqlen=1100, nheads=4, headdim=64, dstate=64, ngroups=2,
                chunk_size=128, io="bf16")
    base.update(kw)
    return workloads.custom_workload(**base)


def test_chunk_size_invariance():
    outs = {}
    for Q in (64, 128, 256):
        inp = workloads.make_inputs(_wl(chunk_size=Q), seed=11)
        outs[Q] = run_gpu(inp)
    for Q in (64, 128):
        assert max_rel(outs[Q][0], outs[256][0]) <= TOL["bf16"]
        assert max_rel(outs[Q][1], outs[256][1]) <= TOL["bf16"]


def test_split_length_invariance():
    inp = workloads.make_inputs(_wl(), seed=12)
    y0, f0 = run_gpu(inp, split_len=0)
    for sl in (128, 256, 640):
        y, f = run_gpu(inp, split_len=sl)
        assert max_rel(y, y0) <= TOL["bf16"] and max_rel(f, f0) <= TOL["bf16"]


def test_two_calls_compose_through_state():
    """[0, T/2) then [T/2, T) from the carried state equals one call (page
    "Parallel Scan and Hardware-Aware SSM Kernels", "The scan": affine
    composition)."""
    import dataclasses
    inp = workloads.make_inputs(_wl(seqlen=1024), seed=13)
    y, f = run_gpu(inp)
    half = 512
    first = dataclasses.replace(inp, wl=dataclasses.replace(inp.wl, seqlen=half),
                                x=inp.x[:, :half], dt=inp.dt[:, :half], B=inp.B[:, :half],
                                C=inp.C[:, :half])
    second = dataclasses.replace(inp, wl=dataclasses.replace(inp.wl, seqlen=half),
                                 x=inp.x[:, half:], dt=inp.dt[:, half:], B=inp.B[:, half:],
                                 C=inp.C[:, half:])
    y1, f1 = run_gpu(first)
    y2, f2 = run_gpu(second, init_states=f1.astype(np.float32))
    assert max_rel(np.concatenate([y1, y2], axis=1), y) <= TOL["bf16"]
    assert max_rel(f2, f) <= TOL["bf16"]


def test_bitwise_determinism():
    inp = workloads.make_inputs(_wl(), seed=14)
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_zero_leakage_bitwise():
    """Perturbing one document changes no bit of any other document's output
    (page "Parallel Scan and Hardware-Aware SSM Kernels", "When it breaks")."""
    wl = _wl(batch=1, seqlen=2000, packed=True, doc_range=(50, 600), doc_count=(3, 64))
    inp = workloads.make_inputs(wl, seed=15)
    y0, _ = run_gpu(inp)
    lens = inp.doc_lens
    starts = np.concatenate([[0], np.cumsum(lens)])
    d = len(lens) // 2
    s0, s1 = starts[d], starts[d + 1]
    inp.x[:, s0:s1] = workloads.bf16_round(inp.x[:, s0:s1] * 3.0 + 1.0)
    inp.B[:, s0:s1] = workloads.bf16_round(-inp.B[:, s0:s1])
    y1, _ = run_gpu(inp)
    other = np.ones(y0.shape[1], dtype=bool)
    other[s0:s1] = False
    assert np.array_equal(y0[:, other], y1[:, other])
    assert not np.array_equal(y0[:, s0:s1], y1[:, s0:s1])


def test_batch_rows_independent():
    inp = workloads.make_inputs(_wl(batch=3), seed=16)
    y, f = run_gpu(inp)
    inp.x[1] = workloads.bf16_round(inp.x[1] * -2.0)
    y2, f2 = run_gpu(inp)
    assert np.array_equal(y[0], y2[0]) and np.array_equal(y[2], y2[2])
    assert np.array_equal(f[0], f2[0]) and np.array_equal(f[2], f2[2])


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_zero_B_gives_skip_only(io):
    """B = 0 leaves only the skip term D x (and a zero state).  The fp32 path
    forms D x in fp32; the bf16 path carries D on the diagonal of the bf16
    intra-chunk matrix, so its skip is x times D rounded to bf16, exactly
    (one product of two bf16 values is exact in fp32), then rounded to bf16."""
    inp = workloads.make_inputs(_wl(io=io), seed=17)
    inp.B[:] = 0.0
    y, f = run_gpu(inp)
    D = inp.D if io == "f32" else workloads.bf16_round(inp.D)
    ref = (D[None, None, :, None] * inp.x).astype(np.float32)   # fp32 product
    if io == "bf16":
        ref = workloads.bf16_round(ref)
    assert np.array_equal(y, ref.astype(np.float64))
    # and within the parity bound of the exact skip term
    exact = inp.D[None, None, :, None].astype(np.float64) * inp.x
    assert max_rel(y, exact) <= TOL[io]
    assert np.all(f == 0)


def test_reset_every_token():
    """A document boundary at every token leaves only the diagonal of M."""
    inp = workloads.make_inputs(_wl(batch=1, seqlen=300), seed=18)
    inp = type(inp)(**{**inp.__dict__})
    inp.seq_idx = np.arange(300, dtype=np.int32)[None, :]
    y, f = run_gpu(inp)
    yr, fr = oracle_slice(inp, [0], range(4))
    assert max_rel(y, yr) <= TOL["bf16"] and max_rel(f, fr) <= TOL["bf16"]


def test_reuse_group_operands_is_bitwise_identical():
    """A call told that the workspace already holds the per-group operands
    (C B^T blocks, token-transposed B) of these B and C gives exactly the
    result of the full call that wrote them."""
    import ssd_chunked_scan_amd as ssd
    import torch
    inp = workloads.make_inputs(_wl(), seed=19)
    t = to_device(inp)
    wl = inp.wl
    shape = ssd.Shape(wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups)
    ws = torch.empty(ssd.ssd_fwd_workspace_bytes(shape, wl.chunk_size, 1), dtype=torch.uint8,
                     device="cuda")
    y0, f0 = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["seq_idx"],
                         chunk_size=wl.chunk_size, workspace=ws)
    y1, f1 = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["seq_idx"],
                         chunk_size=wl.chunk_size, workspace=ws, reuse_group_operands=True)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)


@pytest.mark.parametrize("Q", [128, 256])
def test_headdim_block_invariance(Q):
    """Every headdim block size (whole head, halves, quarters) gives the same
    outputs and final state bit for bit: each output element and state
    element goes through the same sequence of operations whichever
    workgroup owns its column; and against the oracle, with and without
    sequence splits."""
    wl = _wl(headdim=128, seqlen=1000, chunk_size=Q)
    inp = workloads.make_inputs(wl, seed=19)
    whole = -(-1000 // Q) * Q     # one split per row (the planner would split this row)
    y0, f0 = run_gpu(inp, headdim_block=16, split_len=whole)
    for hb in (32, 64, 128):
        if Q == 256 and hb == 128:
            continue   # the 256 x 128 tiles do not fit the LDS (SSD_ERR_UNSUPPORTED)
        y, f = run_gpu(inp, headdim_block=hb, split_len=whole)
        assert np.array_equal(y, y0) and np.array_equal(f, f0), f"headdim_block {hb}"
        ys, fs = run_gpu(inp, headdim_block=hb, split_len=2 * Q)
        assert max_rel(ys, y0) <= TOL["bf16"] and max_rel(fs, f0) <= TOL["bf16"]
    yr, fr = oracle_slice(inp, range(2), range(4))
    assert max_rel(y0, yr) <= TOL["bf16"] and max_rel(f0, fr) <= TOL["bf16"]


@pytest.mark.parametrize("split_len", [0, 128], ids=["one_split", "forced_splits"])
def test_workspace_poison_does_not_change_outputs(split_len):
    """Every workspace byte a kernel reads is written earlier in the same call:
    a workspace filled with 0xff bytes (NaN as fp32 and as bf16) gives the
    same bits as a zeroed one, with and without sequence splits (split states,
    per-group C B^T, B^T and C operands)."""
    import torch
    import ssd_chunked_scan_amd as ssd
    inp = workloads.make_inputs(_wl(), seed=16)
    t = to_device(inp)
    h0 = torch.from_numpy(np.random.default_rng(17).standard_normal((2, 4, 64, 64)).astype(np.float32)).cuda()
    shape = ssd.Shape(2, 1100, 4, 64, 64, 2)
    nbytes = ssd.ssd_fwd_workspace_bytes(shape, 128, 1, split_len=split_len)
    assert nbytes > 0
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        y, f = ssd.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], None, chunk_size=128,
                           init_states=h0, split_len=split_len, workspace=ws)
        torch.cuda.synchronize()
        outs.append((y.clone(), f.clone()))
    assert torch.isfinite(outs[0][0].float()).all()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
