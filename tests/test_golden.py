"""The seeded generator and the oracle still reproduce the frozen samples
written by tests/golden/make_golden.py (CPU only)."""
import os

import numpy as np

import oracle
import workloads


def test_tiny_golden_samples():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_seed0.txt")
    inp = workloads.make_inputs(workloads.WORKLOADS["tiny"], seed=0)
    y, fs = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D)
    n = 0
    for line in open(path):
        if line.startswith("#"):
            continue
        parts = line.split()
        if parts[0] == "ymax":
            assert abs(np.abs(y).max() - float(parts[1])) <= 1e-12 * float(parts[1])
            continue
        idx = tuple(int(v) for v in parts[1:5])
        ref = float(parts[5])
        got = (y if parts[0] == "y" else fs)[idx]
        assert abs(got - ref) <= 1e-12 * max(1.0, abs(ref)), (parts, got)
        n += 1
    assert n == 12


def test_generator_shapes_and_ranges():
    # the packed workload draws its document lengths first
    lens = workloads.doc_lengths(np.random.default_rng(0), 32768)
    assert 8 <= len(lens) <= 64 and lens.sum() == 32768 and lens.min() >= 1
    assert lens[:-1].min() >= 64 and lens.max() <= 8192
    inp = workloads.make_inputs(workloads.custom_workload(seqlen=512, packed=True, doc_range=(8, 128), doc_count=(2, 64)), seed=3)
    assert inp.seq_idx.shape == (1, 512) and np.all(np.diff(inp.seq_idx[0]) >= 0)
    small = workloads.make_inputs(workloads.WORKLOADS["decay"], seed=0, seqlen=1024)
    assert small.dt.min() >= 1e-2 * (1 - 1e-6) and small.dt.max() <= 1.0
    assert np.all(-small.A >= 4.0 * (1 - 1e-6)) and np.all(-small.A <= 64.0 * (1 + 1e-6))
    # bf16 rounding: values representable in bf16, round to nearest even
    assert np.array_equal(workloads.bf16_round(small.x), small.x)
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5e-3], dtype=np.float32)
    r = workloads.bf16_round(v)
    assert r[0] == 1.0 and r[1] == 1.0 + 4 * 2 ** -8
    assert abs(r[2] - v[2]) <= 2 ** -9 * abs(v[2])
    wl = workloads.WORKLOADS["layer27b"]
    assert wl.algorithmic_bytes() == 370_147_328 + 2 * 80 * 4
