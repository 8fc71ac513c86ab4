"""The fp64 oracle pinned to facts other than itself (CPU only).

The pins live in oracle_pins.py.  Each also runs against copies of the C
oracle with a planted mistake (a dropped term, a wrong sign, a transposed
operand, an index off by one ...), compiled on the CPU, to show that every
such mistake fails at least one pin.
"""
import ctypes
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import oracle_pins as pins


def fwd_real(x, dt, A, B, C, D, seq_idx, init_states):
    return oracle.ssd_forward(x, dt, A, B, C, D, seq_idx, init_states)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    ok, info = pin(fwd_real)
    assert ok, f"{pin.__name__}: {info}"


# --------------------------------------------------------- decay-mask pins

def _segsum_mask(dt, A, seq_idx, Q, c):
    """exp of fp64 segment sums from cumulative sums (a different route
    from the oracle's running product) for chunk c."""
    b, L, H = dt.shape
    t0 = c * Q
    n = min(Q, L - t0)
    out = np.zeros((b, H, Q, Q))
    for bi in range(b):
        for h in range(H):
            ld = dt[bi, t0:t0 + n, h] * A[h]
            cs = np.cumsum(ld)
            seg = cs[:, None] - cs[None, :]
            m = np.tril(np.exp(np.minimum(seg, 0)))
            if seq_idx is not None:
                s = seq_idx[bi, t0:t0 + n]
                doc = np.concatenate([[0], np.cumsum(s[1:] != s[:-1])])
                m = m * (doc[:, None] == doc[None, :])
            out[bi, h, :n, :n] = m
    return out


def test_mask_matches_segment_sums():
    x, dt, A, B, C, D = pins.small_inputs(seed=5, b=2, L=70, H=3)
    seq_idx = np.zeros((2, 70), dtype=np.int32)
    seq_idx[0, 13:] = 1
    seq_idx[0, 40:] = 2
    seq_idx[1, 33:] = 4
    Q = 16
    m = oracle.decay_mask(dt, A, seq_idx, chunk_size=Q)
    assert m.shape == (2, 3, 5, Q, Q)
    for c in range(5):
        ref = _segsum_mask(dt, A, seq_idx, Q, c)
        assert np.abs(m[:, :, c] - ref).max() < 1e-12


def test_mask_special_cases():
    b, L, H, Q = 1, 40, 2, 8
    dt = np.full((b, L, H), 0.25)
    A = np.array([0.0, -2.0])
    m = oracle.decay_mask(dt, A, chunk_size=Q)
    i, j = np.meshgrid(np.arange(Q), np.arange(Q), indexing="ij")
    # a = 1: causal all-ones lower triangle, exactly
    assert np.array_equal(m[0, 0], np.broadcast_to(np.tril(np.ones((Q, Q))), (5, Q, Q)))
    # constant decay: L_ij = exp(dt A (i - j))
    ref = np.where(i >= j, np.exp(0.25 * -2.0 * (i - j)), 0.0)
    assert np.abs(m[0, 1] - ref).max() < 1e-14
    # ragged tail: the last chunk holds L - 4*Q = 8 tokens, rest zero
    m2 = oracle.decay_mask(dt[:, :35], A, chunk_size=Q)
    assert m2.shape[2] == 5 and np.all(m2[0, :, 4, 3:, :] == 0) and np.all(m2[0, :, 4, :, 3:] == 0)


def test_mask_invariants_fp64():
    x, dt, A, B, C, D = pins.small_inputs(seed=6, b=1, L=64, H=2, dt_lo=1e-3, dt_hi=1.0,
                                           a_lo=1.0, a_hi=64.0)
    m = oracle.decay_mask(dt, A, chunk_size=64)[0, :, 0]
    assert np.all(m >= 0) and np.all(m <= 1)
    assert np.all(np.diagonal(m, axis1=-2, axis2=-1) == 1)
    # non-increasing along each row away from the diagonal
    for h in range(2):
        for i in range(64):
            row = m[h, i, :i + 1]
            assert np.all(np.diff(row) >= 0)
    # semiseparable product rule L_ik = L_ij L_jk for i >= j >= k
    for h in range(2):
        for (i, j, k) in [(63, 40, 3), (20, 20, 5), (50, 10, 10), (33, 32, 31)]:
            assert abs(m[h, i, k] - m[h, i, j] * m[h, j, k]) <= 1e-14 * max(1.0, m[h, i, k])


def test_oracle_threads_and_errors():
    assert oracle.max_threads() >= 1
    x, dt, A, B, C, D = pins.small_inputs(seed=7)
    with pytest.raises(ValueError):
        oracle.ssd_forward(x, dt[:, :-1], A, B, C, D)


# --------------------------------------------------------- planted mistakes

MUTATIONS = {
    "drop_dt_in_input": ("const double ux = dtv * xt[p];", "const double ux = xt[p];"),
    "decay_sign": ("exp(dtv * Ah)", "exp(-dtv * Ah)"),
    "decay_without_dt": ("exp(dtv * Ah)", "exp(Ah)"),
    "skip_uses_dt_x": ("yt[p] = acc + Dh * xt[p];", "yt[p] = acc + Dh * ux;"),
    "skip_dropped": ("yt[p] = acc + Dh * xt[p];", "yt[p] = acc;"),
    "swap_B_C": ("Sp[n] = a * Sp[n] + ux * Bt[n];\n                    acc += Ct[n] * Sp[n];",
                 "Sp[n] = a * Sp[n] + ux * Ct[n];\n                    acc += Bt[n] * Sp[n];"),
    "output_before_update": ("Sp[n] = a * Sp[n] + ux * Bt[n];\n                    acc += Ct[n] * Sp[n];",
                             "acc += Ct[n] * Sp[n];\n                    Sp[n] = a * Sp[n] + ux * Bt[n];"),
    "decay_on_input_too": ("Sp[n] = a * Sp[n] + ux * Bt[n];", "Sp[n] = a * (Sp[n] + ux * Bt[n]);"),
    "group_map_modulo": ("const int64_t g = h / heads_per_group;", "const int64_t g = h % G;"),
    "no_reset": ("memset(S, 0, (size_t)(P * N) * sizeof(double));\n            const double dtv",
                 "(void)0;\n            const double dtv"),
    "reset_one_late": ("seq_idx[b * seqlen + t] != seq_idx[b * seqlen + t - 1])",
                       "t > 1 && seq_idx[b * seqlen + t - 1] != seq_idx[b * seqlen + t - 2])"),
    "init_state_ignored": ("if (init_states)\n            memcpy", "if (0)\n            memcpy"),
    "state_transposed_read": ("const double *xt = x + ((b * seqlen + t) * H + h) * P;",
                              "const double *xt = x + ((b * seqlen + t) * H + (H - 1 - h)) * P;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return tmp_path_factory.mktemp("mutants")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, mutant_dir):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")).read()
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    path_c = os.path.join(mutant_dir, f"{name}.c")
    path_so = os.path.join(mutant_dir, f"{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", path_so,
                    path_c, "-lm"], check=True)
    lib = oracle.bind(ctypes.CDLL(path_so))

    def fwd(x, dt, A, B, C, D, seq_idx, init_states):
        return oracle.ssd_forward(x, dt, A, B, C, D, seq_idx, init_states, lib=lib)

    failed = [p.__name__ for p in pins.ALL_PINS if not p(fwd)[0]]
    assert failed, f"planted mistake {name} passed every pin"


def test_mask_invariant_checker_accepts_oracle_and_rejects_violations():
    """The invariant checker used on the GPU mask accepts the fp64 oracle's
    mask and rejects planted violations."""
    from mask_invariants import check_mask_invariants
    x, dt, A, B, C, D = pins.small_inputs(seed=8, b=1, L=96, H=2, dt_lo=1e-3, dt_hi=1.0)
    m = oracle.decay_mask(dt, A, chunk_size=32)
    check_mask_invariants(m)
    bad = m.copy()
    bad[0, 0, 1, 20, 5] = min(1.0, bad[0, 0, 1, 20, 6] * 1.5 + 1e-3)   # increases leftwards
    with pytest.raises(AssertionError):
        check_mask_invariants(bad)
    bad = m.copy()
    bad[0, 1, 0, 3, 4] = 0.5                                            # above the diagonal
    with pytest.raises(AssertionError):
        check_mask_invariants(bad)
