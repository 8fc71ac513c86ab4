"""Pins of the oracle's backward pass, oracle.ssd_backward (CPU only).

ssd_backward differentiates the fp64 recurrence in reverse (page "State Space
Duality and Mamba-2", "The Mathematical Bridge"; resets as on page "Parallel
Scan and Hardware-Aware SSM Kernels", "When it breaks").  Its gradients are
checked against routes that share none of its code:

  * central finite differences of J = <dy, y> + <dfinal, final_states>
    evaluated by the C forward oracle (oracle.ssd_forward), every element
    of every input, with resets, groups and an initial state;
  * Euler's identity for inputs the outputs are linear in: with a zero
    initial state y and final_states are linear in x, so <dJ/dx, x> = J;
    y - D x and final_states are linear in B, so <dJ/dB, B> = J - <dy, D x>;
    y - D x is linear in C and final_states does not depend on C, so
    <dJ/dC, C> = <dy, y - D x>;
    <dJ/dD, D> = <dy, D x>; with x = 0, J is linear in init_states;
  * planted mistakes in copies of the function (a dropped term, a wrong
    sign, a decay applied on the wrong side of the step, a reset ignored),
    each of which fails a pin.
"""
import inspect

import numpy as np
import pytest

import oracle
import oracle_pins as pins


def _inputs(seed=3, b=2, L=13, H=4, P=3, N=4, G=2, resets=True):
    x, dt, A, B, C, D = pins.small_inputs(seed=seed, b=b, L=L, H=H, P=P, N=N, G=G,
                                          dt_lo=0.05, dt_hi=0.9, a_lo=0.2, a_hi=3.0)
    r = np.random.default_rng(seed + 100)
    dy = r.standard_normal(x.shape)
    dfinal = r.standard_normal((b, H, P, N))
    h0 = r.standard_normal((b, H, P, N))
    seq = None
    if resets:
        seq = np.zeros((b, L), dtype=np.int32)
        seq[0, 5:] = 1
        seq[0, 6:] = 2          # a one-token document
        seq[1, 9:] = 7
    return x, dt, A, B, C, D, dy, dfinal, h0, seq


def _J(x, dt, A, B, C, D, seq, h0, dy, dfinal):
    y, fs = oracle.ssd_forward(x, dt, A, B, C, D, seq, h0)
    return float(np.sum(dy * y) + np.sum(dfinal * fs))


def pin_finite_differences(bwd):
    """Every gradient element against a central difference of J (step 1e-6,
    truncation and rounding error far below the 1e-6 relative bound)."""
    x, dt, A, B, C, D, dy, dfinal, h0, seq = _inputs()
    grads = bwd(x, dt, A, B, C, D, dy, seq, h0, dfinal)
    args = {"x": x, "dt": dt, "A": A, "B": B, "C": C, "D": D, "init": h0}
    names = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "init": "dinit"}
    eps = 1e-6
    worst = 0.0
    for k, arr in args.items():
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            jp = _J(x, dt, A, B, C, D, seq, h0, dy, dfinal)
            arr[idx] = old - eps
            jm = _J(x, dt, A, B, C, D, seq, h0, dy, dfinal)
            arr[idx] = old
            fd[idx] = (jp - jm) / (2 * eps)
        g = grads[names[k]]
        err = float(np.abs(g - fd).max() / max(np.abs(fd).max(), 1e-12))
        worst = max(worst, err)
    return worst < 1e-6, worst


def pin_euler_identities(bwd):
    """Degree-one homogeneity of J in x, B, C, D and init_states."""
    x, dt, A, B, C, D, dy, dfinal, h0, seq = _inputs(seed=5)
    y, fs = oracle.ssd_forward(x, dt, A, B, C, D, seq, None)
    J = float(np.sum(dy * y) + np.sum(dfinal * fs))
    g = bwd(x, dt, A, B, C, D, dy, seq, None, dfinal)
    Dx = D[None, None, :, None] * x
    checks = [
        (float(np.sum(g["dx"] * x)), J),
        (float(np.sum(g["dB"] * B)), J - float(np.sum(dy * Dx))),
        (float(np.sum(g["dC"] * C)), float(np.sum(dy * (y - Dx)))),
        (float(np.sum(g["dD"] * D)), float(np.sum(dy * Dx))),
    ]
    z = np.zeros_like(x)
    y0, fs0 = oracle.ssd_forward(z, dt, A, B, C, D, seq, h0)
    g0 = bwd(z, dt, A, B, C, D, dy, seq, h0, dfinal)
    checks.append((float(np.sum(g0["dinit"] * h0)), float(np.sum(dy * y0) + np.sum(dfinal * fs0))))
    errs = [abs(a - b) / max(abs(b), 1e-12) for a, b in checks]
    return max(errs) < 1e-11, errs


def pin_no_decay_gradient_of_A(bwd):
    """A = 0 and no resets: dJ/dA_h = sum_t dt_t dJ/da_t, and with a = 1 the
    state is the running sum of the inputs, so dJ/da_t = <g_t, h_{t-1}> can be
    formed from prefix sums (page "State Space Duality and Mamba-2", "The
    Duality Revealed": causal linear attention)."""
    x, dt, A, B, C, D, dy, dfinal, h0, _ = _inputs(seed=7, G=1, resets=False)
    A = np.zeros_like(A)
    g = bwd(x, dt, A, B, C, D, dy, None, None, dfinal)
    Bg, Cg = B[:, :, 0, :], C[:, :, 0, :]
    outer = np.einsum("blh,blhp,bln->blhpn", dt, x, Bg)
    hs = np.cumsum(outer, axis=1)                                     # h_t
    # g_t = dfinal + sum_{s >= t} dy_s C_s^T (no decay)
    dyc = np.einsum("blhp,bln->blhpn", dy, Cg)
    gs = np.cumsum(dyc[:, ::-1], axis=1)[:, ::-1] + dfinal[:, None]
    hprev = np.concatenate([np.zeros_like(hs[:, :1]), hs[:, :-1]], axis=1)
    da = np.einsum("blhpn,blhpn->blh", gs, hprev)
    dA_ref = np.einsum("blh,blh->h", da, dt)
    err = float(np.abs(g["dA"] - dA_ref).max() / np.abs(dA_ref).max())
    return err < 1e-11, err


BACKWARD_PINS = [pin_finite_differences, pin_euler_identities, pin_no_decay_gradient_of_A]


@pytest.mark.parametrize("pin", BACKWARD_PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    ok, info = pin(oracle.ssd_backward)
    assert ok, f"{pin.__name__}: {info}"


# ----------------------------------------------------- planted mistakes

MUTATIONS = {
    "decay_term_dropped": ("ddt[:, t] += ga * A[None, :]", "ddt[:, t] += 0.0 * ga"),
    "decay_term_sign": ("ddt[:, t] += ga * A[None, :]", "ddt[:, t] -= ga * A[None, :]"),
    "dA_without_dt": ("dA += (ga * dt[:, t]).sum(axis=0)", "dA += ga.sum(axis=0)"),
    "propagate_before_step": ("hprev = hs[:, t - 1] if t > 0 else h0",
                              "hprev = hs[:, t]"),
    "reset_ignored": ("a = np.where(reset[:, :, None], 0.0, a)", "a = a"),
    "dB_missing_dt": ("dBh[:, t] = dt[:, t, :, None] * np.einsum(", "dBh[:, t] = 1.0 * np.einsum("),
    "dC_from_next_state": ('dCh[:, t] = np.einsum("bhpn,bhp->bhn", hs[:, t], dy[:, t])',
                           'dCh[:, t] = np.einsum("bhpn,bhp->bhn", hs[:, max(t - 1, 0)], dy[:, t])'),
    "skip_gradient_dropped": ("dx += D[None, None, :, None] * dy", "dx += 0.0 * dy"),
}


def _mutant(name):
    src = inspect.getsource(oracle.ssd_backward)
    old, new = MUTATIONS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    ns = {"np": np}
    exec(src.replace(old, new), ns)
    return ns["ssd_backward"]


def test_unmutated_copy_is_the_oracle():
    src = inspect.getsource(oracle.ssd_backward)
    ns = {"np": np}
    exec(src, ns)
    x, dt, A, B, C, D, dy, dfinal, h0, seq = _inputs(seed=9)
    g1 = ns["ssd_backward"](x, dt, A, B, C, D, dy, seq, h0, dfinal)
    g2 = oracle.ssd_backward(x, dt, A, B, C, D, dy, seq, h0, dfinal)
    for k in g1:
        assert (g1[k] is None and g2[k] is None) or np.array_equal(g1[k], g2[k])


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_pins_catch_planted_mistake(name):
    bwd = _mutant(name)
    failed = [p.__name__ for p in BACKWARD_PINS if not p(bwd)[0]]
    assert failed, f"planted mistake {name} passed every backward pin"
