"""Pins of the oracle's fused prologue and epilogue (CPU only).

oracle.dt_prologue, oracle.gate and oracle.ssd_forward_fused add to the scan
the element-wise work around it (page "NVIDIA Accelerates Mamba-2 Forward
Kernel with CUDA Tile": element-wise gating in "What CUDA Tile Is and Why It
Suits Writing Mamba-2 Kernels"; fusion of the gating that follows the scan
in "From Python DSL to Production-Grade Kernels").  Readings: dt =
softplus(raw + bias) clamped to [lo, hi]; out = (y + D x) * silu(z).

Every expected value comes from a route other than the oracle's own code:
closed forms of softplus and silu at special points, numpy's logaddexp and
scipy's expit, and the dense quadratic form of the scan (oracle_pins).
Each pin also runs against copies of the oracle functions with a planted
mistake, and every such mistake fails at least one pin.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle
import oracle_pins as pins

RTOL = 1e-12


# ------------------------------------------------------------ the pins
# Each pin takes (softplus, gate, fused) under test and returns (ok, info).

def pin_softplus_closed_forms(sp, gate, fused):
    """softplus(0) = ln 2; softplus(ln(e - 1)) = 1; softplus(v) - softplus(-v)
    = v for every v; softplus(v) ~ e^v for v -> -inf (first-order term of
    log1p) and ~ v for v -> +inf; against numpy's logaddexp(0, v) on a grid."""
    v = np.linspace(-60.0, 60.0, 2401)
    got = sp(v)
    errs = [abs(sp(np.array([0.0]))[0] - math.log(2.0)) / math.log(2.0),
            abs(sp(np.array([math.log(math.e - 1.0)]))[0] - 1.0),
            float(np.max(np.abs((got - sp(-v)) - v) / np.maximum(1.0, np.abs(v)))),
            float(np.max(np.abs(got - np.logaddexp(0.0, v)) / np.logaddexp(0.0, v)))]
    tiny = np.array([-700.0, -40.0])
    errs.append(float(np.max(np.abs(sp(tiny) - np.exp(tiny)) / np.exp(tiny))))
    errs.append(abs(sp(np.array([700.0]))[0] - 700.0) / 700.0)
    return max(errs) < RTOL and bool(np.all(np.isfinite(got))), errs


def pin_gate_closed_forms(sp, gate, fused):
    """silu(0) = 0; sigma(ln 3) = 3/4 and sigma(-ln 3) = 1/4, so
    gate(y, +-ln 3) = +-y ln 3 (3/4 or 1/4); gate(y, z) -> y z for large z and
    -> 0 without NaN for very negative z; against y z expit(z) on a grid."""
    y = np.array([1.7, -0.3, 2.0])
    l3 = math.log(3.0)
    errs = [float(np.max(np.abs(gate(y, np.zeros(3))))),
            float(np.max(np.abs(gate(y, np.full(3, l3)) - y * l3 * 0.75))),
            float(np.max(np.abs(gate(y, np.full(3, -l3)) + y * l3 * 0.25)))]
    big = gate(y, np.full(3, 60.0))
    errs.append(float(np.max(np.abs(big - 60.0 * y) / np.abs(60.0 * y))))
    neg = gate(y, np.full(3, -1000.0))
    errs.append(0.0 if np.all(np.isfinite(neg)) and np.all(np.abs(neg) < 1e-300) else 1.0)
    r = np.random.default_rng(3)
    yy = r.standard_normal(500)
    zz = 8.0 * r.standard_normal(500)
    ref = yy * zz * expit(zz)
    errs.append(float(np.max(np.abs(gate(yy, zz) - ref)) / np.max(np.abs(ref))))
    return max(errs) < RTOL, errs


def _fused_inputs(seed):
    x, dt, A, B, C, D = pins.small_inputs(seed=seed, b=2, L=29, H=4, P=3, N=5, G=2)
    r = np.random.default_rng(seed + 1)
    raw = r.standard_normal(dt.shape) - 2.0          # pre-softplus values
    bias = r.uniform(-1.0, 1.0, size=(dt.shape[2],))
    z = 2.0 * r.standard_normal(x.shape)
    return x, raw, bias, A, B, C, D, z


def pin_fused_dense_form(sp, gate, fused):
    """The fused forward against the dense quadratic form of the scan
    (oracle_pins.dense_quadratic_form, page "State Space Duality and
    Mamba-2", "The Mathematical Bridge") applied to dt = logaddexp(0, raw +
    bias) clipped to [lo, hi], with the gate y z expit(z) on the output that
    already holds D x; with resets and an initial state."""
    x, raw, bias, A, B, C, D, z = _fused_inputs(seed=91)
    b, L = x.shape[:2]
    seq_idx = np.zeros((b, L), dtype=np.int32)
    seq_idx[0, 11:] = 1
    seq_idx[1, 4:] = 3
    h0 = np.random.default_rng(92).standard_normal((b, x.shape[2], x.shape[3], B.shape[3]))
    lo, hi = 0.05, 0.6
    dt = np.clip(np.logaddexp(0.0, raw + bias[None, None, :]), lo, hi)
    assert (dt == lo).any() and (dt == hi).any(), "the clamp must bind somewhere"
    yr, fsr = pins.dense_quadratic_form(x, dt, A, B, C, D, seq_idx, h0)
    out_ref = yr * z * expit(z)
    out, fs = fused(x, raw, A, B, C, D, seq_idx, h0, dt_bias=bias, dt_softplus=True,
                    dt_limit=(lo, hi), z=z)
    errs = [pins.rel_err(out, out_ref), pins.rel_err(fs, fsr)]
    # no gate, no clamp: the plain scan on softplus(raw + bias)
    dt2 = np.logaddexp(0.0, raw + bias[None, None, :])
    yr2, fsr2 = pins.dense_quadratic_form(x, dt2, A, B, C, D)
    out2, fs2 = fused(x, raw, A, B, C, D, None, None, dt_bias=bias, dt_softplus=True)
    errs += [pins.rel_err(out2, yr2), pins.rel_err(fs2, fsr2)]
    # no prologue at all: raw values are the step sizes
    dt3 = np.exp(raw)
    yr3, _ = pins.dense_quadratic_form(x, dt3, A, B, C, D)
    out3, _ = fused(x, dt3, A, B, C, D, None, None, z=z)
    errs.append(pins.rel_err(out3, yr3 * z * expit(z)))
    return max(errs) < 1e-10, errs


def pin_gate_leaves_state(sp, gate, fused):
    """The gate touches only the output: final_states with and without z are
    identical, and z = 0 gives an exactly zero output."""
    x, raw, bias, A, B, C, D, z = _fused_inputs(seed=95)
    _, f1 = fused(x, raw, A, B, C, D, None, None, dt_bias=bias, dt_softplus=True, z=z)
    _, f2 = fused(x, raw, A, B, C, D, None, None, dt_bias=bias, dt_softplus=True)
    o0, _ = fused(x, raw, A, B, C, D, None, None, dt_bias=bias, dt_softplus=True,
                  z=np.zeros_like(z))
    return bool(np.array_equal(f1, f2)) and bool(np.all(o0 == 0)), []


FUSED_PINS = [pin_softplus_closed_forms, pin_gate_closed_forms, pin_fused_dense_form,
              pin_gate_leaves_state]


def real_fused(x, dt_raw, A, B, C, D, seq_idx, init_states, **kw):
    return oracle.ssd_forward_fused(x, dt_raw, A, B, C, D, seq_idx, init_states, **kw)


@pytest.mark.parametrize("pin", FUSED_PINS, ids=lambda p: p.__name__)
def test_fused_pin(pin):
    ok, info = pin(oracle.softplus, oracle.gate, real_fused)
    assert ok, f"{pin.__name__}: {info}"


# ----------------------------------------------------- planted mistakes

def _mut_softplus_no_log1p(v):          # log(1 + e^v) with e^v alone
    return np.exp(np.asarray(v, dtype=np.float64))


def _mut_softplus_relu(v):              # the v > 0 branch without its correction
    v = np.asarray(v, dtype=np.float64)
    return np.where(v > 0, v, np.log1p(np.exp(v)))


def _mut_gate_sign(y, z):                # sigma(-z) instead of sigma(z)
    z = np.asarray(z, dtype=np.float64)
    return np.asarray(y) * z * expit(-z)


def _mut_gate_no_z(y, z):                # y sigma(z): a sigmoid gate, not silu
    return np.asarray(y) * expit(np.asarray(z, dtype=np.float64))


def _fused_with(sp=None, gate=None, order=None):
    """oracle.ssd_forward_fused rebuilt from its parts, with one part or the
    order of the steps replaced."""
    sp = sp or oracle.softplus
    gate = gate or oracle.gate

    def fused(x, dt_raw, A, B, C, D, seq_idx, init_states, dt_bias=None, dt_softplus=False,
              dt_limit=None, z=None):
        dt = np.asarray(dt_raw, dtype=np.float64).copy()
        if order == "bias_after_softplus":
            if dt_softplus:
                dt = sp(dt)
            if dt_bias is not None:
                dt = dt + dt_bias[None, None, :]
        else:
            if dt_bias is not None:
                dt = dt + dt_bias[None, None, :]
            if dt_softplus and order != "clamp_before_softplus":
                dt = sp(dt)
        if dt_limit is not None:
            dt = np.clip(dt, dt_limit[0], dt_limit[1])
        if dt_softplus and order == "clamp_before_softplus":
            dt = sp(dt)
        if order == "gate_before_skip" and z is not None:
            y, fs = oracle.ssd_forward(x, dt, A, B, C, None, seq_idx, init_states)
            y = gate(y, z) + (0.0 if D is None else D[None, None, :, None] * x)
            return y, fs
        y, fs = oracle.ssd_forward(x, dt, A, B, C, D, seq_idx, init_states)
        if z is not None:
            y = gate(y, z)
        return y, fs

    return sp, gate, fused


MUTANTS = {
    "softplus_no_log1p": lambda: _fused_with(sp=_mut_softplus_no_log1p),
    "softplus_relu": lambda: _fused_with(sp=_mut_softplus_relu),
    "gate_sign": lambda: _fused_with(gate=_mut_gate_sign),
    "gate_sigmoid_only": lambda: _fused_with(gate=_mut_gate_no_z),
    "bias_after_softplus": lambda: _fused_with(order="bias_after_softplus"),
    "clamp_before_softplus": lambda: _fused_with(order="clamp_before_softplus"),
    "gate_before_skip": lambda: _fused_with(order="gate_before_skip"),
}


def test_rebuilt_fused_matches_oracle():
    """The rebuild used for the mutants is the oracle itself when nothing is
    replaced (so a mutant differs only by its planted mistake)."""
    sp, gate, fused = _fused_with()
    x, raw, bias, A, B, C, D, z = _fused_inputs(seed=97)
    kw = dict(dt_bias=bias, dt_softplus=True, dt_limit=(0.05, 0.6), z=z)
    o1, f1 = fused(x, raw, A, B, C, D, None, None, **kw)
    o2, f2 = real_fused(x, raw, A, B, C, D, None, None, **kw)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fused_pins_catch_planted_mistake(name):
    sp, gate, fused = MUTANTS[name]()
    failed = [p.__name__ for p in FUSED_PINS if not p(sp, gate, fused)[0]]
    assert failed, f"planted mistake {name} passed every fused pin"
