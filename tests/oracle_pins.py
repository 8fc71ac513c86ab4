"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Each pin takes the forward function under test, ``fwd(x, dt, A, B, C, D,
seq_idx, init_states) -> (y, final_states)``, so the same checks run on the
real oracle and on copies with a planted mistake (tests/test_oracle.py).  Every
expected value here is computed by a route other than the sequential
recurrence: the quadratic (attention) form, prefix sums, a geometric series,
or structural identities.
"""
from __future__ import annotations

import math

import numpy as np

RTOL_EXACT = 1e-11


def _rng(seed):
    return np.random.default_rng(seed)


def small_inputs(seed=1, b=2, L=37, H=4, P=3, N=5, G=2, dt_lo=0.05, dt_hi=0.9,
                 a_lo=0.2, a_hi=3.0):
    r = _rng(seed)
    x = r.standard_normal((b, L, H, P))
    dt = np.exp(r.uniform(math.log(dt_lo), math.log(dt_hi), size=(b, L, H)))
    A = -np.exp(r.uniform(math.log(a_lo), math.log(a_hi), size=(H,)))
    B = r.standard_normal((b, L, G, N)) / math.sqrt(N)
    C = r.standard_normal((b, L, G, N)) / math.sqrt(N)
    D = r.standard_normal((H,))
    return x, dt, A, B, C, D


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = max(np.abs(b).max(), 1e-300)
    return float(np.abs(a - b).max() / den)


def dense_quadratic_form(x, dt, A, B, C, D, seq_idx=None, init_states=None):
    """The quadratic (attention) form Y = ((C B^T) o L) (dt x) + D x, page
    "State Space Duality and Mamba-2", section "The Mathematical Bridge"
    (M = (C B^T) o L with L_ij = prod_{k=j+1..i} a_k), evaluated densely
    over the whole sequence.  The mask is exp of a segment sum of log-decays
    taken from fp64 cumulative sums, and a document boundary between j and i
    zeroes the entry.  The carried-in state decays by prod_{k=0..i} a_k and
    only reaches the first document."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros((b, L, H, P))
    fs = np.zeros((b, H, P, N))
    ii, jj = np.meshgrid(np.arange(L), np.arange(L), indexing="ij")
    for bi in range(b):
        if seq_idx is None:
            doc = np.zeros(L, dtype=np.int64)
        else:
            # document number = count of boundaries so far (works for any ids)
            s = np.asarray(seq_idx[bi])
            doc = np.concatenate([[0], np.cumsum(s[1:] != s[:-1])])
        same = doc[:, None] == doc[None, :]
        for h in range(H):
            g = h // hpg
            logd = dt[bi, :, h] * A[h]
            cs = np.concatenate([[0.0], np.cumsum(logd)])    # cs[t+1] = sum_{k<=t}
            seg = cs[1:][:, None] - cs[1:][None, :]          # sum_{k=j+1..i}
            Lm = np.where((ii >= jj) & same, np.exp(np.minimum(seg, 0.0)), 0.0)
            CB = C[bi, :, g, :] @ B[bi, :, g, :].T            # [i, j] = C_i . B_j
            M = CB * Lm * dt[bi, :, h][None, :]
            y[bi, :, h, :] = M @ x[bi, :, h, :] + D[h] * x[bi, :, h, :]
            # final state: sum_j L_{T-1, j} dt_j x_j B_j^T (+ decayed h0)
            w = Lm[L - 1, :] * dt[bi, :, h]
            fs[bi, h] = (x[bi, :, h, :] * w[:, None]).T @ B[bi, :, g, :]
            if init_states is not None:
                first = doc == 0
                dec0 = np.exp(cs[1:])                          # prod_{k=0..i} a_k
                h0 = init_states[bi, h]                        # [P, N]
                contrib = (C[bi, :, g, :] @ h0.T) * dec0[:, None]   # [L, P]
                y[bi, :, h, :] += np.where(first[:, None], contrib, 0.0)
                if first[L - 1]:
                    fs[bi, h] += dec0[L - 1] * h0
    return y, fs


# ---------------------------------------------------------------- the pins

def pin_dense_form(fwd):
    """P-1: recurrence == quadratic form (with groups, resets, init state)."""
    errs = []
    x, dt, A, B, C, D = small_inputs(seed=11)
    y, fs = fwd(x, dt, A, B, C, D, None, None)
    yr, fsr = dense_quadratic_form(x, dt, A, B, C, D)
    errs += [rel_err(y, yr), rel_err(fs, fsr)]
    # with document resets and an initial state
    b, L = x.shape[:2]
    seq_idx = np.zeros((b, L), dtype=np.int32)
    seq_idx[0, 9:] = 1
    seq_idx[0, 20:] = 2
    seq_idx[1, 1:] = 5
    seq_idx[1, 30:] = 6
    h0 = _rng(12).standard_normal((b, x.shape[2], x.shape[3], B.shape[3]))
    y, fs = fwd(x, dt, A, B, C, D, seq_idx, h0)
    yr, fsr = dense_quadratic_form(x, dt, A, B, C, D, seq_idx, h0)
    errs += [rel_err(y, yr), rel_err(fs, fsr)]
    return max(errs) < RTOL_EXACT, errs


def pin_linear_attention(fwd):
    """P-2: a_k = 1 (A = 0) gives unnormalised causal linear attention,
    y_i = sum_{j<=i} (C_i . B_j) dt_j x_j + D x_i, page "State Space Duality
    and Mamba-2", section "The Duality Revealed"; evaluated with prefix sums
    of the outer products dt_j x_j B_j^T."""
    x, dt, A, B, C, D = small_inputs(seed=21, G=1)
    A = np.zeros_like(A)
    y, fs = fwd(x, dt, A, B, C, D, None, None)
    outer = np.einsum("blh,blhp,bln->blhpn", dt, x, B[:, :, 0, :])
    pref = np.cumsum(outer, axis=1)                          # [b, L, H, P, N]
    yr = np.einsum("blhpn,bln->blhp", pref, C[:, :, 0, :]) + D[None, None, :, None] * x
    return max(rel_err(y, yr), rel_err(fs, pref[:, -1])) < RTOL_EXACT, [rel_err(y, yr)]


def pin_no_memory(fwd):
    """P-3: a reset at every token leaves only the diagonal of M,
    y_t = (C_t . B_t) dt_t x_t + D x_t."""
    x, dt, A, B, C, D = small_inputs(seed=31, G=1)
    b, L = x.shape[:2]
    seq_idx = np.tile(np.arange(L, dtype=np.int32), (b, 1))
    y, _ = fwd(x, dt, A, B, C, D, seq_idx, None)
    cb = np.einsum("bln,bln->bl", C[:, :, 0, :], B[:, :, 0, :])
    yr = (cb[:, :, None, None] * dt[..., None] + D[None, None, :, None]) * x
    return rel_err(y, yr) < RTOL_EXACT, [rel_err(y, yr)]


def pin_geometric(fwd):
    """Scalar channel (P = N = 1) with constant inputs: the state is a
    geometric series, h_t = dt (1 - a^{t+1}) / (1 - a), so
    y_t = c b dt x (1 - a^{t+1}) / (1 - a) + D x."""
    L = 50
    dtv, Av, xv, bv, cv, Dv = 0.3, -0.7, 1.5, 0.8, -1.1, 0.25
    a = math.exp(dtv * Av)
    x = np.full((1, L, 1, 1), xv)
    dt = np.full((1, L, 1), dtv)
    A = np.array([Av])
    B = np.full((1, L, 1, 1), bv)
    C = np.full((1, L, 1, 1), cv)
    D = np.array([Dv])
    y, fs = fwd(x, dt, A, B, C, D, None, None)
    t = np.arange(L)
    h = dtv * xv * bv * (1 - a ** (t + 1)) / (1 - a)
    yr = cv * h + Dv * xv
    return (rel_err(y[0, :, 0, 0], yr) < RTOL_EXACT and
            rel_err(fs[0, 0, 0, 0], h[-1]) < RTOL_EXACT), [rel_err(y[0, :, 0, 0], yr)]


def pin_zero_inputs(fwd):
    """P-8: B = 0 gives y = D x exactly; C = 0 likewise; and with D = 0 the
    output is exactly 0."""
    x, dt, A, B, C, D = small_inputs(seed=41)
    ok = True
    y, fs = fwd(x, dt, A, np.zeros_like(B), C, D, None, None)
    ok &= bool(np.array_equal(y, D[None, None, :, None] * x)) and bool(np.all(fs == 0))
    y, _ = fwd(x, dt, A, B, np.zeros_like(C), D, None, None)
    ok &= bool(np.array_equal(y, D[None, None, :, None] * x))
    y, _ = fwd(x, dt, A, B, np.zeros_like(C), np.zeros_like(D), None, None)
    ok &= bool(np.all(y == 0))
    return ok, []


def pin_composition(fwd):
    """P-6: running [0, T/2) then [T/2, T) from the carried state equals one
    run over [0, T), the affine composition rule of page "Parallel Scan and
    Hardware-Aware SSM Kernels", section "The scan"."""
    x, dt, A, B, C, D = small_inputs(seed=51, L=40)
    y, fs = fwd(x, dt, A, B, C, D, None, None)
    m = 17
    y1, f1 = fwd(x[:, :m], dt[:, :m], A, B[:, :m], C[:, :m], D, None, None)
    y2, f2 = fwd(x[:, m:], dt[:, m:], A, B[:, m:], C[:, m:], D, None, f1)
    e = max(rel_err(np.concatenate([y1, y2], axis=1), y), rel_err(f2, fs))
    return e < RTOL_EXACT, [e]


def pin_packing(fwd):
    """P-7: a packed row equals independent runs of each document from a
    zero state, bit for bit (page "Parallel Scan and Hardware-Aware SSM
    Kernels", section "When it breaks": no leakage across documents)."""
    x, dt, A, B, C, D = small_inputs(seed=61, b=1, L=45)
    bounds = [0, 7, 8, 26, 45]
    seq_idx = np.zeros((1, 45), dtype=np.int32)
    for d in range(len(bounds) - 1):
        seq_idx[0, bounds[d]:bounds[d + 1]] = 3 * d + 1
    h0 = _rng(62).standard_normal((1, x.shape[2], x.shape[3], B.shape[3]))
    y, fs = fwd(x, dt, A, B, C, D, seq_idx, h0)
    ok = True
    for d in range(len(bounds) - 1):
        s0, s1 = bounds[d], bounds[d + 1]
        yd, fd = fwd(x[:, s0:s1], dt[:, s0:s1], A, B[:, s0:s1], C[:, s0:s1], D,
                     None, h0 if d == 0 else None)
        ok &= bool(np.array_equal(yd, y[:, s0:s1]))
        if d == len(bounds) - 2:
            ok &= bool(np.array_equal(fd, fs))
    return ok, []


def pin_linearity(fwd):
    """With a zero initial state the map x -> y is linear."""
    x, dt, A, B, C, D = small_inputs(seed=71)
    x2 = _rng(72).standard_normal(x.shape)
    y1, f1 = fwd(x, dt, A, B, C, D, None, None)
    y2, f2 = fwd(x2, dt, A, B, C, D, None, None)
    y3, f3 = fwd(2.0 * x - 3.0 * x2, dt, A, B, C, D, None, None)
    e = max(rel_err(y3, 2 * y1 - 3 * y2), rel_err(f3, 2 * f1 - 3 * f2))
    return e < RTOL_EXACT, [e]


def pin_group_map(fwd):
    """Head h reads B/C group h // (H/G) and batch rows are independent:
    each (batch, head) pair equals a single-head, single-group run on its
    own slices, bit for bit."""
    x, dt, A, B, C, D = small_inputs(seed=81, b=2, H=6, G=3)
    y, fs = fwd(x, dt, A, B, C, D, None, None)
    ok = True
    for bi in range(2):
        for h in range(6):
            g = h // 2
            ys, fss = fwd(x[bi:bi + 1, :, h:h + 1], dt[bi:bi + 1, :, h:h + 1], A[h:h + 1],
                          B[bi:bi + 1, :, g:g + 1], C[bi:bi + 1, :, g:g + 1], D[h:h + 1],
                          None, None)
            ok &= bool(np.array_equal(ys[0, :, 0], y[bi, :, h]))
            ok &= bool(np.array_equal(fss[0, 0], fs[bi, h]))
    return ok, []


ALL_PINS = [pin_dense_form, pin_linear_attention, pin_no_memory, pin_geometric,
            pin_zero_inputs, pin_composition, pin_packing, pin_linearity,
            pin_group_map]
