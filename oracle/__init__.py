"""fp64 CPU oracle for the SSD (Mamba-2) chunked forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import anything from here.  The HIP
product path shares no code with this package and never falls back to it.

Contents
  ssd_forward(...)   the sequential fp64 recurrence (plain C, OpenMP over the
                     independent (batch, head) pairs), the definition of what
                     the forward pass computes:
                       a_t = exp(dt_t A_h),  h_t = a_t h_{t-1} + dt_t x_t B_t^T,
                       y_t = h_t C_t + D_h x_t,
                     page "State Space Duality and Mamba-2", section "The
                     Mathematical Bridge" (recurrence, A_t = a_t I), with the
                     dt discretisation of page "NVIDIA Accelerates Mamba-2
                     Forward Kernel with CUDA Tile" (section "What CUDA Tile
                     Is") and the document reset of page "Parallel Scan and
                     Hardware-Aware SSM Kernels" (section "When it breaks").
  decay_mask(...)    the 1-semiseparable decay mask of each chunk, by its
                     definition L_ij = prod_{k=j+1..i} a_k for i >= j, else 0
                     (page "State Space Duality and Mamba-2", section "The
                     Mathematical Bridge", definition of L), with entries
                     across a document boundary set to zero.
  dt_prologue(...)   the step sizes from raw per-token values: plus a
                     per-head bias, then optionally softplus, then optionally
                     clamped to [lo, hi].
  gate(...)          the element-wise output gate y * silu(z), silu(z) =
                     z / (1 + e^-z).
  ssd_backward(...)  gradients of the forward pass w.r.t. every input, by
                     reverse-mode differentiation of the same recurrence
                     (fp64, small inputs).
  ssd_forward_fused(...)  dt_prologue, then ssd_forward, then gate: the scan
                     with the lightweight element-wise work around it that
                     page "NVIDIA Accelerates Mamba-2 Forward Kernel with
                     CUDA Tile" names as its neighbours ("What CUDA Tile Is
                     and Why It Suits Writing Mamba-2 Kernels": element-wise
                     gating; "From Python DSL to Production-Grade Kernels":
                     the scan is followed by gating, fused into one kernel).
                     The pages do not spell the gate or the dt map out; the
                     readings taken are Mamba-2's own: dt = softplus(raw +
                     bias) and out = (y + D x) * silu(z).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the C oracle with gcc (-O3, OpenMP, portable x86-64 code)."""
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    _lib = bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded oracle library."""
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.ssd_oracle_fwd_f64.argtypes = [i64] * 6 + [dp] * 6 + [
        ctypes.POINTER(ctypes.c_int32), dp, dp, dp, ctypes.c_int]
    lib.ssd_oracle_fwd_f64.restype = ctypes.c_int
    lib.ssd_oracle_max_threads.argtypes = []
    lib.ssd_oracle_max_threads.restype = ctypes.c_int
    return lib


def _dptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def ssd_forward(x, dt, A, B, C, D=None, seq_idx=None, init_states=None,
                nthreads: int = 0, return_final: bool = True, lib=None):
    """fp64 recurrence.  Arrays may be any float dtype; they are widened to
    fp64 exactly.  Shapes: x [b,L,H,P], dt [b,L,H], A [H], B/C [b,L,G,N],
    D [H] or None, seq_idx [b,L] int or None, init_states [b,H,P,N] or None.
    Returns (y [b,L,H,P] fp64, final_states [b,H,P,N] fp64 or None).
    ``lib`` selects another build of the same C source (tests only)."""
    if lib is None:
        lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    dt = np.ascontiguousarray(dt, dtype=np.float64)
    A = np.ascontiguousarray(A, dtype=np.float64)
    B = np.ascontiguousarray(B, dtype=np.float64)
    C = np.ascontiguousarray(C, dtype=np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dt.shape != (b, L, H) or A.shape != (H,) or B.shape != (b, L, G, N) or C.shape != B.shape:
        raise ValueError("oracle: inconsistent shapes")
    Dd = None if D is None else np.ascontiguousarray(D, dtype=np.float64)
    si = None
    if seq_idx is not None:
        si = np.ascontiguousarray(seq_idx, dtype=np.int32)
        if si.shape != (b, L):
            raise ValueError("oracle: seq_idx shape")
    h0 = None
    if init_states is not None:
        h0 = np.ascontiguousarray(init_states, dtype=np.float64)
        if h0.shape != (b, H, P, N):
            raise ValueError("oracle: init_states shape")
    y = np.empty((b, L, H, P), dtype=np.float64)
    fs = np.empty((b, H, P, N), dtype=np.float64) if return_final else None
    rc = lib.ssd_oracle_fwd_f64(
        b, L, H, P, N, G, _dptr(x), _dptr(dt), _dptr(A), _dptr(B), _dptr(C),
        _dptr(Dd),
        None if si is None else si.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        _dptr(h0), _dptr(y), _dptr(fs), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return y, fs


def decay_mask(dt, A, seq_idx=None, chunk_size: int = 64, chunk_begin: int = 0,
               chunk_count: Optional[int] = None) -> np.ndarray:
    """fp64 decay mask of chunks [chunk_begin, chunk_begin + chunk_count).

    Returns L [b, H, chunk_count, Q, Q] with L[..., i, j] = prod over
    k in (j, i] of a_k for i >= j inside the chunk, 1 on the diagonal and 0
    above it, where a_k = exp(dt_k A_h), masked to 0 at a document boundary
    (seq_idx[k] != seq_idx[k-1]).  Positions past the end of the sequence
    are 0.  The product is formed along each row from the diagonal
    leftwards, which is the definition written as a loop."""
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    b, L, H = dt.shape
    Q = int(chunk_size)
    nchunks = (L + Q - 1) // Q
    if chunk_count is None:
        chunk_count = nchunks - chunk_begin
    out = np.zeros((b, H, chunk_count, Q, Q), dtype=np.float64)
    for ci in range(chunk_count):
        c = chunk_begin + ci
        t0 = c * Q
        n = max(0, min(Q, L - t0))
        if n == 0:
            continue
        a = np.exp(dt[:, t0:t0 + n, :] * A[None, None, :])   # [b, n, H]
        if seq_idx is not None:
            si = np.asarray(seq_idx)
            boundary = np.zeros((b, n), dtype=bool)
            lo = max(t0, 1)
            boundary[:, lo - t0:] = si[:, lo:t0 + n] != si[:, lo - 1:t0 + n - 1]
            a = np.where(boundary[:, :, None], 0.0, a)
        a = np.transpose(a, (0, 2, 1))                          # [b, H, n]
        for i in range(n):
            prod = np.ones((b, H), dtype=np.float64)
            out[:, :, ci, i, i] = 1.0
            for j in range(i - 1, -1, -1):
                prod = prod * a[:, :, j + 1]
                out[:, :, ci, i, j] = prod
    return out


def softplus(v):
    """softplus(v) = log(1 + e^v) in fp64, written as log1p(exp(v)) for
    v <= 0 and as v + log1p(exp(-v)) for v > 0 (the same function; the
    second form avoids overflowing e^v)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    neg = v <= 0
    out[neg] = np.log1p(np.exp(v[neg]))
    pos = ~neg
    out[pos] = v[pos] + np.log1p(np.exp(-v[pos]))
    return out


def dt_prologue(dt_raw, dt_bias=None, dt_softplus: bool = False, dt_limit=None):
    """Step sizes dt [b, L, H] (fp64) from raw values dt_raw [b, L, H]:
    dt = dt_raw + dt_bias[h] (if a bias is given), then softplus (if
    dt_softplus), then clamped to [lo, hi] (if dt_limit = (lo, hi))."""
    dt = np.asarray(dt_raw, dtype=np.float64).copy()
    if dt_bias is not None:
        dt = dt + np.asarray(dt_bias, dtype=np.float64)[None, None, :]
    if dt_softplus:
        dt = softplus(dt)
    if dt_limit is not None:
        lo, hi = float(dt_limit[0]), float(dt_limit[1])
        dt = np.minimum(np.maximum(dt, lo), hi)
    return dt


def gate(y, z):
    """Element-wise output gate y * silu(z) = y * z / (1 + e^-z), fp64.
    For z < 0 the same value is formed as y * z e^z / (1 + e^z), which
    cannot overflow."""
    y = np.asarray(y, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    sig = np.empty_like(z)
    pos = z >= 0
    sig[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    sig[~pos] = ez / (1.0 + ez)
    return y * z * sig


def ssd_forward_fused(x, dt_raw, A, B, C, D=None, seq_idx=None, init_states=None,
                      dt_bias=None, dt_softplus: bool = False, dt_limit=None, z=None,
                      nthreads: int = 0, return_final: bool = True, lib=None):
    """The forward pass with its element-wise neighbours, in order:
    dt = dt_prologue(dt_raw, dt_bias, dt_softplus, dt_limit); the fp64
    recurrence (ssd_forward) on that dt; then, if z [b, L, H, P] is given,
    out = gate(y, z) with y including the skip D x.  final_states is the
    recurrence's state (the gate touches only the output).  Returns
    (out, final_states) like ssd_forward."""
    dt = dt_prologue(dt_raw, dt_bias, dt_softplus, dt_limit)
    y, fs = ssd_forward(x, dt, A, B, C, D, seq_idx, init_states, nthreads=nthreads,
                        return_final=return_final, lib=lib)
    if z is not None:
        y = gate(y, z)
    return y, fs


def ssd_backward(x, dt, A, B, C, D, dy, seq_idx=None, init_states=None, dfinal=None):
    """Gradients of the forward pass, fp64, by reverse-mode differentiation of
    the recurrence (what a backward pass computes; pure-Python loop over
    tokens, small inputs only).

    With y, final_states = ssd_forward(x, dt, A, B, C, D, seq_idx, init_states)
    and the scalar J = <dy, y> + <dfinal, final_states> (dfinal None = 0),
    returns a dict of dJ/d(input): dx [b,L,H,P], ddt [b,L,H], dA [H],
    dB, dC [b,L,G,N], dD [H] (None if D is None), dinit [b,H,P,N] (None if
    init_states is None).  The recurrence is the one of ssd_forward: with
    a_t = exp(dt_t A_h), set to 0 where a document starts (page "Parallel
    Scan and Hardware-Aware SSM Kernels", "When it breaks": no gradient flows
    through a reset), h_t = a_t h_{t-1} + dt_t x_t B_t^T and
    y_t = h_t C_t + D_h x_t (page "State Space Duality and Mamba-2", "The
    Mathematical Bridge").  Walking t from the end: g_t = dJ/dh_t collects
    dy_t C_t^T, feeds dx_t, dB_t, ddt_t through the input term and
    dJ/da_t = <g_t, h_{t-1}> through the decay (a_t A_h into ddt_t,
    a_t dt_t into dA_h), then g_{t-1} = a_t g_t."""
    x = np.asarray(x, dtype=np.float64)
    dt = np.asarray(dt, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    grp = np.arange(H) // hpg
    Bh = B[:, :, grp, :]                                   # [b, L, H, N]
    Ch = C[:, :, grp, :]
    a = np.exp(dt * A[None, None, :])                      # [b, L, H]
    if seq_idx is not None:
        si = np.asarray(seq_idx)
        reset = np.zeros((b, L), dtype=bool)
        reset[:, 1:] = si[:, 1:] != si[:, :-1]
        a = np.where(reset[:, :, None], 0.0, a)
    h0 = (np.zeros((b, H, P, N)) if init_states is None
          else np.asarray(init_states, dtype=np.float64).copy())
    # forward, keeping every state
    hs = np.empty((b, L, H, P, N))
    h = h0.copy()
    for t in range(L):
        h = a[:, t, :, None, None] * h + (dt[:, t, :, None, None] * x[:, t, :, :, None]) * Bh[:, t, :, None, :]
        hs[:, t] = h
    # reverse
    g = np.zeros((b, H, P, N)) if dfinal is None else np.asarray(dfinal, dtype=np.float64).copy()
    dx = np.zeros_like(x)
    ddt = np.zeros_like(dt)
    dA = np.zeros(H)
    dBh = np.zeros((b, L, H, N))
    dCh = np.zeros((b, L, H, N))
    for t in range(L - 1, -1, -1):
        g = g + dy[:, t, :, :, None] * Ch[:, t, :, None, :]                   # y_t = h_t C_t
        dCh[:, t] = np.einsum("bhpn,bhp->bhn", hs[:, t], dy[:, t])
        gB = np.einsum("bhpn,bhn->bhp", g, Bh[:, t])                           # g_t B_t
        dx[:, t] = dt[:, t, :, None] * gB
        dBh[:, t] = dt[:, t, :, None] * np.einsum("bhpn,bhp->bhn", g, x[:, t])
        ddt[:, t] = np.einsum("bhp,bhp->bh", gB, x[:, t])                      # input term
        hprev = hs[:, t - 1] if t > 0 else h0
        ga = np.einsum("bhpn,bhpn->bh", g, hprev) * a[:, t]                   # dJ/da_t * a_t
        ddt[:, t] += ga * A[None, :]
        dA += (ga * dt[:, t]).sum(axis=0)
        g = a[:, t, :, None, None] * g                                         # dJ/dh_{t-1}
    dD = None
    if D is not None:
        D = np.asarray(D, dtype=np.float64)
        dx += D[None, None, :, None] * dy
        dD = np.einsum("blhp,blhp->h", dy, x)
    dB = dBh.reshape(b, L, G, hpg, N).sum(axis=3)
    dC = dCh.reshape(b, L, G, hpg, N).sum(axis=3)
    return {"dx": dx, "ddt": ddt, "dA": dA, "dB": dB, "dC": dC, "dD": dD,
            "dinit": None if init_states is None else g}
