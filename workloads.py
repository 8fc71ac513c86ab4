"""Seeded synthetic inputs for the SSD chunked forward pass.

This module only draws random numbers and rounds them to the storage dtype.  It
holds none of the method's arithmetic, so both the fp64 CPU oracle and the HIP
path can consume exactly the same arrays without sharing any computation.

Workloads (value distributions follow the pages' description of the Mamba-2
selective SSM: x, B, C per token; dt > 0 per token and head; A < 0 per head):

  tiny      1 x 256,   H=2,  P=16,  N=16,  G=1, Q=64,  fp32 everywhere
  layer27b  8 x 2048,  H=80, P=64,  N=128, G=1, Q=256, bf16 x/B/C (the
            Mamba-2 2.7B-shaped layer)
  sweep     32768 tokens per call, (batch, seqlen) in
            {(32,1024),(16,2048),(8,4096),(4,8192),(2,16384)},
            H=32, P=64, N=128, G=1, Q in {128, 256}, bf16
  decay     1 x 65536, H=16, P=64, N=64, G=1, Q=256, bf16, strong decay
  packed    1 x 32768, H=32, P=128, N=64, G=8, Q=128, bf16, 8..64 packed
            documents with log-uniform lengths in [64, 8192]

Draw order (numpy PCG64, one generator per workload, seed 0 by default):
  1. document lengths (packed only)
  2. x  ~ N(0, 1)                      [b, L, H, P]
  3. dt = exp(U(ln lo, ln hi))          [b, L, H]   (log-uniform, > 0)
  4. A  = -exp(U(ln a_lo, ln a_hi))     [H]
  5. B  ~ N(0, 1) / sqrt(N)             [b, L, G, N]
  6. C  ~ N(0, 1) / sqrt(N)             [b, L, G, N]
  7. D  ~ N(0, 1)                       [H]
All draws are fp64, cast to fp32; x, B and C are then rounded to bf16 with
round-to-nearest-even when the workload stores them in bf16.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "SWEEP_SHAPES",
    "make_inputs",
    "custom_workload",
    "bf16_round",
    "bf16_bits",
    "doc_lengths",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk_size: int
    io: str  # "f32" or "bf16": storage dtype of x, B, C and y
    dt_range: tuple = (1e-3, 1e-1)
    a_range: tuple = (1.0, 16.0)
    packed: bool = False
    doc_range: tuple = (64, 8192)      # document lengths, log-uniform
    doc_count: tuple = (8, 64)         # accepted number of documents per row

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def algorithmic_bytes(self, with_final_states: bool = True) -> int:
        """Bytes one forward call must move at minimum: read x, dt, A, B, C,
        D (and seq_idx when packed), write y and final_states."""
        es = 2 if self.io == "bf16" else 4
        b, L, H, P, N, G = (self.batch, self.seqlen, self.nheads, self.headdim,
                            self.dstate, self.ngroups)
        n = 2 * b * L * H * P * es            # x in, y out
        n += 2 * b * L * G * N * es           # B, C
        n += b * L * H * 4                    # dt
        n += 2 * H * 4                        # A, D
        if self.packed:
            n += b * L * 4                    # seq_idx
        if with_final_states:
            n += b * H * P * N * 4
        return n


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 2, 16, 16, 1, 64, "f32"),
    "layer27b": Workload("layer27b", 8, 2048, 80, 64, 128, 1, 256, "bf16"),
    "decay": Workload("decay", 1, 65536, 16, 64, 64, 1, 256, "bf16",
                      dt_range=(1e-2, 1.0), a_range=(4.0, 64.0)),
    "packed": Workload("packed", 1, 32768, 32, 128, 64, 8, 128, "bf16",
                       packed=True),
}

SWEEP_SHAPES = [(32, 1024), (16, 2048), (8, 4096), (4, 8192), (2, 16384)]
for _b, _L in SWEEP_SHAPES:
    for _q in (128, 256):
        _n = f"sweep_b{_b}_L{_L}_q{_q}"
        WORKLOADS[_n] = Workload(_n, _b, _L, 32, 64, 128, 1, _q, "bf16")


def custom_workload(name="custom", batch=1, seqlen=256, nheads=2, headdim=16,
                    dstate=16, ngroups=1, chunk_size=64, io="f32",
                    dt_range=(1e-3, 1e-1), a_range=(1.0, 16.0),
                    packed=False, doc_range=(64, 8192), doc_count=(8, 64)) -> Workload:
    return Workload(name, batch, seqlen, nheads, headdim, dstate, ngroups,
                    chunk_size, io, tuple(dt_range), tuple(a_range), packed,
                    tuple(doc_range), tuple(doc_count))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    return (bf16_bits(a).astype(np.uint32) << 16).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The bf16 bit patterns (uint16) of fp32 values, round-to-nearest-even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> 16
    return r.astype(np.uint16)


def doc_lengths(rng: np.random.Generator, seqlen: int, lo=64, hi=8192,
                min_docs=8, max_docs=64) -> np.ndarray:
    """Document lengths for one packed row: draw round(exp(U(ln lo, ln hi)))
    until the total reaches seqlen, trim the last one to fit, and redraw the
    whole list when the count falls outside [min_docs, max_docs]."""
    if seqlen < min_docs or (max_docs * hi < seqlen):
        raise ValueError("doc_lengths: no list of lengths can meet the bounds")
    for _ in range(100000):
        lens = []
        total = 0
        while total < seqlen:
            n = int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
            lens.append(n)
            total += n
        lens[-1] -= total - seqlen      # stays >= 1: the total was < seqlen before it
        if min_docs <= len(lens) <= max_docs:
            return np.asarray(lens, dtype=np.int64)
    raise ValueError("doc_lengths: bounds too tight for the length distribution")


@dataclasses.dataclass
class Inputs:
    """Host arrays of one forward call.  x, B, C hold values already rounded
    to the storage dtype (fp32 arrays); *_bits hold the bf16 payload."""
    wl: Workload
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray
    seq_idx: Optional[np.ndarray]
    doc_lens: Optional[np.ndarray]


def make_inputs(wl: Workload, seed: int = 0, batch: Optional[int] = None,
                seqlen: Optional[int] = None) -> Inputs:
    """Draw the inputs of workload ``wl`` (optionally overriding batch or
    seqlen for a bounded sample of the same distribution)."""
    b = wl.batch if batch is None else batch
    L = wl.seqlen if seqlen is None else seqlen
    if batch is not None or seqlen is not None:
        wl = dataclasses.replace(wl, batch=b, seqlen=L)
    H, P, N, G = wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    rng = np.random.default_rng(seed)
    seq_idx = None
    lens = None
    if wl.packed:
        rows = []
        all_lens = []
        for _ in range(b):
            lens_r = doc_lengths(rng, L, wl.doc_range[0], wl.doc_range[1],
                                 wl.doc_count[0], wl.doc_count[1])
            all_lens.append(lens_r)
            rows.append(np.repeat(np.arange(len(lens_r), dtype=np.int32), lens_r))
        seq_idx = np.stack(rows).astype(np.int32)
        lens = all_lens[0] if b == 1 else all_lens
    x = rng.standard_normal((b, L, H, P)).astype(np.float32)
    lo, hi = wl.dt_range
    dt = np.exp(rng.uniform(math.log(lo), math.log(hi), size=(b, L, H))).astype(np.float32)
    alo, ahi = wl.a_range
    A = (-np.exp(rng.uniform(math.log(alo), math.log(ahi), size=(H,)))).astype(np.float32)
    Bm = (rng.standard_normal((b, L, G, N)) / math.sqrt(N)).astype(np.float32)
    Cm = (rng.standard_normal((b, L, G, N)) / math.sqrt(N)).astype(np.float32)
    D = rng.standard_normal((H,)).astype(np.float32)
    if wl.io == "bf16":
        x, Bm, Cm = bf16_round(x), bf16_round(Bm), bf16_round(Cm)
    return Inputs(wl, x, dt, A, Bm, Cm, D, seq_idx, lens)


@dataclasses.dataclass
class FusedInputs:
    """Extra inputs of the fused prologue/epilogue: raw per-token step-size
    values (before bias and softplus), a per-head bias and the gate input z
    (z already rounded to the storage dtype)."""
    dt_raw: np.ndarray     # [b, L, H] fp32
    dt_bias: np.ndarray    # [H] fp32
    z: np.ndarray          # [b, L, H, P] fp32 values


def make_fused_inputs(inp: Inputs, seed: int = 0) -> FusedInputs:
    """Draw the fused-path inputs for ``inp`` from a stream of their own (the
    arrays of make_inputs are unchanged): dt_raw ~ N(0, 0.5^2), dt_bias ~
    U(-7, -2) per head (so that softplus(dt_raw + dt_bias) lies mostly in
    [1e-3, 0.2], the range of the workloads' step sizes), z ~ N(0, 1)."""
    wl = inp.wl
    b, L, H, P = inp.x.shape
    rng = np.random.default_rng([seed, 1])
    dt_raw = (0.5 * rng.standard_normal((b, L, H))).astype(np.float32)
    dt_bias = rng.uniform(-7.0, -2.0, size=(H,)).astype(np.float32)
    z = rng.standard_normal((b, L, H, P)).astype(np.float32)
    if wl.io == "bf16":
        z = bf16_round(z)
    return FusedInputs(dt_raw, dt_bias, z)
