"""Benchmark of the SSD chunked forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload layer27b]

A step is one full forward pass (every kernel of the path) over one batch of
seeded synthetic inputs already resident in HBM; the default workload is the
Mamba-2 2.7B-shaped layer: batch 8, seqlen 2048, 80 heads, headdim 64, dstate
128, 1 group, chunk 256, x/B/C/y in bf16, dt/A/D and the states in fp32.

Prints one JSON line with the throughput (tokens/s over K back-to-back
steps), the HBM roofline of the forward pass (algorithmic bytes per call over
its average duration, each call timed cold -- a 512 MiB scratch buffer written
before it, so that neither L2 nor the Infinity Cache holds its inputs -- with
HIP events on the stream the kernels run on; the head kernel alone and the
back-to-back figures beside it), and the fp64 CPU oracle timed on the host
cores as a reported baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP32_MFMA_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix
METRIC = "SSD fwd tokens/s + HBM GB/s (% of peak), Mamba-2 2.7B layer, L=2048"
HEAD_KERNEL_SOURCES = ("ssd_api.cpp", "ssd_cb.hip", "ssd_common.hpp", "ssd_scan_bf16.hpp",
                       "ssd_scan_bf16_q64.hip", "ssd_scan_bf16_q128.hip", "ssd_scan_bf16_q256.hip",
                       "ssd_segsum.hpp", "ssd_tiles.hpp")


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (a comment edit does not
    change the kernels the counters were taken on)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_digest() -> str:
    """Digest of the code (comments stripped) of the sources that define the
    bf16 forward kernels and their launch (the counters are only valid for
    them)."""
    csrc = os.path.join(ROOT, "ssd_chunked_scan_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f in HEAD_KERNEL_SOURCES:
            h.update(f.encode())
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per forward pass (both kernels) from the committed rocprofv3
    counter summary of this workload, if it was taken on the current kernel
    sources."""
    path = os.path.join(ROOT, "profiles", f"ssd_fwd_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_forward"])
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, repeats: int = 3):
    """The fp64 oracle on the host cores over the whole workload (every batch
    row and head); median of ``repeats`` runs.  The oracle parallelises over
    the independent (batch row, head) pairs with OpenMP, so the threads it
    uses are the smaller of its thread count and that pair count."""
    import oracle
    threads = oracle.max_threads()
    units = inp.wl.batch * inp.wl.nheads
    times = []
    for _ in range(repeats):
        t = time.perf_counter()
        oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.seq_idx)
        times.append(time.perf_counter() - t)
    times.sort()
    med = times[len(times) // 2]
    return {"value": inp.wl.tokens / med, "unit": "tokens/s", "cores": min(threads, units),
            "kind": "oracle", "omp_threads": threads, "os_cpu_count": os.cpu_count(),
            "cpu_model": cpu_model(),
            "sample": f"whole workload ({inp.wl.batch}x{inp.wl.seqlen} tokens x {inp.wl.nheads} "
                      f"heads), fp64 recurrence, median of {repeats} runs of {med:.2f} s"}


def segsum_ablation(wl, inp, args):
    """One JSON line: the segsum ablation (page "GPU Hierarchy Meets
    Structured Matrices", abstract: direct segsum ~30% slower than the diff
    segsum; hierarchy-aware 1.35-1.40x faster than a naive direct one).

    head_kernel: the bf16 head kernels of the forward pass (every launch but
    the per-group operand kernel, whose output the workspace already holds)
    with each evaluation of the mask on the output path, cold (the 512 MiB
    flush before every call) and warm, per call on the kernels' stream; the
    variants take turns call by call so that they see the same machine state.
    mask_export: the mask evaluation alone over every (batch row, head, chunk),
    through the sums-only mask export (no mask traffic)."""
    import torch
    import ssd_chunked_scan_amd as ssd
    dev = torch.device("cuda:0")
    variants = ("hierarchy", "direct", "diff")
    stream = torch.cuda.current_stream(dev)
    res = {"workload": wl.name}
    if wl.io == "bf16" and wl.chunk_size == 256:
        t = lambda a, d=torch.float32: torch.from_numpy(a).to(dev).to(d).contiguous()
        io = torch.bfloat16
        x, dt, A, B, C, D = t(inp.x, io), t(inp.dt), t(inp.A), t(inp.B, io), t(inp.C, io), t(inp.D)
        seq = None if inp.seq_idx is None else torch.from_numpy(inp.seq_idx).to(dev)
        y = torch.empty_like(x)
        fs = torch.empty((wl.batch, wl.nheads, wl.headdim, wl.dstate), dtype=torch.float32, device=dev)
        shape = ssd.Shape(wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups)
        ws = torch.empty(max(ssd.ssd_fwd_workspace_bytes(shape, wl.chunk_size, 1), 16),
                         dtype=torch.uint8, device=dev)
        full, _, _ = ssd.prepare_fwd(x, dt, A, B, C, D, seq, chunk_size=wl.chunk_size, y=y,
                                     final_states=fs, workspace=ws)
        full()   # the per-group operands into the workspace
        heads = {v: ssd.prepare_fwd(x, dt, A, B, C, D, seq, chunk_size=wl.chunk_size, y=y,
                                    final_states=fs, workspace=ws, reuse_group_operands=True,
                                    segsum=v)[0] for v in variants}
        for _ in range(args.warmup):
            for v in variants:
                heads[v]()
        torch.cuda.synchronize(dev)
        flush_buf = torch.ones(512 << 18, dtype=torch.float32, device=dev)   # 512 MiB
        flush_sink = torch.empty((), dtype=torch.float32, device=dev)
        mk = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        cold = {v: [] for v in variants}
        warm = {v: [] for v in variants}
        for k in range(args.steps):
            for v in variants:
                torch.sum(flush_buf, dim=0, out=flush_sink)
                e = mk()
                e[0].record(stream)
                heads[v]()
                e[1].record(stream)
                cold[v].append(e)
        for k in range(args.steps):
            for v in variants:
                e = mk()
                e[0].record(stream)
                heads[v]()
                e[1].record(stream)
                warm[v].append(e)
        torch.cuda.synchronize(dev)
        del flush_buf
        summ = lambda evs: (lambda ms: {"avg_us": sum(ms) / len(ms) * 1e3, "median_us": ms[len(ms) // 2] * 1e3,
                                        "p10_us": ms[len(ms) // 10] * 1e3,
                                        "p90_us": ms[(9 * len(ms)) // 10] * 1e3})(
            sorted(a.elapsed_time(b) for a, b in evs))
        hk = {"cold": {v: summ(cold[v]) for v in variants}, "warm": {v: summ(warm[v]) for v in variants}}
        for kind in ("cold", "warm"):
            u = {v: hk[kind][v]["avg_us"] for v in variants}
            hk[kind]["direct_over_hierarchy"] = u["direct"] / u["hierarchy"]
            hk[kind]["diff_over_hierarchy"] = u["diff"] / u["hierarchy"]
            hk[kind]["direct_over_diff"] = u["direct"] / u["diff"]
            print(f"bench: head kernels {kind}: " + ", ".join(f"{v} {u[v]:.1f} us" for v in variants),
                  file=sys.stderr, flush=True)
        res["head_kernel"] = hk
        del heads, full, ws, x, B, C, y
    dt = torch.from_numpy(inp.dt).to(dev)
    A = torch.from_numpy(inp.A).to(dev)
    seq = None if inp.seq_idx is None else torch.from_numpy(inp.seq_idx).to(dev)
    mx = {}
    for v in variants:
        run = lambda: ssd.ssd_debug_chunk_mask(dt, A, seq, chunk_size=wl.chunk_size, variant=v,
                                               sums_only=True)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize(dev)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record(stream)
            run()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        tt = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
        mx[v] = sum(tt) / len(tt)
        print(f"bench: mask export {v}: {mx[v]:.1f} us per launch (p10 {tt[len(tt) // 10]:.1f})",
              file=sys.stderr, flush=True)
    units = wl.batch * wl.nheads * ((wl.seqlen + wl.chunk_size - 1) // wl.chunk_size)
    res["mask_export"] = {"us": mx, "chunk_units": units,
                          "direct_over_hierarchy": mx["direct"] / mx["hierarchy"],
                          "diff_over_hierarchy": mx["diff"] / mx["hierarchy"]}
    print(json.dumps({"metric": "segsum ablation: time per call by mask evaluation", "unit": "us",
                      "higher_is_better": False, **res}), flush=True)


def decode_step_bench(wl, inp, args):
    """One JSON line: the decode step (one token per (batch row, head)) at the
    workload's sizes, timed with HIP events per launch; roofline against HBM:
    algorithmic bytes = state read + written (fp32) + x, y, B, C, dt, A, D."""
    import numpy as np
    import torch
    import ssd_chunked_scan_amd as ssd
    dev = torch.device("cuda:0")
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    esz = 2 if wl.io == "bf16" else 4
    b, H, P, N, G = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    t = lambda a, d=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(d)
    x, dt, A = t(inp.x[:, 0], io), t(inp.dt[:, 0]), t(inp.A)
    B, C, D = t(inp.B[:, 0], io), t(inp.C[:, 0], io), t(inp.D)
    state = torch.zeros((b, H, P, N), dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    run = lambda: ssd.ssd_decode_step(x, dt, A, B, C, D, state, y=y)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        run()
        e1.record(stream)
    torch.cuda.synchronize(dev)
    us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in ev)
    avg = sum(us) / len(us)
    nbytes = 2 * b * H * P * N * 4 + 2 * b * H * P * esz + 2 * b * G * N * esz + b * H * 4 + 2 * H * 4
    gbs = nbytes / (avg * 1e-6) / 1e9
    print(f"bench: decode step {b}x{H} heads P{P} N{N}: {avg:.2f} us per launch "
          f"(p10 {us[len(us) // 10]:.2f}), {gbs:.0f} GB/s", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": "decode step time per launch", "unit": "us", "value": avg, "higher_is_better": False,
        "config": {"workload": wl.name + " decode step", "batch": b, "nheads": H, "headdim": P,
                   "dstate": N, "ngroups": G, "io": wl.io},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": 8000.0, "unit": "GB/s",
                     "frac": gbs / 8000.0, "bytes_per_launch": nbytes}}), flush=True)


def backward_bench(wl, inp, args):
    """One JSON line: the backward pass (ssd_bwd) at the workload's sizes,
    per-launch time with HIP events on its stream; roofline against HBM with
    the algorithmic bytes of the gradients' inputs and outputs (x, dy, B, C,
    dt, D read; dx, ddt, dB, dC written in fp32; the entering states the
    pass writes and reads once each)."""
    import numpy as np
    import torch
    import ssd_chunked_scan_amd as ssd
    dev = torch.device("cuda:0")
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    t = lambda a, d=torch.float32: torch.from_numpy(a).to(dev).to(d).contiguous()
    x, dt, A, B, C, D = t(inp.x, io), t(inp.dt), t(inp.A), t(inp.B, io), t(inp.C, io), t(inp.D)
    dy = t(np.random.default_rng(1).standard_normal(inp.x.shape).astype(np.float32), io)
    for _ in range(args.warmup):
        ssd.ssd_bwd(x, dt, A, B, C, D, dy)
    torch.cuda.synchronize(dev)
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for e0, e1 in ev:
        e0.record(stream)
        ssd.ssd_bwd(x, dt, A, B, C, D, dy)
        e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    avg = sum(ms) / len(ms)
    b, L, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    esz = 2 if wl.io == "bf16" else 4
    nch = (L + 63) // 64
    alg = (2 * b * L * H * P * esz + 2 * b * L * G * N * esz + b * L * H * 4     # x, dy, B, C, dt
           + b * L * H * P * 4 + b * L * H * 4 + 2 * b * L * G * N * 4          # dx, ddt, dB, dC
           + 2 * b * H * nch * P * N * 4)                                       # states
    gbs = alg / (avg * 1e-3) / 1e9
    # MFMA work the backward kernel executes, per 64-token chunk and (batch
    # row, head).  bf16 inputs: every product on bf16 16x16x32 steps (16384
    # flop): the masked ones over the pairs of 16-row blocks a triangle
    # touches, the ones with a carried state (B G^T, x G, dY H, u dy C^T) as
    # hi + lo steps, C B^T and dY X^T over the lower tiles when bf16 rows are
    # staged (headdim <= 64), else on fp32 steps.  fp32 inputs: fp32 16x16x4
    # steps (2048 flop) throughout, the triangles over whole 16-row blocks.
    nb, ntri = 4, 10                          # 16-row blocks per chunk, lower tiles
    c32 = lambda k: (k + 31) // 32
    if wl.io == "bf16":
        m_up = sum(1 for j in range(nb) for q in range(nb // 2) if 2 * q + 1 >= j)   # dX, dB
        m_lo = sum(1 for t in range(nb) for q in range(nb // 2) if 2 * q <= t)       # dC
        bf = ((P // 16) * (m_up + nb * 2 * c32(N))                 # dX: masked, B G^T
              + (N // 16) * (m_up + m_lo + 2 * nb * 2 * c32(P))    # dB, dC: masked, x G, dY H
              + (P // 16) * (N // 16) * nb)                        # adjoint update
        f32 = 0
    else:
        tri = 4 * ntri                        # steps of one column tile's triangle
        bf = 0
        f32 = ((P // 16) * tri + nb * (P // 16) * (N // 4)          # dX: (L o S)^T dY, G B_j
               + (N // 16) * 2 * tri + nb * (N // 16) * 2 * (P // 4)  # dB, dC and their state terms
               + (P // 16) * (N // 16) * 16)                        # state adjoint update
    if wl.io == "bf16" and P <= 64:
        bf += ntri * (max(1, N // 32) + max(1, P // 32))
    else:
        f32 += ntri * (N // 4 + P // 4)
    units = b * H * nch
    flop = units * (f32 * 2048 + bf * 16384)
    # the mix's peak: its flops over the time the matrix pipes take at their
    # published rate for each step type, so frac is the pipes' busy fraction
    pipe_s = units * (bf * 16384 / (BF16_MFMA_PEAK_TFLOPS * 1e12) + f32 * 2048 / (FP32_MFMA_PEAK_TFLOPS * 1e12))
    peak = flop / pipe_s / 1e12
    tflops = flop / (avg * 1e-3) / 1e12
    print(json.dumps({
        "metric": "SSD backward time per launch", "unit": "us", "value": avg * 1e3,
        "higher_is_better": False, "steps": args.steps, "warmup": args.warmup, "dtype": wl.io,
        "data": "synthetic", "tokens_per_s": wl.tokens / (avg * 1e-3),
        "config": {"workload": wl.name, "batch": b, "seqlen": L, "nheads": H, "headdim": P,
                   "dstate": N, "ngroups": G, "backward_chunk": 64},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": alg},
        # executed MFMA flops over the whole pass's time (a lower bound for the
        # kernel alone) against the peak of the step mix (bf16 and fp32 steps
        # each at their published dense rate)
        "mfma": {"flop_per_launch": flop, "bf16_steps_per_chunk": bf, "fp32_steps_per_chunk": f32,
                 "achieved": tflops, "peak": peak, "unit": "TFLOP/s", "frac": tflops / peak},
        "p10_us": ms[len(ms) // 10] * 1e3, "p90_us": ms[(9 * len(ms)) // 10] * 1e3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer27b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="instead of the forward pass: time the single-token decode step at the "
                         "workload's batch, heads and state size (state read and written once)")
    ap.add_argument("--segsum-ablation", action="store_true",
                    help="instead of the forward pass: time the three segsum evaluations of the "
                         "decay mask (hierarchy-aware, direct, prefix difference) inside the bf16 "
                         "head kernel (chunk 256) and in the mask export alone")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the forward pass: time the backward pass (ssd_bwd)")
    ap.add_argument("--flush", choices=["write", "read"], default="read",
                    help="how the caches are emptied before each cold call: write a 512 MiB scratch "
                         "buffer (also leaves dirty lines to write back), or read one")
    ap.add_argument("--cold-only", action="store_true",
                    help="only the cold per-call timing of the forward pass (the flush before "
                         "each call), then one 256 MiB device copy: the command the rocprofv3 "
                         "kernel statistics and counters are taken with, so that every profiled "
                         "call is a cold one and the copy calibrates the byte counters")
    ap.add_argument("--fused", action="store_true",
                    help="time the forward pass with the fused prologue (raw dt + bias, softplus) "
                         "and the silu(z) output gate; z counts as algorithmic bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the forward pass shards by head or by sequence without a collective for the "
              "head split, but no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ssd_chunked_scan_amd as ssd
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    inp = workloads.make_inputs(wl, seed=0)
    if args.segsum_ablation:
        segsum_ablation(wl, inp, args)
        return
    if args.decode:
        decode_step_bench(wl, inp, args)
        return
    if args.backward:
        backward_bench(wl, inp, args)
        return
    dev = torch.device("cuda:0")
    io = torch.bfloat16 if wl.io == "bf16" else torch.float32
    t = lambda a, d=torch.float32: torch.from_numpy(a).to(dev).to(d).contiguous()
    x, dt, A, B, C, D = t(inp.x, io), t(inp.dt), t(inp.A), t(inp.B, io), t(inp.C, io), t(inp.D)
    seq = None if inp.seq_idx is None else torch.from_numpy(inp.seq_idx).to(dev)
    y = torch.empty_like(x)
    fs = torch.empty((wl.batch, wl.nheads, wl.headdim, wl.dstate), dtype=torch.float32, device=dev)
    shape = ssd.Shape(wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups)
    io_code = 1 if wl.io == "bf16" else 0
    ws_bytes = ssd.ssd_fwd_workspace_bytes(shape, wl.chunk_size, io_code)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    split_len = ssd.ssd_plan_split_len(shape, wl.chunk_size, io_code)

    # Fused prologue/epilogue variant: raw dt through bias + softplus, and the
    # silu(z) output gate (z read once more: its bytes count as algorithmic).
    fused_kw = {}
    extra_bytes = 0
    if args.fused:
        fz = workloads.make_fused_inputs(inp, seed=0)
        dt = t(fz.dt_raw)
        fused_kw = dict(dt_bias=t(fz.dt_bias), dt_softplus=True, z=t(fz.z, io))
        extra_bytes = fz.z.size * (2 if wl.io == "bf16" else 4) + fz.dt_bias.size * 4

    # Arguments are checked and marshalled once; each step is one call into
    # the C ABI (host work per step: one ctypes call and the library's own
    # validation), so the timed loop measures the device, not Python.
    step, _, _ = ssd.prepare_fwd(x, dt, A, B, C, D, seq, chunk_size=wl.chunk_size, y=y,
                                 final_states=fs, workspace=ws, **fused_kw)

    print(f"bench: {wl.name} {wl.batch}x{wl.seqlen} H{wl.nheads} P{wl.headdim} N{wl.dstate} "
          f"G{wl.ngroups} Q{wl.chunk_size} {wl.io}; split {split_len} tokens; warmup "
          f"{args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)

    stream = torch.cuda.current_stream(dev)
    flush_buf = torch.ones(512 << 18, dtype=torch.float32, device=dev)   # 512 MiB
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush(k):
        if args.flush == "write":
            flush_buf.fill_(float(k & 0xFF))
        else:
            torch.sum(flush_buf, dim=0, out=flush_sink)

    if args.cold_only:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for k, (e0, e1) in enumerate(ev):
            flush(k)
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        avg = sum(ms) / len(ms)
        # a plain device copy of known size after the timed calls: under
        # rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE give the factors from
        # counter units to bytes
        cal = 256 << 20
        cal_src = torch.ones(cal, dtype=torch.uint8, device=dev)
        cal_dst = torch.empty_like(cal_src)
        cal_dst.copy_(cal_src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"metric": "forward pass time per call, cold", "unit": "us", "flush": args.flush,
                          "workload": wl.name, "steps": args.steps, "avg_us": avg * 1e3,
                          "median_us": ms[len(ms) // 2] * 1e3,
                          "p10_us": ms[len(ms) // 10] * 1e3, "p90_us": ms[(9 * len(ms)) // 10] * 1e3,
                          "gbs": (wl.algorithmic_bytes() + extra_bytes) / (avg * 1e-3) / 1e9,
                          "calibration_copy_bytes": cal}),
              flush=True)
        return

    # Whole-job timing: K back-to-back steps between two synchronisations.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # Per-launch timing with HIP events on the stream the kernels run on: the
    # whole forward pass, and the head kernel alone (the same call told that
    # the workspace already holds the per-group operands, which the previous
    # step wrote).

    def event_times(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        return sorted(e0.elapsed_time(e1) for e0, e1 in ev)

    # The same step captured in a HIP graph and replayed (no host launch work
    # between kernels); every replay's outputs are checked against the eager
    # step's before the graph is timed.
    gstream = torch.cuda.Stream(dev)
    with torch.cuda.stream(gstream):
        gstep, gy, gfs = ssd.prepare_fwd(x, dt, A, B, C, D, seq, chunk_size=wl.chunk_size,
                                         workspace=torch.empty_like(ws),
                                         stream=gstream.cuda_stream, **fused_kw)
        gstep()
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=gstream):
        gstep()
    step()
    torch.cuda.synchronize(dev)
    for _ in range(3):
        gy.zero_()
        torch.cuda.synchronize(dev)
        graph.replay()
        torch.cuda.synchronize(dev)
        if not (torch.equal(gy, y) and torch.equal(gfs, fs)):
            raise RuntimeError("bench: graph replay differs from the eager step")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize(dev)
    graph_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    print(f"bench: graph replay {graph_ms_per_step * 1e3:.1f} us/step (eager {ms_per_step * 1e3:.1f})",
          file=sys.stderr, flush=True)

    # Cold timing: before every timed call a 512 MiB scratch buffer is
    # written or read (outside the events), which evicts the inputs and the
    # per-group operands from L2 and from the 256 MB Infinity Cache, so each
    # call streams x from HBM.  Per-call HIP events on the kernels' stream.
    def cold_times(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for k, (e0, e1) in enumerate(ev):
            flush(k)
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize(dev)
        return sorted(e0.elapsed_time(e1) for e0, e1 in ev)

    def summary(ms):
        n = len(ms)
        return {"avg_us": sum(ms) / n * 1e3, "median_us": ms[n // 2] * 1e3,
                "p10_us": ms[n // 10] * 1e3, "p90_us": ms[(9 * n) // 10] * 1e3}

    alg_bytes = wl.algorithmic_bytes() + extra_bytes
    head_only = wl.io == "bf16" and split_len >= wl.seqlen
    head_step, _, _ = ssd.prepare_fwd(x, dt, A, B, C, D, seq, chunk_size=wl.chunk_size, y=y,
                                      final_states=fs, workspace=ws, reuse_group_operands=True,
                                      **fused_kw)
    fwd_cold = summary(cold_times(step, args.steps))
    fwd_warm = summary(event_times(step))
    # The head kernel alone is timed back to back only: a flush before a
    # head-only call would also evict the per-group operands, which inside a
    # forward call the per-group kernel has just written to L2 (the cold split
    # between the kernels is in the rocprofv3 kernel statistics under profiles/).
    head_warm = summary(event_times(head_step)) if head_only else None
    gbs = lambda us: alg_bytes / (us * 1e-6) / 1e9
    print(f"bench: wall {ms_per_step * 1e3:.1f} us/step back to back; forward pass cold "
          f"avg {fwd_cold['avg_us']:.1f} us (median {fwd_cold['median_us']:.1f}, p10 "
          f"{fwd_cold['p10_us']:.1f}, p90 {fwd_cold['p90_us']:.1f}), warm avg {fwd_warm['avg_us']:.1f} us",
          file=sys.stderr, flush=True)
    if head_only:
        print(f"bench: head kernel alone, back to back: avg {head_warm['avg_us']:.1f} us",
              file=sys.stderr, flush=True)
    achieved = gbs(fwd_cold["avg_us"])

    # Measured device-to-device copy moving the same number of bytes (half
    # read, half written), timed cold like the forward pass: the attainable-
    # bandwidth reference, and the plain copy kernel whose counters calibrate
    # the HBM-traffic counters.
    copy_src = torch.empty(alg_bytes // 2, dtype=torch.uint8, device=dev)
    copy_dst = torch.empty_like(copy_src)
    for _ in range(3):
        copy_dst.copy_(copy_src)
    copy_cold = summary(cold_times(lambda: copy_dst.copy_(copy_src), max(10, args.steps // 2)))
    copy_gbs = gbs(copy_cold["avg_us"])
    del copy_src, copy_dst, flush_buf
    print(f"bench: forward pass {achieved:.0f} GB/s algorithmic (cold); copy of the same bytes "
          f"{copy_gbs:.0f} GB/s (cold)", file=sys.stderr, flush=True)
    traffic = None if args.fused else counter_traffic(wl.name)
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": ("forward pass: ssd_cb_kernel + ssd_scan_bf16_kernel" if wl.io == "bf16"
                           else "forward pass: ssd_chunk_f32_kernel"),
                "timing": f"cold: 512 MiB scratch {'written' if args.flush == 'write' else 'read'} before "
                          "each call; HIP events per call, average",
                "algorithmic_bytes_per_launch": alg_bytes,
                "avg_launch_us": fwd_cold["avg_us"], "median_us": fwd_cold["median_us"],
                "p10_us": fwd_cold["p10_us"], "p90_us": fwd_cold["p90_us"],
                "back_to_back": {"avg_us": fwd_warm["avg_us"], "frac": gbs(fwd_warm["avg_us"]) / HBM_PEAK_GBS}}
    if head_only:
        roofline["head_kernel"] = {
            "kernel": "ssd_scan_bf16_kernel (per-group operands already in the workspace)",
            "back_to_back": dict(head_warm, frac=gbs(head_warm["avg_us"]) / HBM_PEAK_GBS)}
    out = {
        "metric": METRIC,
        "value": wl.tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "graph_ms_per_step": graph_ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.io,
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: " + ("Mamba-2 2.7B-shaped SSD layer" if wl.name == "layer27b"
                                                 else "SSD forward, synthetic inputs")
                               + (", fused dt softplus(dt + bias) and silu(z) gate" if args.fused else ""),
                   "batch": wl.batch,
                   "seqlen": wl.seqlen, "nheads": wl.nheads, "headdim": wl.headdim,
                   "dstate": wl.dstate, "ngroups": wl.ngroups, "chunk_size": wl.chunk_size,
                   "split_len": split_len, "parallelism": "single GPU"},
        "tokens_per_s_cold": wl.tokens / (fwd_cold["avg_us"] * 1e-6),
        "hbm_gbs": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": alg_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": roofline,
        "copy_reference": {"gbs": copy_gbs, "bytes": alg_bytes, "timing": "cold",
                           "frac_of_copy": achieved / copy_gbs},
    }
    if not args.no_cpu_baseline and not args.fused:
        print("bench: timing the fp64 CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
