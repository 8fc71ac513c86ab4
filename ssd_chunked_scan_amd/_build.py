"""Build libssd.so (the C-ABI library with the gfx950 kernels) in-tree.

    python -m ssd_chunked_scan_amd._build      # or __graft_entry__.build()

Every source under csrc/ is compiled by hipcc for gfx950 only, in parallel,
then linked into ssd_chunked_scan_amd/libssd.so.  Packed-fp32 instructions
are disabled in device code (-packed-fp32-ops), and so is floating-point
contraction (-ffp-contract=off): the kernels write every FMA they want as
fmaf, and the segsum relies on each term being rounded before it is added.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libssd.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", CSRC, "-I", INCLUDE,
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the gfx950 kernels cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(hipcc: str, src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *COMMON_FLAGS, "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc, *COMMON_FLAGS, "-x", "hip", "-c", src, "-o", obj]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"  {os.path.basename(src)}: {time.time() - t:.1f}s", file=sys.stderr)
    return obj


_REG = re.compile(r"([vas])\[(\d+):(\d+)\]|\b([vas])(\d+)\b")

# v_mfma_f32_16x16x32_bf16 on gfx950 with a VGPR destination: a VALU, memory
# or MFMA A/B read of its result needs 8 wait states on the hardware (measured:
# the first result registers are valid after 7, the last after 8).  Results
# read as the accumulator of a following MFMA (same registers) need none, and
# v_accvgpr_read of an AGPR destination is interlocked (measured: valid at 0).
MFMA_READ_WAIT_STATES = 8
# v_mfma_f32_16x16x4_f32 takes twice the passes (8): a result read needs
# passes + 3 wait states.
MFMA_READ_WAIT_STATES_BY_OP = {"v_mfma_f32_16x16x4_f32": 11}


def _regs(text: str):
    out = set()
    for m in _REG.finditer(text):
        if m.group(1):
            f, a, b = m.group(1), int(m.group(2)), int(m.group(3))
        else:
            f, a, b = m.group(4), int(m.group(5)), int(m.group(5))
        if f in ("v", "a"):
            out.update((f, r) for r in range(a, b + 1))
    return out


def _parse_functions(asm_text: str):
    """Split assembly into functions: lists of (kind, text) with kind 'label'
    or 'ins'."""
    funcs, cur = [], None
    for raw in asm_text.splitlines():
        if "ssd lookahead wait" in raw and cur is not None:
            cur.append(("mark", "ssd lookahead wait"))   # see vmem_lds_sync_lookahead
            continue
        if "ssd touch wait" in raw and cur is not None:
            cur.append(("mark", "ssd touch wait"))       # see vmem_lds_sync_touch
            continue
        if "ssd touch" in raw and cur is not None:
            cur.append(("mark", "ssd touch"))            # see l2_touch
            continue
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") and not line.startswith("."):
            cur = []
            funcs.append((line[:-1], cur))
            continue
        if cur is None:
            continue
        if line.endswith(":") and line.startswith(".LBB"):
            cur.append(("label", line[:-1]))
        elif not line.startswith("."):
            cur.append(("ins", line))
    return funcs


def check_mfma_result_reads(asm_text: str, where: str) -> int:
    """Follow every path (fall-through and branch targets) from each MFMA and
    fail if an instruction reads its result registers, other than as the
    accumulator of the next MFMA, within MFMA_READ_WAIT_STATES wait states."""
    n = 0
    for fname, items in _parse_functions(asm_text):
        labels = {t: i for i, (k, t) in enumerate(items) if k == "label"}
        for i, (kind, text) in enumerate(items):
            if kind != "ins" or not text.startswith("v_mfma"):
                continue
            n += 1
            ops = [o.strip() for o in text.split(None, 1)[1].split(",")]
            dst = _regs(ops[0])
            need = MFMA_READ_WAIT_STATES_BY_OP.get(text.split()[0], MFMA_READ_WAIT_STATES)
            stack, seen = [(i + 1, 0)], set()
            while stack:
                j, ws = stack.pop()
                while j < len(items) and ws < need:
                    if (j, ws) in seen:
                        break
                    seen.add((j, ws))
                    k2, t2 = items[j]
                    if k2 in ("label", "mark"):
                        j += 1
                        continue
                    op = t2.split()[0]
                    rest = t2.split(None, 1)[1] if " " in t2 else ""
                    if op.startswith("s_nop"):
                        ws += int(rest) + 1
                        j += 1
                        continue
                    parts = [p.strip() for p in rest.split(",")] if rest else []
                    if op.startswith("v_mfma"):
                        srcab = _regs(",".join(parts[1:3]))
                        if dst & srcab:
                            raise RuntimeError(f"{where}: {fname}: MFMA result read as an A/B "
                                               f"operand after {ws} wait states: {text} -> {t2}")
                        if _regs(parts[0]) == dst:
                            break          # same accumulator: result consumed in place
                    elif op.startswith("v_accvgpr_read"):
                        pass               # interlocked read of an AGPR result
                    elif op.startswith(("v_", "ds_", "global_", "buffer_", "flat_", "scratch_")):
                        srcs = _regs(",".join(parts[1:])) if op.startswith("v_") else _regs(rest)
                        if op.startswith(("global_load", "buffer_load", "ds_read", "scratch_load",
                                          "flat_load")):
                            srcs = _regs(",".join(parts[1:]))
                        if dst & srcs:
                            raise RuntimeError(f"{where}: {fname}: MFMA result read after only {ws} "
                                               f"wait states: {text} -> {t2}")
                    if op in ("s_branch", "s_setpc_b64", "s_endpgm"):
                        if op == "s_branch" and rest in labels:
                            stack.append((labels[rest], ws + 1))
                        break
                    if op.startswith("s_cbranch") and rest in labels:
                        stack.append((labels[rest], ws + 1))
                    ws += 1
                    j += 1
    return n


_VMEM = ("global_load", "global_store", "buffer_load", "buffer_store", "scratch_load",
         "scratch_store", "flat_load", "flat_store", "global_atomic", "buffer_atomic")
_WAIT_VM = re.compile(r"s_waitcnt\s+vmcnt\((\d+)\)")
VMCNT_MAX = 63


def check_counted_barrier_waits(asm_text: str, where: str) -> int:
    """A barrier whose wait leaves K > 0 vector-memory operations in flight is
    only correct if the K most recent ones are not direct-to-LDS loads (whose
    data the barrier publishes).  Walk back from every such wait over
    straight-line code: K ordinary vector-memory operations must come before
    any global_load_lds, label or branch."""
    n = 0
    for fname, items in _parse_functions(asm_text):
        for i, (kind, text) in enumerate(items):
            if kind != "ins":
                continue
            m = _WAIT_VM.search(text)
            # vmcnt(0): waits for all; vmcnt(63), the field's maximum on gfx9,
            # waits for none (the wait is for other counters)
            if not m or int(m.group(1)) in (0, VMCNT_MAX):
                continue
            nxt = next((t for k, t in items[i + 1:] if k == "ins"), "")
            if not nxt.startswith("s_barrier"):
                continue
            need, j = int(m.group(1)), i - 1
            n += 1
            # the marker of vmem_lds_sync_lookahead / vmem_lds_sync_touch:
            # before the wait, with no label or vector-memory operation in
            # between
            marked, touch, q = False, False, i - 1
            while q >= 0 and items[q][0] != "label":
                if items[q][0] == "mark" and items[q][1] in ("ssd lookahead wait", "ssd touch wait"):
                    marked = True
                    touch = items[q][1] == "ssd touch wait"
                    break
                if items[q][0] == "ins" and items[q][1].startswith(_VMEM):
                    break
                q -= 1
            if touch:
                # the K newest vector-memory operations, on straight-line code,
                # may be stores, ordinary loads or L2 prefetches; a
                # direct-to-LDS load among them must be a prefetch: the
                # nearest vector-memory item before it is its touch marker
                while need > 0:
                    if j < 0 or items[j][0] == "label":
                        raise RuntimeError(f"{where}: {fname}: touch wait '{text}' reaches a label "
                                           f"before {m.group(1)} vector-memory operations")
                    k2, t = items[j]
                    if k2 == "ins":
                        op = t.split()[0] if t.split() else ""
                        if op.startswith(("s_branch", "s_cbranch", "s_setpc")):
                            raise RuntimeError(f"{where}: {fname}: touch wait '{text}' reaches a "
                                               f"branch before {m.group(1)} vector-memory operations")
                        if op.startswith(("global_load_lds", "buffer_load_lds")):
                            q2 = j - 1
                            while q2 >= 0 and items[q2][0] == "ins" and not items[q2][1].startswith(_VMEM):
                                q2 -= 1
                            if not (q2 >= 0 and items[q2] == ("mark", "ssd touch")):
                                raise RuntimeError(f"{where}: {fname}: touch wait '{text}' would leave "
                                                   f"a direct-to-LDS tile load in flight: {t}")
                            need -= 1
                        elif op.startswith(_VMEM):
                            need -= 1
                    j -= 1
                continue
            if marked:
                # run-ahead tile loads: the K newest vector-memory operations
                # must be exactly direct-to-LDS loads on straight-line code
                # (the tile the barrier publishes was issued before them)
                while need > 0:
                    if j < 0 or items[j][0] == "label":
                        raise RuntimeError(f"{where}: {fname}: lookahead wait '{text}' reaches a "
                                           f"label before {m.group(1)} direct-to-LDS loads")
                    t = items[j][1]
                    op = t.split()[0] if t.split() else ""
                    if op.startswith(("s_branch", "s_cbranch", "s_setpc")):
                        raise RuntimeError(f"{where}: {fname}: lookahead wait '{text}' reaches a "
                                           f"branch before {m.group(1)} direct-to-LDS loads")
                    if op.startswith(("global_load_lds", "buffer_load_lds")):
                        need -= 1
                    elif op.startswith(_VMEM):
                        raise RuntimeError(f"{where}: {fname}: lookahead wait '{text}' would leave "
                                           f"an ordinary vector-memory operation in flight: {t}")
                    j -= 1
                continue
            while need > 0:
                if j < 0 or items[j][0] == "label":
                    raise RuntimeError(f"{where}: {fname}: counted barrier wait '{text}' reaches "
                                       f"a label before {m.group(1)} vector-memory operations")
                t = items[j][1]
                op = t.split()[0]
                if op.startswith("global_load_lds") or op.startswith("buffer_load_lds"):
                    raise RuntimeError(f"{where}: {fname}: counted barrier wait '{text}' would leave "
                                       f"a direct-to-LDS load in flight: {t}")
                if op.startswith(("s_branch", "s_cbranch", "s_setpc")):
                    raise RuntimeError(f"{where}: {fname}: counted barrier wait '{text}' reaches "
                                       f"a branch before {m.group(1)} vector-memory operations")
                if op.startswith(_VMEM):
                    need -= 1
                j -= 1
    return n


def _asm_check(hipcc: str, src: str) -> int:
    cmd = [hipcc, *COMMON_FLAGS, "-S", "--cuda-device-only", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed on {src}:\n{r.stderr}")
    check_counted_barrier_waits(r.stdout, os.path.basename(src))
    return check_mfma_result_reads(r.stdout, os.path.basename(src))


def build(verbose: bool = True, jobs: int = 0) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or max(1, (os.cpu_count() or 4))
    t = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, hipcc, s, verbose) for s in srcs]
        chk = [ex.submit(_asm_check, hipcc, s) for s in srcs if s.endswith(".hip")]
        objs = [f.result() for f in futs]
        n_mfma = sum(f.result() for f in chk)
    if verbose:
        print(f"  checked {n_mfma} MFMA instructions: every read of a result is at least "
              f"{MFMA_READ_WAIT_STATES} wait states (fp32 MFMA: 11) away on every path", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
