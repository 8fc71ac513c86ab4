"""Sanitizer builds of the host code (CPU only).

* The C ABI's host side (ssd_api.cpp: validation, the split planner, the
  workspace layout and every launch's arguments), compiled host-only with
  AddressSanitizer and UndefinedBehaviorSanitizer and linked with stub
  launchers that read and write every byte each kernel would
  (tests/host_sanitize/stub_launchers.cpp; they also answer the planner's
  HIP device queries as a host without a GPU, so no device runtime is
  linked), driven through every entry point
  with host buffers of exactly the documented sizes and through the error
  paths (tests/host_sanitize/abi_driver.c).
* The fp64 C oracle under the same sanitizers, on small problems with
  identities that hold exactly in the recurrence
  (tests/host_sanitize/oracle_driver.c).

The host code is also built with every local variable pattern-initialised,
so that an argument-block field the API forgets to set reaches a stub as a
wild pointer instead of a lucky zero.  The device code is not instrumented:
each of these flags reaches the host compiler only.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
CSRC = os.path.join(ROOT, "ssd_chunked_scan_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
LLVM = "/opt/rocm/lib/llvm/bin"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]

pytestmark = pytest.mark.skipif(not (os.path.exists(os.path.join(LLVM, "clang")) and shutil.which("hipcc")
                                     or os.path.exists("/opt/rocm/bin/hipcc")),
                                reason="needs the ROCm toolchain")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _hipcc_host(src, obj):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    host_san = []
    # every local starts as a 0xaa pattern, so that a field of an argument
    # block left unset becomes a wild pointer the stubs write through
    for f in SAN + ["-ftrivial-auto-var-init=pattern"]:
        host_san += ["-Xarch_host", f]
    _run([hipcc, "--offload-arch=gfx950", "--cuda-host-only", "-x", "hip", "-std=c++17", "-O1", "-g",
          *host_san, "-I", CSRC, "-I", INCLUDE, "-c", src, "-o", obj])


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    api, stubs, drv = (str(tmp_path / n) for n in ("api.o", "stubs.o", "drv.o"))
    _hipcc_host(os.path.join(CSRC, "ssd_api.cpp"), api)
    _hipcc_host(os.path.join(HERE, "stub_launchers.cpp"), stubs)
    _run([os.path.join(LLVM, "clang"), "-std=c11", "-O1", "-g", *SAN, "-I", INCLUDE, "-c",
          os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([os.path.join(LLVM, "clang++"), *SAN, drv, api, stubs, "-o", exe])
    r = _run([exe], env=_env(), timeout=600)
    assert "all checks passed" in r.stdout, r.stdout + r.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run([os.path.join(LLVM, "clang"), "-std=c11", "-O1", "-g", *SAN,
          os.path.join(ROOT, "oracle", "ssd_oracle.c"), os.path.join(HERE, "oracle_driver.c"), "-lm",
          "-o", exe])
    r = _run([exe], env=_env(), timeout=600)
    assert "all checks passed" in r.stdout, r.stdout + r.stderr
