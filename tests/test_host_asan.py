"""Host-side sanitizer build of the C ABI (CPU only, no GPU).

Every .hip source is compiled for the host only (``--cuda-host-only``: the kernels become
launch stubs and no device code is built) with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code, linked into a throw-away library, and driven by ``host_asan/abi_driver.cpp``,
which calls each entry point of ``include/moe.h`` on the paths that return before any HIP call:
argument validation, workspace sizing and the capacity helper.  A heap overflow, a
use-after-free, signed overflow in the workspace arithmetic or a leak fails the test.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_17_amd", "csrc")
INC = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not installed")
def test_abi_validation_under_host_sanitizers(tmp_path):
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        rc, out = _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-fno-omit-frame-pointer", *SAN, "-I" + INC, "-I" + CSRC, "-c", src, "-o", obj])
        assert rc == 0, f"{os.path.basename(src)}:\n{out[-3000:]}"
        return obj

    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libmoe_asan.so")
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *SAN, "-o", lib, *objs])
    assert rc == 0, out[-3000:]
    exe = str(tmp_path / "abi_driver")
    rc, out = _run([CLANG, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-I" + INC,
                    os.path.join(ROOT, "tests", "host_asan", "abi_driver.cpp"), "-o", exe, lib,
                    "-Wl,-rpath," + str(tmp_path), "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"])
    assert rc == 0, out[-3000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    rc, out = _run([exe], env=env, timeout=300)
    assert rc == 0, out[-4000:]
    assert "failed" in out and ", 0 failed" in out, out[-2000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
