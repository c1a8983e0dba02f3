"""Build the gfx950 HIP library libmoe_mi355x.so in-tree with hipcc.

Each .hip source under csrc/ is compiled to an object in parallel, then linked
into one shared library next to this file.  Runs on a machine without a GPU
(hipcc cross-compiles for gfx950).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU instructions.
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-variable",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


# Per-source extra flags.  grouped_gemm.hip: the atomic that draws a dynamically scheduled
# block's next tile runs on one lane and its result is used only after the tile's epilogue; the
# atomic optimizer would rewrite it into a wave-wide form that reads the result back at once.
FILE_FLAGS = {"grouped_gemm.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link LIB; returns its path.  Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    # a kernel whose host stub the compiler dropped shows up as an undefined symbol
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in nm.stdout.splitlines() if "3moe" in l]
    if missing:
        raise RuntimeError("library has undefined kernel symbols: " + ", ".join(missing[:5]))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
