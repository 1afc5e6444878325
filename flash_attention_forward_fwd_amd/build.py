"""Build libfa.so (the gfx950 HIP kernels + the C-ABI front end) in-tree.

    python -m flash_attention_forward_fwd_amd.build

hipcc cross-compiles for gfx950 without a GPU present.  Objects go to
_build/ at the repository root; the shared library lands next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

SOURCES = ["fa_api.cpp", "fa_prefill.hip", "fa_decode.hip", "fa_backward.hip"]

# Packed fp32 VALU forms are kept out of the generated code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err)


def build(verbose: bool = False, jobs: int | None = None, defines=(), out: str | None = None,
          objdir: str | None = None) -> str:
    """Compile every source and link libfa.so; returns the library path.

    `defines` (e.g. ["FA_PREFILL_WAVES=4"]) and `out` build a variant of the
    library elsewhere for A/B measurements; the default is the in-tree build."""
    cc = hipcc()
    objdir = objdir or BUILD
    out = out or LIB
    os.makedirs(objdir, exist_ok=True)
    objs, cmds = [], []
    dflags = [f"-D{d}" for d in defines]
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc, *COMMON, *DEVICE_FLAGS, *dflags, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = out + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
