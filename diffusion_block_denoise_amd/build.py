"""Build libdllm.so (HIP kernels for gfx950 + host runtime + C ABI) in-tree with hipcc.

Usage: ``python -m diffusion_block_denoise_amd.build`` (or ``build()`` from Python).
Always recompiles every source.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build", "obj")
LIB = os.path.join(PKG, "libdllm.so")

ARCH = "gfx950"
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             # no packed fp32 instructions in any kernel
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]
SOURCES = ["gemm.hip", "attention.hip", "misc.hip", "scratch.hip", "dllm.cpp"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _quiet(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature flag; that warning is harmless.
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l
                     and "is not a recognized feature for this target" not in l)


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(OBJ, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        cmd = [cc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT, text=True)))
    objs = []
    failed = []
    for src, obj, pr in procs:
        out, _ = pr.communicate()
        out = _quiet(out)
        if out.strip():
            print(out, file=sys.stderr)
        if pr.returncode:
            failed.append(src)
        objs.append(obj)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
