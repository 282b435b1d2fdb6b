"""Build the C-ABI library libecw.so in-tree for gfx950 (hipcc; host part with g++)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libecw.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -amdgpu-kernarg-preload-count: the first 11 dwords of kernel arguments arrive in
# scalar registers (k_decode's block-to-tensor fields); code objects keep a
# load-based entry for firmware without preloading.
HIP_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mcode-object-version=5", "-mllvm", "-amdgpu-kernarg-preload-count=11", "-Wall", "-Wno-unused-result",
             f"-I{ROOT}"]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", f"-I{ROOT}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {cmd[0]} ... ({r.returncode})")
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)


def build(verbose: bool = False) -> str:
    bdir = os.path.join(HERE, "_build")
    os.makedirs(bdir, exist_ok=True)
    host_o = os.path.join(bdir, "ecw_host.o")
    _run(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, "ecw_host.cpp"), "-o", host_o], verbose)
    objs = [host_o]
    for src in ("ecw_kernels.hip", "ecw_probes.hip"):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
