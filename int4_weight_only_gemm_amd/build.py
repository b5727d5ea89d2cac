"""Builds libw4a16.so in-tree with hipcc for gfx950 (run: python -m int4_weight_only_gemm_amd.build)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "csrc", "w4a16.hip")
OUT = os.path.join(HERE, "libw4a16.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first 14 dwords of each kernel's arguments are preloaded into scalar registers at
    # wave launch (the kernels put what they need before their first load there); code
    # objects keep a scalar-load prologue for firmware without preload
    "-mllvm", "-amdgpu-kernarg-preload-count=14",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *FLAGS, "-I", os.path.join(ROOT, "include"), SOURCE, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libw4a16.so")
    if verbose:
        lines = [l for l in (res.stdout + res.stderr).splitlines() if "not a recognized feature" not in l]
        if lines:
            print("\n".join(lines))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
