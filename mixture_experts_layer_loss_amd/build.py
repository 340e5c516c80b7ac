"""Build the HIP library ``libmoe.so`` in-tree for gfx950 with hipcc.

    python -m mixture_experts_layer_loss_amd.build        # or build() from Python
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [hipcc, *FLAGS, "-I", os.path.join(os.path.dirname(HERE), "include"), *sources(), "-o", tmp]
    t0 = time.time()
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l]
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB)
    if verbose:
        if msgs:
            print("\n".join(msgs))
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
