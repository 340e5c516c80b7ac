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
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # packed fp32 ops stay off for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# the compiler's per-kernel resource remarks (registers, scratch, LDS), kept in a report beside the
# library; no kernel may use scratch memory (tests/test_abi.py reads the report)
RESOURCE_FLAGS = ["-Rpass-analysis=kernel-resource-usage", "-fno-caret-diagnostics"]
REPORT = os.path.join(HERE, "libmoe.resources.json")


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l]
    return proc.returncode, msgs


def _resources(msgs):
    """Splits the resource remarks off the compiler messages: {function: {field: value}}."""
    res, other, cur = {}, [], None
    for line in msgs:
        if "[-Rpass-analysis=kernel-resource-usage]" not in line:
            other.append(line)
            continue
        body = line.split("remark:", 1)[-1].replace("[-Rpass-analysis=kernel-resource-usage]", "")
        key, _, val = body.strip().partition(":")
        if key == "Function Name":
            cur = res.setdefault(val.strip(), {})
        elif cur is not None and key:
            try:
                cur[key.strip()] = int(val.strip())
            except ValueError:
                cur[key.strip()] = val.strip()
    return res, other


def build(verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), then links the shared library."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    inc = ["-I", os.path.join(os.path.dirname(HERE), "include")]
    tag = f".tmp{os.getpid()}"
    objs = [os.path.join(CSRC, os.path.basename(src)[:-4] + tag + ".o") for src in sources()]
    t0 = time.time()
    jobs = max(1, min(len(objs), int(os.environ.get("MAX_JOBS", "0")) or (os.cpu_count() or 4)))
    with ThreadPoolExecutor(jobs) as pool:
        results = list(pool.map(
            lambda so: _run([hipcc, *FLAGS, *RESOURCE_FLAGS, *inc, "-c", so[0], "-o", so[1]]),
            zip(sources(), objs)))
    resources, msgs = {}, []
    for _, ms in results:
        r, other = _resources(ms)
        resources.update(r)
        msgs += other
    tmp = LIB + tag
    rc = max(r for r, _ in results)
    if rc == 0:
        rc, link_msgs = _run([hipcc, *FLAGS, "-shared", *objs, "-o", tmp])
        msgs += link_msgs
    for o in objs:
        if os.path.exists(o):
            os.remove(o)
    if rc != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    os.replace(tmp, LIB)
    import hashlib
    import json
    with open(LIB, "rb") as fh:
        digest = hashlib.sha256(fh.read()).hexdigest()
    with open(REPORT, "w") as fh:
        json.dump({"library_sha256": digest, "functions": resources}, fh, indent=1, sort_keys=True)
    if verbose:
        if msgs:
            print("\n".join(msgs))
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
