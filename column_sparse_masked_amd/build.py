"""Build libfm.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m column_sparse_masked_amd.build

compiles every csrc/*.hip file with hipcc into _build/ and links
column_sparse_masked_amd/libfm.so.  It always recompiles.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libfm.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["tiles.hip", "fwd.hip", "fwd_fp8.hip", "bwd.hip", "bwd_dq.hip", "bwd_dq_cached.hip", "localize.hip",
           "api.hip"]
ARCH = os.environ.get("FM_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU instructions are turned off for all device code.  The
# atomic optimizer is off: it turns a one-lane atomic with a uniform address
# into a wave-wide one whose result every lane needs at once, which makes the
# kernels wait for their work-queue ticket right where they take it.
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in l]
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(msgs))
    return msgs


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for msgs in ex.map(_run, cmds):
            if verbose and msgs:
                print("\n".join(msgs))
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
