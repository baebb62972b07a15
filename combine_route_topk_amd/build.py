"""Build libmoe_ep.so in-tree with hipcc for gfx950.

Every HIP source is compiled with packed-FP32 instruction selection turned
off (plain float code must not be lowered to v_pk_{add,mul,fma}_f32); the
host pass warns that it does not know that feature, which is harmless.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libmoe_ep.so")

SOURCES = ["api.hip", "route_topk.hip", "layout.hip", "permute.hip", "combine.hip", "regroup.hip", "fp8.hip", "expert.hip", "floor.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed: {' '.join(cmd)}")
    # drop the host pass's note about the device-only feature
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if msg.strip() and verbose:
        sys.stderr.write(msg + "\n")


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libmoe_ep.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
