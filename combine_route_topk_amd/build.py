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

SOURCES = ["api.hip", "route_topk.hip", "layout.hip", "permute.hip", "combine.hip", "regroup.hip", "fp8.hip", "expert.hip", "floor.hip", "route_layout.hip"]
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


def resource_usage(sources=None):
    """Per-kernel resources the compiler reports for gfx950 (VGPRs, AGPRs,
    SGPRs, LDS bytes, waves per SIMD), as (source, kernel, fields) rows."""
    import re
    rows = []
    for src in sources or SOURCES:
        cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", os.devnull,
               "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        cur = None
        for line in r.stderr.splitlines():
            m = re.search(r"remark: +Function Name: (\S+)", line)
            if m:
                cur = {"kernel": m.group(1)}
                rows.append((src, cur))
                continue
            m = re.search(r"remark: +([A-Za-z ]+?)(?: \[[^]]*\])?: (\d+)", line)
            if m and cur is not None:
                cur[m.group(1).strip()] = int(m.group(2))
    return rows


def _demangle(names):
    r = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    return r.stdout.splitlines() if r.returncode == 0 else names


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        rows = resource_usage()
        names = _demangle([f["kernel"] for _, f in rows])
        print("| source | kernel | VGPRs | AGPRs | SGPRs | LDS bytes | waves per SIMD |")
        print("|---|---|---|---|---|---|---|")
        for (src, f), name in zip(rows, names):
            name = name.replace("moe::(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            print(f"| {src} | `{name}` | {f.get('VGPRs')} | {f.get('AGPRs')} | {f.get('TotalSGPRs')} | "
                  f"{f.get('LDS Size')} | {f.get('Occupancy')} |")
    else:
        print(build(verbose=True))
