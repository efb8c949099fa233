"""Compile the HIP library libmoe_w4a16.so for gfx950 (in-tree).

Usage: python w4a16_routed_expert_router_amd/build_lib.py  (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_w4a16.so")

SOURCES = ["api.hip", "router.hip", "group.hip", "expert_gemv.hip", "expert_mfma.hip", "expert_stream.hip",
           "decode_fused.hip", "decode_spec.hip", "debug.hip", "policy.cpp", "trace_analysis.cpp"]

HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++20",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed FP32 instructions are never emitted
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
    return res.returncode


def build(verbose: bool = False) -> str:
    """Compiles every source to an object in parallel (in-tree, under
    _build/), then links libmoe_w4a16.so.  Always recompiles."""
    from concurrent.futures import ThreadPoolExecutor
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    missing = [s for s in srcs if not os.path.exists(s)]
    if missing:
        raise RuntimeError(f"missing sources: {missing}")
    obj_dir = os.path.join(ROOT, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    # policy.cpp and trace_analysis.cpp have no device code; hipcc compiles them as host C++.
    jobs = []
    for src in srcs:
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        jobs.append((obj, [hipcc(), *HIP_FLAGS, *inc, "-c", src, "-o", obj]))
    workers = max(1, min(len(jobs), len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        rcs = list(ex.map(lambda j: _run(j[1], verbose), jobs))
    if any(rcs):
        raise RuntimeError("hipcc failed compiling the library sources")
    tmp = LIB + ".tmp"
    if _run([hipcc(), *HIP_FLAGS, "-shared", "-o", tmp, *[j[0] for j in jobs], "-lpthread"], verbose):
        raise RuntimeError("hipcc failed linking libmoe_w4a16.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
