"""Build libglowq.so (HIP, gfx950) in-tree with hipcc.

    python -m rank_error_compensation_amd.build        # or __graft_entry__.build()

Every translation unit is compiled for gfx950 only, with packed-fp32 instruction selection
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops) and without the compiler's
wave-aggregation of atomics (-mllvm -amdgpu-atomic-optimizer-strategy=None): the kernels issue
their atomics from one lane and read the returned value much later, which the aggregated form
(it broadcasts the result at once) would turn into a wait for every load in flight.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libglowq.so")
PROBE_LIB = os.path.join(PKG, "libglowq_probe.so")

SOURCES = ["format.hip", "proj.hip", "decode.hip", "prefill.hip", "w4a8.hip", "mx8.hip", "moe.hip", "score.hip", "moment.hip", "solve.hip",
           "abi.cpp"]
PROBE_SOURCES = ["probe.hip", "handoff_probe.hip"]  # measurement and protocol probes, a library of their own
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libglowq)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
            "-I", INCLUDE, "-I", CSRC, "-Wno-unused-command-line-argument"]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + common_flags() + list(extra)
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, extra), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
