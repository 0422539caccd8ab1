"""Build libkvq.so (HIP C++ for gfx950) in-tree with hipcc.

Sources on the codec path are compiled with -ffp-contract=off (the codec's
binary32 steps must stay separate multiplies and adds to reproduce the oracle
bit for bit); packed-fp32 instruction generation is disabled everywhere.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")
TIMELINE_LIB = os.path.join(PKG, "libkvq_timeline.so")

SOURCES = ["kvq_api.hip", "kvq_quant.hip", "kvq_attn.hip", "kvq_attn_fast.hip", "kvq_attn_m128.hip", "kvq_rfft.hip"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


# The MFMA decode kernel is checked against the oracle within a tolerance, so it
# may fuse multiply-adds; every file on the bit-exact codec path may not.  Its LDS
# step counter is bumped by one 64-lane atomic (one lane adds 1), which the atomic
# optimizer would otherwise turn into a per-lane scan loop.
PER_FILE = {"kvq_attn_fast.hip": ["-ffp-contract=fast", "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str, extra=(), tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
    cmd = [HIPCC, *FLAGS, *PER_FILE.get(src, ["-ffp-contract=off"]), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True, timeline: bool = False) -> str:
    """Compile every source and link libkvq.so; with timeline, link libkvq_timeline.so
    instead, whose MFMA decode records per-wavefront clock stamps (KVQ_TIMELINE; the
    other objects are the default build's)."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]

    def comp(src):
        if timeline and src == "kvq_attn_fast.hip":
            return _compile(src, ("-DKVQ_TIMELINE",), "_timeline")
        return _compile(src)

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    lib = TIMELINE_LIB if timeline else LIB
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build(timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
