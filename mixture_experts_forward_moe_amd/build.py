"""Build libmoe_mi355x.so in-tree with hipcc for gfx950 (no JIT, no torch)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe_mi355x.so")
SOURCES = ["sort.hip", "gemm.hip", "gemm_wide.hip", "gemm_mx.hip", "gemm_mxw.hip", "gemm_nvfp4.hip",
           "decode.hip", "finalize.hip", "capi.cpp", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # keep packed fp32 instructions out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# per-source extras: the decode kernel's thread-0 counter claims must stay
# plain atomics (a wavefront-aggregated rewrite waits for the result at once)
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        msg = "\n".join(l for l in out.splitlines() if "is not a recognized feature" not in l)
        if p.returncode != 0:
            failed.append(src)
            sys.stderr.write(msg + "\n")
        elif verbose and msg.strip():
            sys.stderr.write(msg + "\n")
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
