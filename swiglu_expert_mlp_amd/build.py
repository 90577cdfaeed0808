"""Build libmoe.so (HIP, gfx950) in-tree with hipcc.

    python -m swiglu_expert_mlp_amd.build

Every HIP source is compiled with the packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops): the compiler otherwise
forms v_pk_* fp32 ops from ordinary float code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmoe.so")
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

SOURCES = ["moe_api.cpp", "route.hip", "prep.hip", "gemm_bf16.hip", "gemm_mxfp8.hip",
           "finalize.hip", "pack.hip"]
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


# per-file code generation options
FILE_FLAGS = {}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [_hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS + FILE_FLAGS.get(src, [])
    if src.endswith(".cpp"):
        cmd = [_hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # keep warnings visible, drop the host pass's note about the device-only feature
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if msg.strip():
        print(f"[{src}]\n{msg}", file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-o", tmp] + objs + [f"--offload-arch={ARCH}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
