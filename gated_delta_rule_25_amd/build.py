"""Build libgdn2.so (the C-ABI library and its gfx950 kernels) in-tree with hipcc.

Usage: python -m gated_delta_rule_25_amd.build   (or call build()).
Each source is compiled separately (in parallel) and linked into one shared library next to
this file. Packed-fp32 instruction selection is switched off for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn2.so")
SOURCES = ["gdn2_api.cpp", "recurrent.hip", "chunk.hip", "chunk_fused.hip", "chunk_split.hip", "chunk_varlen.hip", "chunk_bwd.hip", "rmsnorm.hip", "sdm.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libgdn2.so)")


def common_flags() -> list[str]:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-parameter", "-Wno-unused-variable",
            "-I", os.path.join(HERE, "..", "include")]


def build(verbose: bool = False, jobs: int | None = None) -> str:
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        path = os.path.join(CSRC, src)
        obj = os.path.join(obj_dir, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [cc, *common_flags(), *lang, "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs or min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
