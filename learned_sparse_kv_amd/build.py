"""Build liblsa.so (HIP, gfx950) in-tree with hipcc.

    python -m learned_sparse_kv_amd.build [--jobs N]

Every source is compiled on each call (the "does it build" check), objects
go to _build/, and the shared library lands next to this file.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblsa.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["score_select.hip", "score_sigmoid.hip", "policy.hip", "grow.hip", "refine_topk.hip", "refine_band.hip", "attn_decode.hip", "gather.hip",
           "api.cpp", "pool.cpp", "step64.cpp", "timing.cpp"]

# -ffp-contract=off + explicit fmaf: the scores that decide selections follow
# one written fp32 order; denormals are kept; packed fp32 ops are disabled.
HIPFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-Wall", "-Wno-unused-function",
            "-I" + os.path.join(ROOT, "include")]


def hipcc() -> str:
    return shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *HIPFLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    print(build(ap.parse_args().jobs))
