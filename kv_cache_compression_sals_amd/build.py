"""Build libsals.so (HIP kernels for gfx950 + the C ABI) in place, next to this file.

    python -m kv_cache_compression_sals_amd.build [-j N]

hipcc cross-compiles for gfx950 without a GPU. Packed fp32 VALU instructions are disabled
(-packed-fp32-ops); hipcc's host pass warns that it does not know that feature, which is
harmless.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsals.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = [
    "sals_api.cpp",
    "kernels/latent_query.hip",
    "kernels/latent_score.hip",
    "kernels/topk.hip",
    "kernels/select_attend.hip",
    "kernels/select_attend_bf16_d128.hip",
    "kernels/select_attend_bf16_d64.hip",
    "kernels/select_attend_f32_d128.hip",
    "kernels/select_attend_f32_d64.hip",
    "kernels/value.hip",
    "kernels/select_shared.hip",
    "kernels/reconstruct.hip",
    "kernels/project.hip",
    "kernels/compact.hip",
    "kernels/outlier.hip",
    "kernels/quant.hip",
    "kernels/budget.hip",
    "kernels/probe.hip",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libsals.so")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace("/", "_") + ".o")
    cmd = [hipcc()] + COMMON_FLAGS + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 0, verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    # every symbol must resolve at link time (a kernel template whose host stub is missing
    # would otherwise only fail when the library is loaded)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=0)
    build(ap.parse_args().j)
