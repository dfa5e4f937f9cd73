"""Build the HIP libraries in-tree for gfx950 with hipcc.

* ``libmxmoe.so``        -- the MoE layer (C ABI in include/mxmoe.h)
* ``libmxmoe_inputs.so`` -- GPU twin of the seeded input generator

Usage: ``python -m mxfp4_expert_grouped_amd.build`` (always recompiles).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-function", "-Wno-unused-variable",
    "-fno-gpu-flush-denormals-to-zero",
    # packed-fp32 VALU forms stay off: plain float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

LIBS = {
    "libmxmoe.so": ["api.cpp", "kernels_route.hip", "kernels_gemm.hip", "kernels_pack.hip",
                    "kernels_tail.hip"],
    "libmxmoe_inputs.so": ["gen_inputs.hip"],
}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> dict:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for lib, srcs in LIBS.items():
        for s in srcs:
            src = os.path.join(CSRC, s)
            obj = os.path.join(BUILD, s + ".o")
            jobs.append((src, obj))

    def compile_one(job):
        src, obj = job
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        _run([HIPCC] + FLAGS + lang + ["-c", src, "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(compile_one, jobs))
    out = {}
    for lib, srcs in LIBS.items():
        objs = [os.path.join(BUILD, s + ".o") for s in srcs]
        target = os.path.join(PKG, lib)
        tmp = target + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs)
        os.replace(tmp, target)
        out[lib] = target
        if verbose:
            print("built", target)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
