"""Compile the HIP sources of the MoE-layer library for gfx950 with hipcc.

Produces int4_quantized_expert_amd/libmoe_layer.so next to this file.  Every
call recompiles (objects go to a temporary build directory), so a stale library
is never picked up after a source change.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe_layer.so")
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off",                       # only explicit fmaf() fuses
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build the library")
    return path


def _compile(src: str, obj: str) -> None:
    cmd = [hipcc(), *HIP_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stdout}\n{r.stderr}")


def build_library(out: str = LIB, sources_dir: str = CSRC, jobs: int = 8) -> str:
    srcs = sorted(os.path.join(sources_dir, f) for f in os.listdir(sources_dir) if f.endswith(".hip"))
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
            list(ex.map(_compile, srcs, objs))
        tmp_out = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build_library())
