"""Build the gfx950 shared library libspec.so in-tree with hipcc.

Every HIP source under csrc/ is compiled for gfx950 only, with packed-fp32
instruction selection disabled, and linked with the host-side ABI layer.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libspec.so")
OBJ = os.path.join(HERE, "_build")
SOURCES = ["abi.cpp", "timing.cpp", "syrk.hip", "gram.hip", "small_eig.hip", "descriptors.hip", "postproc.hip", "eig_large.hip",
           "project.hip", "screen.hip", "sliding.hip", "small_eigh.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
         "-Wno-unused-parameter"]
DEVICE_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(OBJ, src + ".o")
    cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = DEVICE_FLAGS
    else:
        cmd[1:1] = ["-D__HIP_PLATFORM_AMD__"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip():
        sys.stderr.write(out + "\n")
    return obj


def build() -> str:
    os.makedirs(OBJ, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
