"""Build libbsf8.so for gfx950 with hipcc (in-tree).

    python -m block_scaled_fp8_linear_amd.build [--jobs N] [--asm]

Every source is compiled for gfx950 only.  Packed FP32 instructions are
switched off on the device side (``-packed-fp32-ops``): the kernels are written
with scalar and vector F32 code and do not rely on them.
"""
from __future__ import annotations

import argparse
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
LIB = os.path.join(PKG, "libbsf8.so")

SOURCES = ["bsf8_host.cpp", "bsf8_inspect.cpp", "bsf8_quant.hip", "bsf8_w8a16.hip", "bsf8_w8a8.hip", "bsf8_dense.hip",
           "bsf8_stream.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libbsf8)")


def common_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def compile_one(src: str, asm: bool) -> str:
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    if asm and src.endswith(".hip"):
        cmd += ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{msgs}")
    if msgs.strip():
        sys.stderr.write(msgs + "\n")
    return obj


def build(jobs: int = 4, asm: bool = False) -> str:
    with cf.ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, asm), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    ap.add_argument("--asm", action="store_true", help="keep the device assembly under _build/")
    a = ap.parse_args(argv)
    print(build(a.jobs, a.asm))


if __name__ == "__main__":
    main()
