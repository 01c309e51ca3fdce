"""A host-sanitized build of libbsf8 for the CPU tests.

The host C++ (the validator, the weight handle, the ABI layer and the
safetensors header reader) is compiled with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer; the kernel translation units are linked in from
the regular build unchanged (their device code is not instrumented).  The
result is a library with the same exports, loaded through the binding by
setting BSF8_LIBRARY, in a Python process that has the sanitizer runtimes
preloaded.  CPU only: nothing here runs on a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp8_linear_amd", "csrc")
REGULAR = os.path.join(ROOT, "_build")
OUT = os.path.join(ROOT, "_build", "host_sanitized")
HOST_SOURCES = ["bsf8_host.cpp", "bsf8_inspect.cpp"]
KERNEL_OBJECTS = ["bsf8_quant.o", "bsf8_w8a16.o", "bsf8_w8a8.o", "bsf8_dense.o", "bsf8_stream.o"]
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def runtimes():
    """Paths of g++'s ASan and UBSan shared runtimes, or None when they are missing."""
    out = []
    for lib in ("libasan.so", "libubsan.so"):
        r = subprocess.run(["g++", f"-print-file-name={lib}"], capture_output=True, text=True)
        p = os.path.realpath(r.stdout.strip()) if r.returncode == 0 else ""
        if not p or not os.path.exists(p):
            return None
        out.append(p)
    return out


def build() -> str:
    """Compile the host sources sanitized and link them with the regular kernel objects."""
    if shutil.which("g++") is None:
        raise RuntimeError("g++ is not available")
    if not all(os.path.exists(os.path.join(REGULAR, o)) for o in KERNEL_OBJECTS):
        from block_scaled_fp8_linear_amd import build as regular
        regular.build()
    os.makedirs(OUT, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OUT, src.replace(".cpp", ".o"))
        cmd = (["g++", "-std=c++17", "-O1", "-g", "-fPIC"] + SAN +
               ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                "-c", os.path.join(CSRC, src), "-o", obj])
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr}")
        objs.append(obj)
    lib = os.path.join(OUT, "libbsf8.so")
    cmd = (["g++", "-shared"] + SAN + ["-o", lib] + objs + [os.path.join(REGULAR, o) for o in KERNEL_OBJECTS] +
           ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"{' '.join(cmd)}\n{r.stderr}")
    return lib
