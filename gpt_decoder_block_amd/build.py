"""Build the gfx950 HIP library `libgdb.so` in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only (one object per file, in
parallel), then linked into a shared library next to this file.  Packed fp32
instructions are disabled on the device side (-packed-fp32-ops off).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgdb.so")
BUILD = os.path.join(HERE, "_build")
ARCH = "gfx950"
SOURCES = ["elementwise.hip", "gemm.hip", "attention.hip", "decode.hip", "optim.hip", "extras.hip", "fp8.hip", "order.hip",
           "api.cpp"]
# per-file code-generation options: the attention kernels run their softmax on
# the MFMA results, so those stay in VGPRs (no AGPR round trips)
EXTRA = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-result", "-I", os.path.join(os.path.dirname(HERE), "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + _flags() + EXTRA.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return obj


def build_sanitized(verbose: bool = False) -> str:
    """_build_san/libgdb_san.so: the host code (argument validation, workspace carving,
    launch logic in api.cpp) built with AddressSanitizer and
    UndefinedBehaviorSanitizer, the device code as in the normal build.  Load
    it with GDB_LIB=<path> and the clang ASan runtime preloaded."""
    san = os.path.join(HERE, "_build_san")
    os.makedirs(san, exist_ok=True)
    if any(not os.path.exists(os.path.join(BUILD, s + ".o")) for s in SOURCES if s != "api.cpp"):
        build()  # the device objects of the normal build
    objs = []
    for src in SOURCES:
        obj = os.path.join(san if src == "api.cpp" else BUILD, os.path.basename(src) + ".o")
        if src == "api.cpp":
            cmd = [hipcc()] + _flags() + ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                                          "-fsanitize=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                                          "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
        objs.append(obj)
    out = os.path.join(san, "libgdb_san.so")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-fsanitize=address", "-fsanitize=undefined",
           "-shared-libsan", "-o", out] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    if verbose:
        print(f"built {out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
