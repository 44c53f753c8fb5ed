"""Build the gfx950 HIP library of the MoE layer in-tree: libmoe_mi355x.so.

Usage: python -m mixture_experts_layer_03_amd.build   (or build() from Python)
Every .hip file under csrc/ is compiled for gfx950 and linked into one shared
library next to this file.  Packed-FP32 instruction forms are disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
OUT = os.path.join(HERE, "libmoe_mi355x.so")
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = shutil.which("hipcc") or os.path.join(rocm, "bin", "hipcc")
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build the library)")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    return obj


def _check_isa(src: str) -> list:
    """Device assembly of one source through the inline-asm wait-state check."""
    from mixture_experts_layer_03_amd import isa_check
    cmd = [hipcc(), *HIPCC_FLAGS, "--cuda-device-only", "-S", src, "-o", "-"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stderr[-8000:]}")
    return isa_check.check(r.stdout)


def build(verbose: bool = False) -> str:
    """Compile every source (always), check the wait states around the inline-asm
    copies in the device assembly, and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with ThreadPoolExecutor(max(1, min(2 * len(srcs), os.cpu_count() or 1))) as ex:
        objs = ex.map(_compile, srcs)
        isa = ex.map(_check_isa, srcs)
        objs, isa = list(objs), list(isa)
    bad = [v for vs in isa for v in vs]
    if bad:
        raise RuntimeError("wait-state check of the inline-asm copies failed:\n" + "\n".join(bad[:40]))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
