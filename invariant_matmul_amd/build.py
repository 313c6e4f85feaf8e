"""Build libinvariant_matmul.so (HIP kernels + C ABI) in-tree with hipcc for gfx950.

Usage: ``python -m invariant_matmul_amd.build`` (or ``build()`` from Python).
The library is written next to this file so that it travels with the tree.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libinvariant_matmul.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "gemm_kernels.hip", "gemm_dma.hip", "ozaki.hip", "noalloc.hip"]
# The benchmark's HBM read probe: a library of its own, never linked into the GEMM library.
PROBE_SOURCES = ["hbm_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libimm_hbm_probe.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are kept out of all device code.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


# Device assembly of the DMA kernels, written beside the objects: the tests
# check in it that no instruction touches a register an inline-assembly LDS
# read (whose completion the compiler does not track) will still write.
DMA_ASM = os.path.join(BUILD_DIR, "gemm_dma.gfx950.s")


def _device_asm(src: str, out: str, verbose: bool) -> str:
    cmd = [_hipcc(), *HIP_FLAGS, "-x", "hip", "-S", "--offload-device-only",
           os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc -S failed for {src}:\n{r.stdout}\n{r.stderr}")
    return out


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    _check_loads(tmp)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library (and the benchmark's
    probe library); returns the GEMM library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs) + 1) as ex:
        asm = ex.submit(_device_asm, "gemm_dma.hip", DMA_ASM, verbose)
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
        asm.result()
    _link([objs[s] for s in SOURCES], LIB, verbose)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB, verbose)
    return LIB


def _check_loads(path: str) -> None:
    """dlopen the fresh library with immediate binding: a kernel whose host
    stub the compiler dropped shows up here as an undefined symbol."""
    import ctypes
    try:
        ctypes.CDLL(path, mode=os.RTLD_NOW | os.RTLD_LOCAL)
    except OSError as e:
        os.unlink(path)
        raise RuntimeError(f"built library does not load: {e}") from None


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
