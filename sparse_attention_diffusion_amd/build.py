"""Build libmcs.so (the MC-Sparse C-ABI library) in-tree for gfx950 with hipcc.

Usage: python -m sparse_attention_diffusion_amd.build  (or build() from Python).
Always recompiles every source; objects go to sparse_attention_diffusion_amd/_build/.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmcs.so")
SOURCES = ["attn.hip", "select.hip", "pddp.hip", "keybits.hip", "pairs.hip", "blocksel.hip", "api.cpp"]
# Attention keeps its 64x128 fp32 output tile in VGPRs (MFMA accumulators in the
# VGPR form), so the rare rescale of O needs no copies between register files.
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "select.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions stay off: the compiler emits only scalar fp32 VALU ops.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


ASAN_LIB = os.path.join(OUT, "libmcs_asan.so")


def build_asan(verbose: bool = False) -> str:
    """A copy of the library whose host code (the C ABI: argument checks, workspace
    carving, launch set-up) is built with AddressSanitizer; the device code is the
    same as in libmcs.so.  For host-side checks only: load it in a process that has
    the clang ASan runtime (asan_runtime()) preloaded."""
    build()
    obj = os.path.join(OUT, "api_asan.o")
    cmd = [HIPCC, *COMMON, "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of api.cpp with AddressSanitizer failed:\n{r.stderr}")
    objs = [obj] + [os.path.join(OUT, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "api.cpp"]
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-shared-libasan", "-o", ASAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of the AddressSanitizer library failed:\n{r.stderr}")
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that hipcc links against."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(HIPCC)))
    hits = sorted(glob.glob(os.path.join(root, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so next to hipcc")
    return hits[-1]


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
