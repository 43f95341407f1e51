"""Builds libpsgd.so, the HIP library of this package, for gfx950.

Each source is compiled to an object under _build/ (in parallel), then linked
into rank_gradient_compression_amd/libpsgd.so.  Every call recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpsgd.so")

SOURCES = ["plan.cpp", "api.hip", "kernels_valu.hip", "kernels_mfma.hip", "kernels_rng.hip", "kernels_probe.hip",
           "kernels_diag.hip", "kernels_payload.hip"]

# Packed fp32 instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libpsgd.so")
    return exe


def _compile(src: str, verbose: bool) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
           "-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["--offload-arch=gfx950", "-x", "hip"] + DEVICE_FLAGS
    else:  # host-only C++ (no device code)
        cmd[1:1] = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(hipcc()))), "include")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{res.stdout}\n{res.stderr}")
    noisy = [l for l in res.stderr.splitlines() if l.strip() and "packed-fp32-ops" not in l]
    if verbose and noisy:
        print("\n".join(noisy), file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(max_workers=min(4, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libpsgd.so failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    build_c_smoke(verbose)
    return LIB


C_SMOKE = os.path.join(PKG, "psgd_c_smoke")


def build_c_smoke(verbose: bool = False) -> str:
    """The plain C client (csrc/c_smoke.c), linked against libpsgd.so and the
    HIP runtime with gcc: no HIP compiler, no Python."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(rocm, "include"), os.path.join(CSRC, "c_smoke.c"), "-o", C_SMOKE + ".tmp",
           "-L", PKG, "-lpsgd", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"building the C client failed:\n{res.stdout}\n{res.stderr}")
    os.replace(C_SMOKE + ".tmp", C_SMOKE)
    return C_SMOKE


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
