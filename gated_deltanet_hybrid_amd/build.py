"""Build libhla.so (gfx950) in-tree with hipcc.

Usage: python -m gated_deltanet_hybrid_amd.build   (or build_library() from Python).
Objects go to gated_deltanet_hybrid_amd/_build/, the library to
gated_deltanet_hybrid_amd/libhla.so.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhla.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["chunk.hip", "scan.hip", "prefill.hip", "route.hip", "compose.hip", "decode.hip", "reps.hip", "reps_bwd.hip", "gdn2.hip", "compose_bwd.hip", "chunk_bwd.hip", "gdn2_bwd.hip", "router_bwd.hip", "abi.cpp", "timing.cpp"]

# Packed fp32 VALU ops are disabled for the device: the kernels are written with scalar
# fp32 arithmetic and must not be turned into v_pk_* instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


# Per-source device flags.  prefill.hip keeps the next piece's operands in small register
# arrays while the current piece computes; LLVM would otherwise move such arrays into LDS
# when LDS is free, which turns every prefetch load into a load, a wait and an LDS store.
# Its state pass also scales and converts the MFMA accumulators (the state, E and O^T) with
# vector instructions every piece: with the accumulators in ordinary VGPRs (they fit, 239
# registers at one wave per SIMD) those need no accumulator-register moves (about 256 per
# piece otherwise).
SOURCE_FLAGS = {"prefill.hip": ["-mllvm", "-disable-promote-alloca-to-lds", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host code only (the C ABI's argument checks, workspace sizing and launch set-up) under
# AddressSanitizer and UndefinedBehaviorSanitizer; every flag is scoped to the host pass.
HOST_SOURCES = ("abi.cpp", "timing.cpp")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized(out: str) -> str:
    """A copy of libhla.so whose host code is built with ASan and UBSan, linked against the
    shared sanitizer runtime (preload it to load the library), with the device objects that
    build_library compiled.  Returns the library's path."""
    objs = []
    san_dir = os.path.join(os.path.dirname(os.path.abspath(out)), "san_objs")
    os.makedirs(san_dir, exist_ok=True)
    for src in SOURCES:
        if src in HOST_SOURCES:
            obj = os.path.join(san_dir, os.path.splitext(src)[0] + ".o")
            cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SAN_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        else:
            obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
            if not os.path.exists(obj):
                raise RuntimeError(f"{obj} is missing: run build_library first")
        objs.append(obj)
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, *SAN_FLAGS, "-Xarch_host", "-shared-libsan",
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return out


if __name__ == "__main__":
    build_library(verbose=True)
    sys.exit(0)
