"""Build libzebra.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python linear_global_attention_amd/build.py

Each source is compiled with hipcc for gfx950 into _build/, then linked into
linear_global_attention_amd/libzebra.so next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libzebra.so")
SOURCES = ["zebra.cpp", "pack.hip", "select.hip", "attn.hip", "attn_exact.hip", "linear.hip", "coverage.hip", "block.hip",
           "linear_bwd.hip", "sparse_bwd.hip"]
ARCH = os.environ.get("ZEBRA_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-result",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer build (device
# code is compiled as usual): validation, tile geometry, buffer sizing and
# the fp64 affine solve, exercised on the CPU by tests/test_sanitized_host.py.
SAN_LIB = os.path.join(BUILD, "san", "libzebra_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def _compile_in(src: str, outdir: str, extra) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build_sanitized(verbose: bool = False) -> str:
    outdir = os.path.dirname(SAN_LIB)
    os.makedirs(outdir, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda f: _compile_in(f, outdir, SAN_FLAGS), SOURCES))
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libasan", "-o", SAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


def build(verbose: bool = False, sanitized: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    if sanitized:
        build_sanitized(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
