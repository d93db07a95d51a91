"""Build libdisco.so (host Psi builder, C-ABI layer and gfx950 HIP kernels).

Usage: python spherical_disco_convolution_amd/build_lib.py [-v]
(run as a script: importing the package requires the built library)
Every call recompiles all sources with hipcc for gfx950 and links the shared
library next to this file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdisco.so")

SOURCES = [
    "psi_host.cpp",
    "disco_api.cpp",
    "kernels_generic.hip",
    "kernels_einsum_mfma.hip",
    "kernels_fused_mfma.hip",
    "kernels_spectral.hip",
    "kernels_backward.hip",
    "spectral_host.cpp",
    "kernel_timing.cpp",
]

# peak micro-benchmarks for the benchmark's roofline check, in a library of
# their own (not part of the DISCO C ABI)
PROBE_SOURCES = ["probe_peaks.hip"]
PROBE_LIB = os.path.join(HERE, "libdisco_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
          "-I" + os.path.join(ROOT, "include")]
# Packed fp32 instructions are disabled for all device code.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON
    if src.endswith(".hip"):
        cmd += ["-x", "hip"] + DEVICE
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{r.stdout}\n{r.stderr}")
    if verbose and r.stderr.strip():
        print(r.stderr, file=sys.stderr)
    return obj


def _link(objs, lib, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    allsrc = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(allsrc), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), allsrc))
    _link(objs[:len(SOURCES)], LIB, verbose)
    _link(objs[len(SOURCES):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
