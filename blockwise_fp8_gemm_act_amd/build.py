"""Build libpuro.so (the gfx950 HIP kernels + C ABI) in-tree with hipcc.

Usage: python blockwise_fp8_gemm_act_amd/build.py  (run as a script: importing the
package would bind the symbols of a stale library before it is rebuilt)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpuro.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["quant.hip", "gemm.hip", "abi.cpp"]

# gfx950 only.  Packed fp32 VALU instructions are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc()] + HIPCC_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), res.stderr))
    return obj


PROBE_SRC = os.path.join(ROOT, "tests", "csrc", "device_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "csrc", "libdevprobe.so")


def build_probe(verbose: bool = False) -> str:
    """The GPU tests' probe module (tests/csrc/device_probe.hip): device code of the
    library exercised on its own.  Not part of the library."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + HIPCC_FLAGS + ["-shared", PROBE_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for the probe module:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print("built", PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    if os.path.exists(PROBE_SRC):
        build_probe(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
