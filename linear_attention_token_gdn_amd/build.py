"""Build libgdn.so (HIP for gfx950) in-tree with hipcc, and libgdn_calib.so (the benchmark's
attainable-peak kernels, include/gdn_calib.h).

Usage: ``python -m linear_attention_token_gdn_amd.build`` or ``build()`` from Python.
Every call recompiles every source.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
CALIB_LIB = os.path.join(PKG, "libgdn_calib.so")
SOURCES = ["gdn_api.hip", "decode.hip", "recurrent.hip", "chunk_mfma.hip", "chunk_split.hip",
           "backward.hip", "backward_chunk.hip", "qsa.hip"]
ARCH = os.environ.get("GDN_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions (v_pk_*_f32) anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + ["calib.hip"]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], CALIB_LIB)
    if verbose:
        print("built", LIB, "and", CALIB_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
