"""Build the HIP library ``libkda.so`` (gfx950) in-tree with hipcc, and the
benchmark's bandwidth-calibration library ``libkda_stream.so`` beside it.

Usage: ``python -m kimi_delta_attention_amd.build`` or ``build()`` from Python.
Objects go to ``_build/`` at the repository root; the shared library is
written next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkda.so")
STREAM_LIB = os.path.join(HERE, "libkda_stream.so")
STREAM_SOURCE = "stream_ceiling.hip"

SOURCES = ["kda_api.cpp", "kda_decode.hip", "kda_conv.hip", "kda_gate.hip", "kda_chunk_fwd.hip", "kda_chunk_bwd.hip",
           "kda_noalloc.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 arithmetic is disabled for all device code (see the comment in
# kda_device.hpp); hipcc's host pass warns that it does not know the feature.
# MFMA accumulators are kept in ordinary VGPRs: the state passes scale and
# round their accumulators every chunk, which the accumulation-register form
# turns into copies between the two register files.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + DEVICE_FLAGS
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [STREAM_SOURCE]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], STREAM_LIB)
    if verbose:
        print("built", LIB, "and", STREAM_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
