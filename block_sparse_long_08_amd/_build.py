"""Build libqsa.so (hand-written HIP for gfx950) in the package directory."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqsa.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["qsa_api.cpp", "elementwise.hip", "index_scores.hip", "topk.hip",
           "attention.hip", "flash_prefill.hip", "distill.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
         # packed fp32 instructions are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]
# The indexer's scores are finite (bf16 inputs, fp32 sums of 128 products):
# without NaN semantics its max over heads needs no quieting moves before
# each v_max (74 fewer VALU instructions per 64-block tile of a wave; the
# selection 2-3% faster at 128K and at a 1M-token context); max of finite
# values is the same value either way.
FILE_FLAGS = {"index_scores.hip": ["-fno-honor-nans"]}


# The benchmark's gather-ceiling probe (a measurement kernel, not part of the
# layer) lives in a library of its own.
PROBE_SRC = "probe_gather.hip"
PROBE_LIB = os.path.join(HERE, "libqsa_probe.so")


def build_probe(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", "-x", "hip", os.path.join(CSRC, PROBE_SRC), "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{errs}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c",
               os.path.join(CSRC, src), "-o", obj]
        if resource_usage:
            cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in r.stderr.splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if (verbose or resource_usage) and errs.strip():
            print(errs, file=sys.stderr)
        objs.append(obj)
    tmp = LIB + ".tmp"
    subprocess.check_call([HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True, resource_usage="--usage" in sys.argv)
    print(LIB)
