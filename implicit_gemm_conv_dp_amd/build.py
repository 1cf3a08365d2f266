"""Builds libskgemm.so for gfx950 in the package directory.

    python -m implicit_gemm_conv_dp_amd.build [-j N]

hipcc cross-compiles the device code, so this runs on a machine without a
GPU.  Object files go to ``_build/`` at the repository root; the shared
library lands next to this file, where the binding loads it from.
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libskgemm.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 instructions are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]

SOURCES = ["skg_host.cpp", "skg_api.hip", "skg_inst_gemm.hip", "skg_inst_gemm_f16.hip",
           "skg_inst_gemm_bf16.hip", "skg_inst_gemm_f8.hip", "skg_inst_wgrad.hip",
           "skg_inst_fwd.hip", "skg_inst_dgrad.hip"]


def _compile(src):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".cpp"):
        cmd = ["g++"] + HOST_FLAGS + ["-c", path, "-o", obj]
    else:
        cmd = [HIPCC] + HIP_FLAGS + ["-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def build(jobs=4, verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s" % (res.stdout, res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=4)
    args = ap.parse_args(argv)
    build(args.j)


if __name__ == "__main__":
    sys.exit(main())
