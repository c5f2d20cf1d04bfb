"""Builds libmoe_ffn.so (the layer) and libmoe_probe.so (the bandwidth and
MFMA microbenchmarks the benchmark reports as measured peaks) in-tree with
hipcc for gfx950.

    python -m sparse_mixture_experts_scan_amd.build [-v]

Each HIP source is compiled to an object in parallel, then linked into the
shared libraries next to this file.  Always rebuilds (it is the "does it build"
check as well as the build)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_ffn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
PROBE_LIB_PATH = os.path.join(PKG, "libmoe_probe.so")
PROBE_SOURCES = ["peak_probe.hip"]
SOURCES = ["route_permute.hip", "gemm_stream.hip", "gemm_tile.hip", "gemm_q4.hip", "gemm_bwd.hip",
           "gemm_bwd_tile.hip",
           "moe_ffn.hip", "plan.cpp"]
ARCH = "gfx950"

# Packed fp32 VALU ops are switched off for all device code; hipcc's host pass
# warns that it does not know the feature, which is harmless.
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


# Per-source additions: the INT4 streaming kernels post-scale every MFMA
# result with the VALU, and with MFMA accumulators in AGPRs each of those
# reads is an extra copy; the VGPR form of the MFMAs avoids it.
SOURCE_FLAGS = {"gemm_q4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    cmds = []

    def obj_of(src):
        return os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    for src in SOURCES + PROBE_SOURCES:
        cmds.append([cc, *HIP_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj_of(src)])
    with ThreadPoolExecutor(min(len(cmds), 8)) as pool:
        list(pool.map(lambda c: _run(c, verbose), cmds))
    for path, srcs in ((LIB_PATH, SOURCES), (PROBE_LIB_PATH, PROBE_SOURCES)):
        tmp = path + ".tmp"
        _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *map(obj_of, srcs), "-o", tmp],
             verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
