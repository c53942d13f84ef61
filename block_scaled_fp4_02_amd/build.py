"""Build libmoe_nvfp4.so (HIP, gfx950 only) in-tree with hipcc.

Every source is compiled for gfx950 with packed-FP32 instruction selection disabled, then
linked into one shared library next to this file.  Object files go to ``_build/`` at the
repository root (git-ignored).
"""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "moe_nvfp4")
LIB_PATH = os.path.join(PKG, "libmoe_nvfp4.so")
SOURCES = ["route_permute.hip", "quantize.hip", "grouped_gemm.hip", "gemm_lds.hip", "gemm_ksplit.hip",
           "gemm_rowmajor.hip", "finalize.hip", "moe_api.hip"]
# the benchmark's measurement kernels (streaming read, MFMA throughput), a library of their own
# (not the MoE ABI)
PROBE_SOURCES = ["stream_probe.hip", "mfma_probe.hip"]
PROBE_LIB_PATH = os.path.join(PKG, "libmoe_probes.so")
# per-source extra flags: the MFMA probe's loop keeps its accumulators in VGPRs only in the
# VGPR form of MFMA
EXTRA_FLAGS = {"mfma_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH_FLAGS = ["--offload-arch=gfx950"]
COMPILE_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
                 "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                 "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *ARCH_FLAGS, *COMPILE_FLAGS, *EXTRA_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 target feature and says so: harmless.
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg)
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, *ARCH_FLAGS, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, path)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    allsrc = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(min(len(allsrc), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, allsrc))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH)
    if verbose:
        print("built", LIB_PATH, "and", PROBE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
