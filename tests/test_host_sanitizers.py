"""The ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The library sources are compiled as for gfx950 with both sanitizers on the host pass only,
linked with `tests/abi_fuzz.c`, and run on the CPU (no call in the driver reaches a launch, so
no GPU is needed): tens of thousands of random and limit-value argument sets go through every entry
point's validation and every host-side query.  Any out-of-bounds access, signed overflow or
other undefined behaviour aborts the run; the driver itself checks that no call with a
missing pointer or workspace is accepted."""
from __future__ import annotations

import os
import shlex
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp4_02_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_INCLUDE = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
SOURCES = ["moe_api.hip", "grouped_gemm.hip", "route_permute.hip", "quantize.hip", "finalize.hip",
           "gemm_lds.hip", "gemm_ksplit.hip", "gemm_rowmajor.hip"]
# host pass only: each sanitizer flag directly after -Xarch_host
SAN = shlex.split("-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
                  "-Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer")
COMMON = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    if not os.path.exists(HIPCC) or shutil.which("gcc") is None:
        pytest.skip("hipcc or gcc not available")
    d = tmp_path_factory.mktemp("abi_san")

    def compile_one(src):
        obj = str(d / (os.path.splitext(src)[0] + ".o"))
        r = subprocess.run([HIPCC, *COMMON, *SAN, "-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv = str(d / "abi_fuzz.o")
    r = subprocess.run([HIPCC, "-x", "c", "-std=c11", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I",
                        os.path.join(ROOT, "include"), "-I", ROCM_INCLUDE, *SAN, "-c", os.path.join(ROOT, "tests", "abi_fuzz.c"),
                        "-o", drv], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(d / "abi_fuzz")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", *SAN, *objs, drv, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_abi_validation_is_clean_under_asan_and_ubsan(fuzz_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([fuzz_binary, "30000"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.startswith("ok "), r.stdout
