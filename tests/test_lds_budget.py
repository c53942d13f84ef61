"""The compile-time LDS budget of the grouped GEMM tiles (csrc/lds_budget.hpp).  CPU only.

1. The header's formula reproduces the pages' shared-memory table for their SM120 tiles
   (tests/golden/lds_budget_sm120.txt) and its fit verdicts against 101,376 bytes.
2. Every tile of this library's plan fits the 163,840 bytes of LDS of a CDNA4 compute
   unit, shared by the workgroups its launch bounds promise.
3. The LDS the compiler actually allocates for every GEMM kernel (hipcc's resource-usage
   remarks for gfx950) is within that kernel's budget entry, and its occupancy is at least
   the waves per SIMD the kernel is designed for.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_fp4_02_amd", "csrc")
GOLDEN = os.path.join(ROOT, "tests", "golden", "lds_budget_sm120.txt")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

PROBE = r"""
#include <stdio.h>
#include "lds_budget.hpp"
using namespace moe::lds;
int main() {
  const long long t[4][3] = {{128, 128, 128}, {128, 128, 256}, {128, 256, 128}, {256, 128, 128}};
  for (auto &m : t)
    printf("sm120 %lld %lld %lld %lld %lld %lld %lld %lld %lld\n", m[0], m[1], m[2],
           (long long)sm120_tile_bytes(m[0], m[1], m[2], 1, false), (long long)sm120_tile_bytes(m[0], m[1], m[2], 1, true),
           (long long)nvfp4_stage_bytes(m[0], m[1], m[2]), (long long)epilogue_staging_bytes(m[0], m[1], false),
           (long long)stages_that_fit(m[0], m[1], m[2], false, kSm120OptInBlockBytes),
           (long long)stages_that_fit(m[0], m[1], m[2], true, kSm120OptInBlockBytes));
  for (const TileEntry &e : kTileTable)
    printf("tile %lld %lld %lld %lld|%s\n", (long long)e.token_rows, (long long)e.weight_rows,
           (long long)e.workgroups_per_cu, (long long)e.lds_bytes, e.name);
  printf("budget %lld %lld %lld\n", (long long)kSm120OptInBlockBytes, (long long)kSm120BytesPerSm,
         (long long)kCdna4BytesPerCu);
  printf("lds %lld %lld ksplit %lld %lld rowmajor %lld %lld %lld lds64 %lld\n", (long long)lds_kernel_bytes(3, 4),
         (long long)lds_kernel_bytes(6, 8), (long long)ksplit_kernel_bytes(2, 4), (long long)ksplit_kernel_bytes(2, 8),
         (long long)rowmajor_kernel_bytes(1), (long long)rowmajor_kernel_bytes(2), (long long)rowmajor_kernel_bytes(4),
         (long long)lds_kernel_bytes(4, 4));
  return 0;
}
"""


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    d = tmp_path_factory.mktemp("lds")
    src = d / "probe.cpp"
    src.write_text(PROBE)
    exe = d / "probe"
    subprocess.run(["g++", "-std=c++17", "-Wall", "-Werror", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    rec = {"sm120": {}, "tiles": []}
    for ln in out.splitlines():
        f = ln.split()
        if f[0] == "sm120":
            v = list(map(int, f[1:]))
            rec["sm120"][tuple(v[:3])] = v[3:]
        elif f[0] == "tile":
            nums, name = ln[5:].split("|")
            rec["tiles"].append((name, *map(int, nums.split())))
        elif f[0] == "budget":
            rec["budget"] = list(map(int, f[1:]))
        elif f[0] == "lds":
            rec["lds4"], rec["lds8"] = int(f[1]), int(f[2])
            rec["ksplit4"], rec["ksplit8"] = int(f[4]), int(f[5])
            rec["rowmajor"] = {1: int(f[7]), 2: int(f[8]), 4: int(f[9])}
            rec["lds64"] = int(f[11])
    return rec


def golden_rows():
    rows = []
    for ln in open(GOLDEN):
        if ln.strip() and not ln.startswith("#"):
            rows.append(list(map(int, ln.split())))
    return rows


def test_pages_table_reproduced(probe):
    budget = probe["budget"][0]
    assert budget == 101376
    for M, N, K, none_kb, fin_kb, none_fits, fin_fits in golden_rows():
        none_b, fin_b, stage, staging, _, _ = probe["sm120"][(M, N, K)]
        # the pages' KB figures are whole multiples of 1024 bytes
        assert none_b == none_kb * 1024 and fin_b == fin_kb * 1024, (M, N, K, none_b, fin_b)
        assert (none_b <= budget) == bool(none_fits) and (fin_b <= budget) == bool(fin_fits), (M, N, K)


def test_pages_large_tile_stage_arithmetic(probe):
    """For 128 x 256 the pages put the BF16 output staging at 64 KB and one mainloop stage at
    about 27.6 KB; what is left of the 99 KB is 35,840 bytes, so exactly one stage does fit
    (their sentence that not even one stage fits contradicts their own two figures)."""
    none_b, fin_b, stage, staging, stages_none, stages_fin = probe["sm120"][(128, 256, 128)]
    assert staging == 65536 and stage == 27648
    assert 101376 - staging == 35840 and stages_none == 1 and stages_fin == 0
    assert probe["sm120"][(128, 128, 256)][5] == 0   # FINALIZE at 128x128x256: no stage left


def test_plan_tiles_fit_cdna4(probe):
    cu = probe["budget"][2]
    assert cu == 163840
    names = [t[0] for t in probe["tiles"]]
    assert any("decode" in n for n in names) and any("wide" in n for n in names)
    for name, rows, wrows, wg_per_cu, nbytes in probe["tiles"]:
        assert nbytes * wg_per_cu <= cu, name
    # the figures of the kernels' shared structs (also static_asserted in the kernels)
    assert probe["lds4"] == 49168 and probe["lds8"] == 110624
    assert probe["ksplit4"] == 32784 and probe["ksplit8"] == 65568
    assert probe["rowmajor"] == {1: 20, 2: 32784, 4: 49168}
    assert probe["lds64"] == 65552


# ---- what the compiler allocates ---------------------------------------------------

KERNEL_FILES = ["gemm_lds.hip", "gemm_ksplit.hip", "gemm_rowmajor.hip"]


def _resource_usage(src: str, outdir: str) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", os.path.join(CSRC, src),
           "-o", os.path.join(outdir, src + ".o"), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return r.stderr


def _parse(remarks: str):
    """{mangled kernel name: {"lds": bytes, "occupancy": waves per SIMD, "scratch": bytes}}"""
    out, cur = {}, None
    for ln in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", ln)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        for key, pat in (("lds", r"LDS Size \[bytes/block\]: (\d+)"), ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"), ("vgpr", r"VGPRs: (\d+)")):
            m = re.search(pat, ln)
            if m and cur:
                out[cur][key] = int(m.group(1))
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("g++") is None, reason="needs hipcc")
def test_compiled_kernels_within_budget(probe, tmp_path):
    with ThreadPoolExecutor(len(KERNEL_FILES)) as ex:
        remarks = list(ex.map(lambda f: _resource_usage(f, str(tmp_path)), KERNEL_FILES))
    kernels = {}
    for r in remarks:
        kernels.update(_parse(r))
    seen = set()
    for name, u in kernels.items():
        # (budget entry, waves per workgroup, waves per SIMD the kernel is designed for)
        if "gemm_lds_wide_kernel" in name:
            entry, waves, waves_per_simd, fam = probe["lds8"], 8, 2, "wide"
        elif "gemm_lds_kernel" in name:
            entry, waves, waves_per_simd, fam = probe["lds4"], 4, 3, "lds"
        elif "gemm_lds64_kernel" in name:
            entry, waves, waves_per_simd, fam = probe["lds64"], 4, 2, "lds64"
        elif "gemm_ksplit_kernel" in name:
            ks = int(re.search(r"gemm_ksplit_kernelILi(\d+)E", name).group(1))
            entry, waves, waves_per_simd, fam = probe["ksplit8" if ks == 8 else "ksplit4"], max(4, ks), 2, "ksplit"
        elif "gemm_rowmajor_kernel" in name:
            ks = int(re.search(r"gemm_rowmajor_kernelILi(\d+)E", name).group(1))
            entry, waves, waves_per_simd, fam = probe["rowmajor"][ks], 4, 2, "rowmajor"
        else:
            continue
        seen.add(fam)
        print(f"{name}: {u}")
        workgroups_per_cu = 4 * waves_per_simd // waves
        assert u["lds"] <= entry, (name, u, entry)
        assert u["lds"] * workgroups_per_cu <= 163840, (name, u)
        assert u["occupancy"] >= waves_per_simd, (name, u)
        assert u["scratch"] == 0, (name, u)   # no register spills
    assert seen == {"wide", "lds", "lds64", "ksplit", "rowmajor"}
