"""The C ABI on the CPU: the library loads, exports every function include/moe_nvfp4.h
declares, and every host-side validation returns its documented status before any HIP
call (no GPU needed: invalid calls never reach a launch)."""
import ctypes as C
import os
import re

import pytest

import block_scaled_fp4_02_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_nvfp4.h")
FAKE = C.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w \*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(moe.EXPORTED) == names


def test_status_strings():
    L = moe.lib()
    for s in range(7):
        assert L.moe_status_string(s)
    assert L.moe_last_hip_error() == 0


def test_route_permute_validation():
    L = moe.lib()
    ws = L.moe_route_permute_workspace(16, 4, 2)
    assert ws > 0
    args = lambda T, E, k, logits=FAKE, ws_bytes=ws: (logits, T, E, k, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws_bytes, None)
    assert L.moe_route_permute(*args(16, 4, 2, logits=None)) == moe.MOE_ERR_NULL
    assert L.moe_route_permute(*args(-1, 4, 2)) == moe.MOE_ERR_SHAPE
    assert L.moe_route_permute(*args(16, 4, 5)) == moe.MOE_ERR_SHAPE      # k > E
    assert L.moe_route_permute(*args(16, 4, 0)) == moe.MOE_ERR_SHAPE
    assert L.moe_route_permute(*args(16, 2048, 2)) == moe.MOE_ERR_SHAPE   # E > 1024
    assert L.moe_route_permute(*args(16, 64, 33)) == moe.MOE_ERR_SHAPE    # k > 32
    assert L.moe_route_permute(*args(16, 4, 2, ws_bytes=ws - 1)) == moe.MOE_ERR_WORKSPACE
    assert L.moe_route_permute_workspace(-1, 4, 2) == 0


def test_quantize_validation():
    L = moe.lib()
    ws = L.moe_quantize_nvfp4_workspace(4, 32)
    q = lambda rows, cols, x=FAKE, dtype=0, mode=1, gs=FAKE, ws_bytes=ws: L.moe_quantize_nvfp4(
        x, dtype, rows, cols, FAKE, FAKE, gs, mode, None, 0, FAKE, ws_bytes, None)
    assert q(4, 24) == moe.MOE_ERR_SHAPE           # C % 16
    assert q(4, 8) == moe.MOE_ERR_SHAPE
    assert q(-1, 32) == moe.MOE_ERR_SHAPE
    assert q(4, 32, x=None) == moe.MOE_ERR_NULL
    assert q(4, 32, gs=None) == moe.MOE_ERR_NULL
    assert q(4, 32, dtype=7) == moe.MOE_ERR_UNSUPPORTED
    assert q(4, 32, mode=9) == moe.MOE_ERR_UNSUPPORTED
    assert q(4, 32, ws_bytes=0) == moe.MOE_ERR_WORKSPACE


def gemm_args(E=8, N=2048, K=6144, R=256, epi=0, null=None, layout=0):
    a = moe.moe_gemm_args()
    for f in ("A", "A_sf", "A_gs", "B", "B_sf", "B_gs", "expert_offsets", "D", "amax_out", "D_sf", "D_gs"):
        setattr(a, f, FAKE)
    a.rows_A, a.E, a.N, a.K, a.R, a.epilogue, a.B_layout = R, E, N, K, R, epi, layout
    if null:
        setattr(a, null, None)
    return a


def test_gemm_can_implement_is_truthful_on_shapes():
    L = moe.lib()
    ok = gemm_args()
    assert L.moe_grouped_gemm_nvfp4_can_implement(C.byref(ok)) == moe.MOE_OK
    assert L.moe_grouped_gemm_nvfp4_workspace(C.byref(ok)) > 0
    assert L.moe_grouped_gemm_nvfp4_amax_slots(C.byref(ok)) > 0
    cases = [
        (dict(K=100), moe.MOE_ERR_SHAPE),           # K % 16
        (dict(K=272), moe.MOE_ERR_UNSUPPORTED),     # K % 256
        (dict(N=100), moe.MOE_ERR_UNSUPPORTED),     # N % 256
        (dict(E=0), moe.MOE_ERR_SHAPE),
        (dict(R=-1), moe.MOE_ERR_SHAPE),
        (dict(epi=5), moe.MOE_ERR_UNSUPPORTED),
        (dict(epi=2), moe.MOE_ERR_UNSUPPORTED),      # SwiGLU + NVFP4 needs packed weights
        (dict(epi=2, layout=1, null="D_gs"), moe.MOE_ERR_NULL),
        (dict(epi=2, layout=1, null="D_sf"), moe.MOE_ERR_NULL),
        (dict(null="B"), moe.MOE_ERR_NULL),
        (dict(null="expert_offsets"), moe.MOE_ERR_NULL),
        (dict(null="D"), moe.MOE_ERR_NULL),
        (dict(epi=1, null="amax_out"), moe.MOE_ERR_NULL),
    ]
    for kw, want in cases:
        a = gemm_args(**kw)
        assert L.moe_grouped_gemm_nvfp4_can_implement(C.byref(a)) == want, kw
        assert L.moe_grouped_gemm_nvfp4(C.byref(a), FAKE, 1 << 30, None) == want, kw
    assert L.moe_grouped_gemm_nvfp4_can_implement(None) == moe.MOE_ERR_NULL
    # activation rows beyond the packed kernel's 32-bit descriptors are refused, also where
    # rows_A * K / 2 would wrap around 2^64
    for rows_a in (2 ** 31 // 128, 2 ** 57, 2 ** 63 - 1):
        a = gemm_args(layout=1, K=256)
        a.rows_A = rows_a
        assert L.moe_grouped_gemm_nvfp4_can_implement(C.byref(a)) == moe.MOE_ERR_UNSUPPORTED, rows_a
    # SwiGLU + NVFP4 with packed weights and all its pointers is supported
    assert L.moe_grouped_gemm_nvfp4_can_implement(C.byref(gemm_args(epi=2, layout=1))) == moe.MOE_OK
    # amax_out is only needed by the SwiGLU epilogue
    assert L.moe_grouped_gemm_nvfp4_can_implement(C.byref(gemm_args(null="amax_out"))) == moe.MOE_OK
    # a short workspace is refused before any launch
    ws = L.moe_grouped_gemm_nvfp4_workspace(C.byref(ok))
    assert L.moe_grouped_gemm_nvfp4(C.byref(ok), FAKE, ws - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_grouped_gemm_nvfp4(C.byref(ok), None, ws, None) == moe.MOE_ERR_WORKSPACE


def test_ksplit_grid_is_capped_at_resident_workgroups():
    """The K-split kernel loops over its work items, so its grid (= the partial-maxima slot
    count) stops at the workgroups that fit on the chip at once -- 256 CUs x one 8-wave or two
    4-wave workgroups -- while the item count can exceed it; the other kernels keep the host's
    upper bound on the items."""
    L = moe.lib()
    slots = lambda **kw: L.moe_grouped_gemm_nvfp4_amax_slots(C.byref(gemm_args(layout=1, **kw)))
    # 8 groups x 32 rows, K 6144: split 8 ways, 256 items (one per workgroup)
    assert slots(E=8, N=2048, K=6144, R=256) == 256
    # 14 groups x 33 rows, K 2048: split 8 ways; 14 x 2 chunks x 32 n tiles = 896 items
    assert slots(E=14, N=2048, K=2048, R=462) == 256
    # 32 groups x 33 rows, K 512: split 2 ways (4-wave workgroups, 128-row n tiles);
    # 32 x 2 x 16 = 1024 items
    assert slots(E=32, N=2048, K=512, R=1056) == 512
    # 100 experts (a schedule kernel writes the item list), K 2048, N 256: split 8 ways
    assert slots(E=100, N=256, K=2048, R=141) == 256
    # the decode layer's 256 experts use the LDS kernel: (ceil(8192 / 48) + 256) x 16 items
    assert slots(E=256, N=4096, K=6144, R=8192) == (8192 // 48 + 1 + 256) * 16


def test_single_step_items_cover_several_n_tiles():
    """K = 256 (one K step) with the NONE epilogue: each item of the four-wave kernel covers
    several 256-row n tiles, as many as keep about three items per workgroup slot (2 at the
    TP8 share's down GEMM: 256 experts, 8192 rows, N 6144); SWIGLU and longer K keep one."""
    L = moe.lib()
    slots = lambda **kw: L.moe_grouped_gemm_nvfp4_amax_slots(C.byref(gemm_args(layout=1, **kw)))
    bound_items = lambda n_tiles: -(-((8192 + 47) // 48 + 256) * n_tiles // 8) * 8
    assert slots(E=256, N=6144, K=256, R=8192) == bound_items(12)
    assert slots(E=256, N=6144, K=256, R=8192, epi=1) == bound_items(24)
    assert slots(E=256, N=6144, K=512, R=8192) == bound_items(24)


def test_plan_two_items_per_cu_uses_64_row_chunks():
    """One item per (expert, n tile) filling two workgroups per CU at tens of rows per expert
    (the TP8 and EP8 shares' gate/up GEMMs) takes 64-row chunks: the grid bound counts
    n_tiles * (ceil(R / 64) + E) items; otherwise 48-row chunks."""
    L = moe.lib()
    slots = lambda **kw: L.moe_grouped_gemm_nvfp4_amax_slots(C.byref(gemm_args(layout=1, **kw)))
    bound = lambda R, E, n_tiles, chunk: -(-(n_tiles * (-(-R // chunk) + E)) // 8) * 8
    assert slots(E=256, N=512, K=6144, R=8192, epi=1) == bound(8192, 256, 2, 64)      # TP8 gate/up
    assert slots(E=32, N=4096, K=6144, R=1024, epi=1) == bound(1024, 32, 16, 64)      # EP8 gate/up
    assert slots(E=256, N=4096, K=6144, R=8192, epi=1) == bound(8192, 256, 16, 48)    # decode: many items
    assert slots(E=256, N=512, K=6144, R=40 * 256 + 1, epi=1) == bound(40 * 256 + 1, 256, 2, 48)   # > 40 rows each


def test_gemm_workspace_grows_with_rows_and_experts():
    """Launches whose items are looked up in the kernel need only the 16-byte item count (up
    to 64 experts, or up to 256 with K >= 1024 outside the K-split kernel); the others hold
    an item list that grows with the rows and the experts."""
    L = moe.lib()
    ws = lambda layout=0, **kw: L.moe_grouped_gemm_nvfp4_workspace(C.byref(gemm_args(layout=layout, **kw)))
    assert ws(E=8, R=256) == 16
    assert ws(E=256, R=131072) == 16
    assert ws(E=256, R=8192, K=7168, N=512, layout=1) == 16
    assert ws(E=256, R=8192, K=512, layout=1) > 16
    assert ws(E=257, R=131072) > ws(E=257, R=8192) > 16
    assert ws(E=256, R=131072, K=256) > ws(E=256, R=8192, K=256) > 16
    # 100 experts whose few rows leave the K-split kernel in charge: listed items
    assert ws(E=100, R=139, K=2048, N=256, layout=1) > 16


def test_finalize_validation():
    L = moe.lib()
    f = lambda T, k, H, R=64, Y=FAKE: L.moe_finalize(Y, R, FAKE, FAKE, T, k, H, FAKE, None)
    assert f(8, 2, 12) == moe.MOE_ERR_UNSUPPORTED     # H % 8
    assert f(8, 0, 64) == moe.MOE_ERR_SHAPE
    assert f(8, 33, 64) == moe.MOE_ERR_SHAPE
    assert f(-1, 2, 64) == moe.MOE_ERR_SHAPE
    assert f(8, 2, 64, R=0) == moe.MOE_ERR_SHAPE
    assert f(8, 2, 64, Y=None) == moe.MOE_ERR_NULL


def test_binding_refuses_to_run_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        moe.lib()


def test_header_is_c11_and_matches_the_binding(tmp_path):
    """include/moe_nvfp4.h compiles as C11 with warnings as errors, and the binding's view of
    it agrees: the size and every field offset of moe_gemm_args, and every enum constant."""
    import ctypes
    import shutil
    import subprocess

    import block_scaled_fp4_02_amd as m

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    fields = [f for f, _ in m.moe_gemm_args._fields_]
    consts = ["MOE_OK", "MOE_ERR_NULL", "MOE_ERR_SHAPE", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE",
              "MOE_ERR_HIP", "MOE_DTYPE_BF16", "MOE_DTYPE_F32", "MOE_GS_STATIC", "MOE_GS_DYNAMIC",
              "MOE_EPI_NONE", "MOE_EPI_SWIGLU", "MOE_EPI_SWIGLU_NVFP4", "MOE_LAYOUT_ROWMAJOR",
              "MOE_LAYOUT_PACKED"]
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "moe_nvfp4.h"', "int main(void) {",
           '  printf("size %zu\\n", sizeof(moe_gemm_args));']
    src += [f'  printf("off {f} %zu\\n", offsetof(moe_gemm_args, {f}));' for f in fields]
    src += [f'  printf("const {c} %d\\n", (int){c});' for c in consts]
    src += ["  return 0;", "}"]
    (tmp_path / "abi.c").write_text("\n".join(src) + "\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "abi"
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
                    str(tmp_path / "abi.c"), "-o", str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        *key, value = ln.split()
        got[" ".join(key)] = int(value)
    assert got["size"] == ctypes.sizeof(m.moe_gemm_args)
    for f in fields:
        assert got[f"off {f}"] == getattr(m.moe_gemm_args, f).offset, f
    for c in consts:
        assert got[f"const {c}"] == getattr(m, c), c


def test_host_queries_survive_random_and_hostile_arguments():
    """Seeded fuzz of the host-only entry points (no launch is ever attempted): for random,
    often invalid shapes, layouts, epilogues and NULL pointers, can_implement returns a
    documented status, and the workspace and amax-slot queries (shapes only) are non-zero
    exactly when can_implement fails for no reason but a NULL pointer; the quantiser and
    routing workspace queries never fail."""
    import numpy as np
    L = moe.lib()
    rng = np.random.default_rng(1234)
    ptrs = ("A", "A_sf", "A_gs", "A_rows", "B", "B_sf", "B_gs", "expert_offsets", "D", "amax_out", "D_sf", "D_gs")

    def dim(mults=(16, 256, 512)):
        kind = rng.integers(0, 5)
        if kind == 0:
            return int(rng.integers(-300, 300))
        if kind == 1:
            return int(rng.choice(mults)) * int(rng.integers(0, 40))
        if kind == 2:
            return int(rng.integers(0, 1 << 31))
        return int(rng.choice(mults)) * int(rng.integers(1, 64))

    seen = set()
    for _ in range(4000):
        a = moe.moe_gemm_args()
        for f in ptrs:
            setattr(a, f, None if rng.random() < 0.08 else FAKE)
        a.E = int(rng.choice([-1, 0, 1, 8, 256, 65536, 65537, int(rng.integers(1, 5000))]))
        a.N, a.K = dim(), dim()
        a.R = int(rng.choice([-1, 0, 1, 256, 8192, 1 << 31, 1 << 40, int(rng.integers(0, 1 << 20))]))
        a.rows_A = int(rng.choice([-1, 0, a.R if a.R >= 0 else 0, 1 << 33, int(rng.integers(0, 1 << 20))]))
        a.epilogue = int(rng.integers(-1, 4))
        a.B_layout = int(rng.integers(-1, 3))
        st = L.moe_grouped_gemm_nvfp4_can_implement(C.byref(a))
        assert st in (moe.MOE_OK, moe.MOE_ERR_NULL, moe.MOE_ERR_SHAPE, moe.MOE_ERR_UNSUPPORTED), st
        ws = L.moe_grouped_gemm_nvfp4_workspace(C.byref(a))
        slots = L.moe_grouped_gemm_nvfp4_amax_slots(C.byref(a))
        if st in (moe.MOE_OK, moe.MOE_ERR_NULL):
            assert ws > 0 and slots > 0, st
        else:
            assert ws == 0 and slots == 0, st
        seen.add(st)
    assert seen == {moe.MOE_OK, moe.MOE_ERR_NULL, moe.MOE_ERR_SHAPE, moe.MOE_ERR_UNSUPPORTED}
    for _ in range(2000):
        rows, cols = int(rng.integers(-5, 1 << 24)), int(rng.integers(-5, 1 << 16))
        L.moe_quantize_nvfp4_workspace(rows, cols)
        T, E, k = int(rng.integers(-5, 1 << 20)), int(rng.integers(-5, 2000)), int(rng.integers(-5, 40))
        L.moe_route_permute_workspace(T, E, k)


def test_noalloc_gemm_refuses_launches_beyond_its_scratch():
    """The no-allocation grouped GEMM validates like the workspace entry point and refuses, on
    the host and before any HIP call, a launch whose work list exceeds its static scratch."""
    L = moe.lib()
    # 65536 experts of one row each: ~65,536 x 24 items of 16 bytes, far beyond 1 MiB
    a = moe.moe_gemm_args()
    a.A, a.A_sf, a.A_gs, a.B, a.B_gs, a.expert_offsets, a.D = (FAKE,) * 7
    a.rows_A, a.E, a.N, a.K, a.R = 65536, 65536, 6144, 256, 65536
    a.epilogue, a.B_layout = moe.MOE_EPI_NONE, moe.MOE_LAYOUT_PACKED
    assert L.moe_grouped_gemm_nvfp4_can_implement(C.byref(a)) == moe.MOE_OK
    assert L.moe_grouped_gemm_nvfp4_workspace(C.byref(a)) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert L.moe_grouped_gemm_nvfp4_noalloc(C.byref(a), None) == moe.MOE_ERR_WORKSPACE
    a.E = 0
    assert L.moe_grouped_gemm_nvfp4_noalloc(C.byref(a), None) == moe.MOE_ERR_SHAPE
    assert L.moe_grouped_gemm_nvfp4_noalloc(None, None) == moe.MOE_ERR_NULL
