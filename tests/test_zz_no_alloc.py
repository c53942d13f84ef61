"""moe_grouped_gemm_nvfp4_noalloc -- the grouped GEMM with the library's static device scratch
in place of a caller workspace -- against moe_grouped_gemm_nvfp4 on the same inputs, through
the C ABI: identical bytes on two calls in a row, the second with a smaller input (the
scratch still holds the first call's longer work list), and the size limit refused on the
host before any launch."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("block_scaled_fp4_02_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    yield
    torch.cuda.synchronize()


def _inputs(sizes, K, N, seed):
    """GPU-quantised operands (both entry points read the same device tensors)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    E = len(sizes)
    R = int(sum(sizes))
    T = max(R, 1) + 3
    A = moe.quantize_alloc(torch.randn(T, K, generator=g).to(torch.bfloat16).cuda())
    W = moe.quantize_experts((torch.randn(E, N, K, generator=g) * 0.02).cuda())
    off = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32).cuda()
    rows = torch.randint(0, T, (max(R, 1),), generator=g, dtype=torch.int32).cuda()
    return A, moe.pack_weights(W), off, rows, R


def _run_both(A, B, off, rows, R, epi):
    N = B.N
    cols = N if epi == moe.MOE_EPI_NONE else N // 2
    outs = []
    for which in ("workspace", "noalloc"):
        D = torch.full((max(R, 1), cols), float("nan"), dtype=torch.bfloat16, device="cuda")
        a = moe._gemm_args_for(A, B, off, R, epi, D, rows)
        amax = None
        if epi == moe.MOE_EPI_SWIGLU:
            amax = torch.full((max(moe.moe_grouped_gemm_nvfp4_amax_slots(a), 1),), -1.0, device="cuda")
            a.amax_out = moe._p(amax)
        if which == "workspace":
            moe.moe_grouped_gemm_nvfp4(a, moe._ws(moe.moe_grouped_gemm_nvfp4_workspace(a), "cuda"))
        else:
            assert moe.moe_grouped_gemm_nvfp4_workspace(a) <= moe.MOE_NOALLOC_SCRATCH_BYTES
            moe.moe_grouped_gemm_nvfp4_noalloc(a)
        torch.cuda.synchronize()
        outs.append((D[:R].clone(), None if amax is None else amax.clone()))
    (d0, m0), (d1, m1) = outs
    assert torch.equal(d0.view(torch.int16), d1.view(torch.int16))
    if m0 is not None:
        assert torch.equal(m0, m1)
    assert not torch.isnan(d1.float()).any()


def test_noalloc_matches_workspace_entry_twice_then_smaller():
    rng = np.random.default_rng(77)
    # 1) 256 experts (> 64: the schedule kernel writes the work list into the scratch), SwiGLU
    sizes1 = [0 if rng.random() < 0.1 else int(rng.integers(1, 70)) for _ in range(256)]
    A, B, off, rows, R = _inputs(sizes1, 512, 1024, seed=1)
    print(f"noalloc call 1: E=256 R={R} SwiGLU", flush=True)
    _run_both(A, B, off, rows, R, moe.MOE_EPI_SWIGLU)
    # 2) a smaller input right after: 100 experts, fewer items, NONE epilogue
    sizes2 = [int(rng.integers(0, 9)) for _ in range(100)]
    A, B, off, rows, R = _inputs(sizes2, 256, 512, seed=2)
    print(f"noalloc call 2: E=100 R={R} NONE", flush=True)
    _run_both(A, B, off, rows, R, moe.MOE_EPI_NONE)
    # 3) few experts (work items derived in the kernels; K split across waves)
    A, B, off, rows, R = _inputs([32] * 8, 2048, 512, seed=3)
    print(f"noalloc call 3: E=8 R={R} NONE (K split)", flush=True)
    _run_both(A, B, off, rows, R, moe.MOE_EPI_NONE)
