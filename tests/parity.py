"""Shared pieces of the GPU parity tests: device upload of oracle-side arrays and the
comparison rules.

Tolerances:
  * Integer and byte outputs (routing ids, offsets, permutation, quantised codes, block
    scales, global-scale bits): bit-exact.
  * bf16 outputs of the GEMM (NONE epilogue), FINALIZE and the whole layer: relative L2
    error <= 1e-2 and max |gpu - ref| <= 2e-2 against the oracle's unrounded FP64 value;
    an element with |ref| >= 8 also passes within one bf16 ulp of ref, because a single
    bf16 rounding step there already exceeds 2e-2.
  * bf16 SwiGLU output: the kernel rounds its fp32 gate/up values to bf16 before SwiGLU;
    where an fp32 value sits within its accumulation error of a bf16 rounding boundary the
    two sides may round differently, so each element is allowed one bf16 ulp of gate and of
    up propagated through silu(g) * u, plus one ulp of the result.
"""
from __future__ import annotations

import numpy as np
import torch

REL_L2 = 1e-2
MAX_ABS = 2e-2


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return dev(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def check_bf16(gpu_bits: np.ndarray, ref: np.ndarray, what: str) -> dict:
    got = bf16_values(gpu_bits).reshape(ref.shape)
    diff = np.abs(got - ref)
    big = np.abs(ref) >= 8
    ok = (diff <= MAX_ABS) | (big & (diff <= bf16_ulp(ref)))
    nref = np.linalg.norm(ref)
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got))
    stats = dict(what=what, n=int(ref.size), rel_l2=rel, max_abs=float(diff.max(initial=0.0)),
                 bad=int((~ok).sum()), max_ref=float(np.abs(ref).max(initial=0.0)))
    print(f"  {what}: {stats}", flush=True)
    assert np.isfinite(got).all(), what
    assert rel <= REL_L2, stats
    assert ok.all(), stats
    return stats


def swiglu_ref_and_bound(y1: np.ndarray, bf16_round) -> tuple[np.ndarray, np.ndarray]:
    """Unrounded FP64 SwiGLU of the oracle's y1 [R, 2I] (gate, up rounded to bf16 as the
    definition says) and the per-element bound described in the module docstring."""
    I = y1.shape[1] // 2
    r = lambda v: bf16_values(bf16_round(v))
    g, u = r(y1[:, :I]), r(y1[:, I:])
    sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))
    ref = silu * u
    bound = 1.01 * (np.abs(dsilu * u) * bf16_ulp(g) + np.abs(silu) * bf16_ulp(u)) + bf16_ulp(ref)
    return ref, bound


def np_bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest even, through torch (float64 -> float32 is
    exact for the values compared here only up to one float32 rounding; used only to
    build tolerance bounds, never as an expected value)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(torch.float32).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
