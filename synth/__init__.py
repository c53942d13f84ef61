"""Seeded synthetic inputs for the NVFP4 MoE path.

The one input generator both sides use: the tests feed its arrays to the CPU
oracle and to the HIP library, and the benchmark feeds them to the HIP library.
It holds none of the method's arithmetic -- only random draws, the bias of the
skewed router logits and the rounding of the drawn activations to bf16.

Recipe (seed 0 unless stated):
  * ``np.random.SeedSequence(seed).spawn(2 + 2*E)``: child 0 draws the router
    logits, child 1 the activations, child 2+2e the gate/up weights of expert e
    and child 3+2e its down weights (for the single grouped GEMM, child 2+2e
    draws B of expert e).
  * Router logits: float64 N(0, 1) cast to float32; the skewed workload adds
    beta * (-s * ln(e + 1)) with s = 1.1 (a Zipf(s) prior over experts) before
    the cast.
  * Activations: float32 N(0, 1) rounded to bf16 (round to nearest even).
  * Weights: 0.02 * float32 N(0, 1), kept in float32 (quantised to NVFP4 by
    whoever consumes them).
The workload shapes are the ones the pages quote for GLM-5-NVFP4 decode: 256
experts, 8 active per token, hidden 6144, expert intermediate 2048, ~32 rows
per expert at 1024 tokens ("Tracing the Failure: Debugging CUTLASS FP4 Tile
Configurations on Blackwell SM120", section "The Broader Context").
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Layer:
    """One MoE layer: T tokens, E experts, top-k, hidden H, expert intermediate I."""
    name: str
    T: int
    E: int
    k: int
    H: int
    I: int
    zipf_beta: float = 0.0

    @property
    def R(self) -> int:
        return self.T * self.k


@dataclass(frozen=True)
class Gemm:
    """One grouped GEMM with E equal groups of M rows, contraction K, N columns."""
    name: str
    E: int
    M: int
    K: int
    N: int


TINY = Layer("tiny_layer_t16_e4_k2_h256_i256", T=16, E=4, k=2, H=256, I=256)
GEMM_DECODE = Gemm("grouped_gemm_e8_m32_k6144_n2048", E=8, M=32, K=6144, N=2048)
LAYER_DECODE = Layer("layer_decode_t1024_e256_k8_h6144_i2048", T=1024, E=256, k=8, H=6144, I=2048)
LAYER_SKEWED = Layer("layer_skewed_t512_e256_k8_h6144_i2048_zipf1.1", T=512, E=256, k=8, H=6144,
                     I=2048, zipf_beta=0.37)
LAYER_PREFILL = Layer("layer_prefill_t16384_e256_k8_h6144_i2048", T=16384, E=256, k=8, H=6144, I=2048)
# One GPU's share of the decode layer under 8-way expert parallelism (32 local experts,
# ~32 rows each, as many rows as tokens x top-8 / 8) and under 8-way tensor parallelism
# (all 256 experts, intermediate 2048 / 8 = 256 per GPU).
LAYER_EP8 = Layer("layer_ep8_share_t128_e32_k8_h6144_i2048", T=128, E=32, k=8, H=6144, I=2048)
LAYER_TP8 = Layer("layer_tp8_share_t1024_e256_k8_h6144_i256", T=1024, E=256, k=8, H=6144, I=256)
# The dense special case: one group, large square GEMM.
GEMM_DENSE = Gemm("dense_gemm_e1_m8192_k8192_n8192", E=1, M=8192, K=8192, N=8192)

ZIPF_S = 1.1


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def children(seed: int, E: int):
    return np.random.SeedSequence(seed).spawn(2 + 2 * E)


def _gen(child) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(child))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def router_logits(L: Layer, seed: int = 0) -> np.ndarray:
    g = _gen(children(seed, L.E)[0])
    z = g.standard_normal((L.T, L.E), dtype=np.float64)
    if L.zipf_beta:
        z = z + L.zipf_beta * (-ZIPF_S * np.log(np.arange(1, L.E + 1, dtype=np.float64)))[None, :]
    return z.astype(np.float32)


def activations_bf16(rows: int, cols: int, child) -> np.ndarray:
    g = _gen(child)
    x = np.empty((rows, cols), np.float32)
    g.standard_normal(out=x, dtype=np.float32)
    return bf16_bits(x)


def layer_activations(L: Layer, seed: int = 0) -> np.ndarray:
    """bf16 bits [T, H]."""
    return activations_bf16(L.T, L.H, children(seed, L.E)[1])


def weight_f32(rows: int, cols: int, child) -> np.ndarray:
    g = _gen(child)
    w = np.empty((rows, cols), np.float32)
    g.standard_normal(out=w, dtype=np.float32)
    w *= np.float32(0.02)
    return w


def layer_w1(L: Layer, e: int, seed: int = 0) -> np.ndarray:
    """Gate/up weights of expert e, float32 [2I, H] (rows 0..I-1 gate, I..2I-1 up)."""
    return weight_f32(2 * L.I, L.H, children(seed, L.E)[2 + 2 * e])


def layer_w2(L: Layer, e: int, seed: int = 0) -> np.ndarray:
    """Down weights of expert e, float32 [H, I]."""
    return weight_f32(L.H, L.I, children(seed, L.E)[3 + 2 * e])


def gemm_a_bf16(G: Gemm, seed: int = 0) -> np.ndarray:
    """Activations of the single grouped GEMM, bf16 bits [E*M, K]."""
    return activations_bf16(G.E * G.M, G.K, children(seed, G.E)[1])


def gemm_b(G: Gemm, e: int, seed: int = 0) -> np.ndarray:
    """Weights of group e of the single grouped GEMM, float32 [N, K]."""
    return weight_f32(G.N, G.K, children(seed, G.E)[2 + 2 * e])


def per_expert(fn, experts, threads: int | None = None):
    """Map fn over experts on a thread pool (numpy draws release the GIL); keeps order."""
    with ThreadPoolExecutor(threads or _threads()) as ex:
        return list(ex.map(fn, experts))
