"""CPU oracle for the NVFP4 MoE hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It wraps ``liboracle.so`` (plain C, built from
``oracle.c`` by ``build()``) with numpy marshalling.  It shares no code with
the HIP library; the definitions and their sources are in ``oracle.h``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (plain C11, OpenMP, no FP contraction)."""
    cmd = ["gcc", "-std=c11", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           os.path.join(_HERE, "oracle.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i64, i32, f32, f64 = C.c_int64, C.c_int, C.c_float, C.c_double
        sig = {
            "orc_e2m1_value": (f64, [i32]),
            "orc_e4m3_value": (f64, [i32]),
            "orc_e4m3_round": (i32, [f32]),
            "orc_e2m1_round": (i32, [f32]),
            "orc_bf16_round": (C.c_uint16, [f64]),
            "orc_bf16_value": (f64, [C.c_uint16]),
            "orc_quantize_nvfp4": (None, [P, i64, i64, i32, f32, P, P, P]),
            "orc_route": (None, [P, i32, i32, i32, P, P]),
            "orc_permute": (None, [P, i32, i32, i32, P, P, P]),
            "orc_grouped_gemm_rows": (None, [P, P, f32, P, P, P, P, P, i32, i32, i32, P, i64, P]),
            "orc_swiglu": (None, [P, i64, i32, P]),
            "orc_finalize": (None, [P, P, P, i32, i32, i32, P, P]),
            "orc_num_threads": (i32, []),
            "orc_set_num_threads": (None, [i32]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---- element formats -------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def e4m3_round(t: float) -> int:
    return lib().orc_e4m3_round(float(t))


def e2m1_round(u: float) -> int:
    return lib().orc_e2m1_round(float(u))


def bf16_round(x: float) -> int:
    return lib().orc_bf16_round(float(x))


def bf16_value(b: int) -> float:
    return lib().orc_bf16_value(int(b))


# ---- quantisation ------------------------------------------------------------

class NVFP4:
    """An NVFP4 tensor: codes [rows, C/2] u8, e4m3 scales [rows, C/16] u8, global scale g."""

    def __init__(self, q: np.ndarray, sf: np.ndarray, g: float):
        self.q, self.sf, self.g = q, sf, np.float32(g)

    @property
    def shape(self):
        return (self.q.shape[0], self.q.shape[1] * 2)


def quantize(x: np.ndarray, g: float | None = None) -> NVFP4:
    """Quantise float32 x[rows, C] (dynamic global scale unless g is given)."""
    x = _c(x, np.float32)
    rows, cols = x.shape
    assert cols % 16 == 0
    q = np.empty((rows, cols // 2), np.uint8)
    sf = np.empty((rows, cols // 16), np.uint8)
    gout = np.zeros(1, np.float32)
    lib().orc_quantize_nvfp4(_p(x), rows, cols, 1 if g is None else 0,
                             0.0 if g is None else float(g), _p(q), _p(sf), _p(gout))
    return NVFP4(q, sf, gout[0] if g is None else np.float32(g))


def quantize_bf16(xb: np.ndarray, g: float | None = None) -> NVFP4:
    """Quantise bf16 bit patterns (uint16) -- widened exactly to float32 first."""
    x = (np.ascontiguousarray(xb, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
    return quantize(x, g)


# ---- routing -----------------------------------------------------------------

def route(logits: np.ndarray, k: int):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    lib().orc_route(_p(logits), T, E, k, _p(ids), _p(w))
    return ids, w


def permute(ids: np.ndarray, E: int):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    off = np.empty(E + 1, np.int32)
    row_src = np.empty(T * k, np.int32)
    tsr = np.empty(T * k, np.int32)
    lib().orc_permute(_p(ids), T, E, k, _p(off), _p(row_src), _p(tsr))
    return off, row_src, tsr


# ---- grouped GEMM, SwiGLU, FINALIZE ----------------------------------------

def grouped_gemm(A: NVFP4, B_q: np.ndarray, B_sf: np.ndarray, gB: np.ndarray,
                 offsets: np.ndarray, A_rows: np.ndarray | None = None,
                 rows: np.ndarray | None = None) -> np.ndarray:
    """Unrounded FP64 y[len(rows), N]; B_q [E, N, K/2], B_sf [E, N, K/16], gB [E]."""
    E, N, half_k = B_q.shape
    K = half_k * 2
    offsets = _c(offsets, np.int32)
    R = int(offsets[-1])
    rows = np.arange(R, dtype=np.int32) if rows is None else _c(rows, np.int32)
    y = np.empty((len(rows), N), np.float64)
    A_rows_c = None if A_rows is None else _c(A_rows, np.int32)
    lib().orc_grouped_gemm_rows(_p(A.q), _p(A.sf), A.g, _p(A_rows_c), _p(_c(B_q, np.uint8)),
                                _p(_c(B_sf, np.uint8)), _p(_c(gB, np.float32)), _p(offsets),
                                E, N, K, _p(rows), len(rows), _p(y))
    return y


def swiglu(y1: np.ndarray) -> np.ndarray:
    """bf16 bits act[R, I] from FP64 y1[R, 2I]."""
    y1 = _c(y1, np.float64)
    R, two_i = y1.shape
    act = np.empty((R, two_i // 2), np.uint16)
    lib().orc_swiglu(_p(y1), R, two_i // 2, _p(act))
    return act


def finalize(y2: np.ndarray, w: np.ndarray, token_slot_row: np.ndarray):
    """(FP64 out[T, H], bf16 bits out[T, H])."""
    y2 = _c(y2, np.float64)
    w = _c(w, np.float64)
    T, k = w.shape
    H = y2.shape[1]
    o64 = np.empty((T, H), np.float64)
    o16 = np.empty((T, H), np.uint16)
    lib().orc_finalize(_p(y2), _p(w), _p(_c(token_slot_row, np.int32)), T, k, H, _p(o64), _p(o16))
    return o64, o16


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """OpenMP threads for the following oracle calls."""
    lib().orc_set_num_threads(int(n))


# ---- the whole layer ---------------------------------------------------------

class LayerResult:
    pass


def moe_layer(logits, x_bf16, W1: list, W2: list, k: int, act_g: float | None = None) -> LayerResult:
    """The MoE layer step by step: route, permute, quantise x, GEMM1, SwiGLU,
    requantise, GEMM2, FINALIZE.  W1[e] / W2[e] are NVFP4 weights of expert e
    ([2I, H] and [H, I]).  act_g: a static global scale for the requantisation of the
    SwiGLU output (the fused-epilogue mode); None for the dynamic per-tensor scale.
    Returns every intermediate."""
    E = len(W1)
    r = LayerResult()
    r.ids, r.w = route(logits, k)
    r.offsets, r.row_src, r.token_slot_row = permute(r.ids, E)
    r.xq = quantize_bf16(x_bf16)
    B1q = np.stack([w.q for w in W1]); B1s = np.stack([w.sf for w in W1])
    g1 = np.array([w.g for w in W1], np.float32)
    r.y1 = grouped_gemm(r.xq, B1q, B1s, g1, r.offsets, A_rows=r.row_src)
    r.act = swiglu(r.y1)
    r.actq = quantize_bf16(r.act, g=act_g)
    B2q = np.stack([w.q for w in W2]); B2s = np.stack([w.sf for w in W2])
    g2 = np.array([w.g for w in W2], np.float32)
    r.y2 = grouped_gemm(r.actq, B2q, B2s, g2, r.offsets)
    r.out64, r.out16 = finalize(r.y2, r.w, r.token_slot_row)
    return r
