"""Python binding of libmoe_nvfp4 (the MI355X NVFP4 MoE hot path).

Argument marshalling only: every function here passes device pointers of torch tensors
and torch's current HIP stream to the C ABI declared in ``include/moe_nvfp4.h`` and
raises :class:`MoeError` on a non-zero status.  Every step of the path runs in the
library's gfx950 kernels; there is no fallback.  If the library has not been built the
import of any entry point fails loudly.

Functions with the C names take caller-allocated tensors exactly like the C calls.  The
``*_alloc`` helpers allocate outputs and workspaces with torch; :func:`pack_weights` turns
an NVFP4 weight tensor into the packed layout once; :class:`MoELayerPlan` pre-allocates one
MoE layer's buffers and sequences its six calls.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_nvfp4.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
MOE_DTYPE_BF16, MOE_DTYPE_F32 = 0, 1
MOE_GS_STATIC, MOE_GS_DYNAMIC = 0, 1
MOE_EPI_NONE, MOE_EPI_SWIGLU, MOE_EPI_SWIGLU_NVFP4 = 0, 1, 2
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_PACKED = 0, 1

EXPORTED = [
    "moe_status_string", "moe_last_hip_error",
    "moe_route_permute_workspace", "moe_route_permute",
    "moe_quantize_nvfp4_workspace", "moe_quantize_nvfp4",
    "moe_grouped_gemm_nvfp4_workspace", "moe_grouped_gemm_nvfp4_amax_slots",
    "moe_grouped_gemm_nvfp4_can_implement", "moe_grouped_gemm_nvfp4", "moe_grouped_gemm_nvfp4_noalloc",
    "moe_pack_weights_nvfp4_bytes", "moe_pack_weights_nvfp4",
    "moe_finalize",
]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str, hip_error: int = 0):
        super().__init__(f"{fn}: status {status} ({msg})" + (f", hipError {hip_error}" if hip_error else ""))
        self.status = status


class moe_gemm_args(C.Structure):
    _fields_ = [
        ("A", C.c_void_p), ("A_sf", C.c_void_p), ("A_gs", C.c_void_p), ("A_rows", C.c_void_p),
        ("rows_A", C.c_int64),
        ("B", C.c_void_p), ("B_sf", C.c_void_p), ("B_gs", C.c_void_p),
        ("expert_offsets", C.c_void_p),
        ("E", C.c_int32), ("N", C.c_int32), ("K", C.c_int32),
        ("R", C.c_int64),
        ("epilogue", C.c_int32),
        ("D", C.c_void_p), ("amax_out", C.c_void_p),
        ("B_layout", C.c_int32),
        ("D_sf", C.c_void_p), ("D_gs", C.c_void_p),
    ]


_lib = None


def lib():
    """The loaded C library; raises if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc, gfx950); there is no fallback path")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, sz = C.c_void_p, C.c_int, C.c_int64, C.c_size_t
        args_p = C.POINTER(moe_gemm_args)
        sig = {
            "moe_status_string": (C.c_char_p, [i32]),
            "moe_last_hip_error": (i32, []),
            "moe_route_permute_workspace": (sz, [i32, i32, i32]),
            "moe_route_permute": (i32, [P, i32, i32, i32, P, P, P, P, P, P, sz, P]),
            "moe_quantize_nvfp4_workspace": (sz, [i64, i64]),
            "moe_quantize_nvfp4": (i32, [P, i32, i64, i64, P, P, P, i32, P, i64, P, sz, P]),
            "moe_grouped_gemm_nvfp4_workspace": (sz, [args_p]),
            "moe_grouped_gemm_nvfp4_amax_slots": (i64, [args_p]),
            "moe_grouped_gemm_nvfp4_can_implement": (i32, [args_p]),
            "moe_grouped_gemm_nvfp4": (i32, [args_p, P, sz, P]),
            "moe_grouped_gemm_nvfp4_noalloc": (i32, [args_p, P]),
            "moe_pack_weights_nvfp4_bytes": (sz, [i64, i32]),
            "moe_pack_weights_nvfp4": (i32, [P, P, i64, i32, P, P]),
            "moe_finalize": (i32, [P, i64, P, P, i32, i32, i32, P, P]),
        }
        for name, (res, argt) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, argt
        _lib = L
    return _lib


def _check(fn: str, st: int):
    if st != MOE_OK:
        L = lib()
        raise MoeError(fn, st, L.moe_status_string(st).decode(),
                       L.moe_last_hip_error() if st == MOE_ERR_HIP else 0)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _ws(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ---- the C entry points ------------------------------------------------------------

def moe_route_permute(logits, k, topk_ids, topk_w, expert_offsets, row_src, token_slot_row,
                      ws, stream=None):
    T, E = logits.shape
    _check("moe_route_permute", lib().moe_route_permute(
        _p(logits), T, E, k, _p(topk_ids), _p(topk_w), _p(expert_offsets), _p(row_src),
        _p(token_slot_row), _p(ws), ws.numel(), _stream(stream)))


def moe_quantize_nvfp4(x, q, sf, gs, gs_mode=MOE_GS_DYNAMIC, amax_in=None, ws=None, stream=None):
    rows, cols = x.shape
    dt = {torch.bfloat16: MOE_DTYPE_BF16, torch.float32: MOE_DTYPE_F32}[x.dtype]
    if ws is None:
        ws = _ws(lib().moe_quantize_nvfp4_workspace(rows, cols), x.device)
    _check("moe_quantize_nvfp4", lib().moe_quantize_nvfp4(
        _p(x), dt, rows, cols, _p(q), _p(sf), _p(gs), gs_mode, _p(amax_in),
        0 if amax_in is None else amax_in.numel(), _p(ws), ws.numel(), _stream(stream)))


def make_gemm_args(A, A_sf, A_gs, B, B_sf, B_gs, expert_offsets, R, epilogue, D=None,
                   amax_out=None, A_rows=None, N=None, K=None, D_sf=None, D_gs=None) -> moe_gemm_args:
    """B / B_sf are row-major NVFP4 [E, N, K/2] / [E, N, K/16]; pass B_sf=None and B as the
    packed buffer [E, N*K*9/16 bytes] (moe_pack_weights_nvfp4) with N and K for the packed
    layout.  D_sf / D_gs: scales and static global scale of D (SWIGLU_NVFP4 only)."""
    packed = B_sf is None
    if packed:
        E = B.shape[0]
    else:
        E, N, half_k = B.shape
        K = 2 * half_k
    a = moe_gemm_args()
    a.A, a.A_sf, a.A_gs, a.A_rows = _p(A), _p(A_sf), _p(A_gs), _p(A_rows)
    a.rows_A = A.shape[0]
    a.B, a.B_sf, a.B_gs, a.expert_offsets = _p(B), _p(B_sf), _p(B_gs), _p(expert_offsets)
    a.E, a.N, a.K, a.R, a.epilogue = E, N, K, int(R), epilogue
    a.D, a.amax_out = _p(D), _p(amax_out)
    a.B_layout = MOE_LAYOUT_PACKED if packed else MOE_LAYOUT_ROWMAJOR
    a.D_sf, a.D_gs = _p(D_sf), _p(D_gs)
    return a


def moe_grouped_gemm_nvfp4_workspace(args: moe_gemm_args) -> int:
    return lib().moe_grouped_gemm_nvfp4_workspace(C.byref(args))


def moe_grouped_gemm_nvfp4_amax_slots(args: moe_gemm_args) -> int:
    return lib().moe_grouped_gemm_nvfp4_amax_slots(C.byref(args))


def moe_grouped_gemm_nvfp4_can_implement(args: moe_gemm_args) -> int:
    return lib().moe_grouped_gemm_nvfp4_can_implement(C.byref(args))


def moe_grouped_gemm_nvfp4(args: moe_gemm_args, ws, stream=None):
    _check("moe_grouped_gemm_nvfp4",
           lib().moe_grouped_gemm_nvfp4(C.byref(args), _p(ws), ws.numel(), _stream(stream)))


MOE_NOALLOC_SCRATCH_BYTES = 1 << 20


def moe_grouped_gemm_nvfp4_noalloc(args: moe_gemm_args, stream=None):
    """The grouped GEMM with the library's static device scratch in place of a workspace
    (nothing is allocated; calls that overlap on one GPU race)."""
    _check("moe_grouped_gemm_nvfp4_noalloc",
           lib().moe_grouped_gemm_nvfp4_noalloc(C.byref(args), _stream(stream)))


def moe_pack_weights_nvfp4(B, B_sf, packed, stream=None):
    """B [..., K/2] codes and B_sf [..., K/16] scales of rows*K elements -> packed bytes."""
    K = B.shape[-1] * 2
    rows = B.numel() // (K // 2)
    _check("moe_pack_weights_nvfp4", lib().moe_pack_weights_nvfp4(
        _p(B), _p(B_sf), rows, K, _p(packed), _stream(stream)))


def moe_finalize(Y, topk_w, token_slot_row, out, stream=None):
    T, k = topk_w.shape
    H = out.shape[1]
    _check("moe_finalize", lib().moe_finalize(
        _p(Y), Y.shape[0], _p(topk_w), _p(token_slot_row), T, k, H, _p(out), _stream(stream)))


# ---- allocating helpers ------------------------------------------------------------

@dataclass
class NVFP4Tensor:
    """Device NVFP4 tensor: codes [..., C/2] u8, scales [..., C/16] u8, global scale(s) f32."""
    q: torch.Tensor
    sf: torch.Tensor
    gs: torch.Tensor


@dataclass
class PackedWeights:
    """Expert weights [E, N, K] in the packed layout: data [E, N*K*9/16] u8, gs [E] f32."""
    data: torch.Tensor
    gs: torch.Tensor
    N: int
    K: int


def pack_weights(W: NVFP4Tensor, stream=None) -> PackedWeights:
    E, N, half_k = W.q.shape
    K = 2 * half_k
    nbytes = lib().moe_pack_weights_nvfp4_bytes(E * N, K)
    if nbytes == 0:
        raise MoeError("moe_pack_weights_nvfp4_bytes", MOE_ERR_UNSUPPORTED, "rows % 32 or K % 256")
    data = torch.empty(E, nbytes // E, dtype=torch.uint8, device=W.q.device)
    moe_pack_weights_nvfp4(W.q, W.sf, data, stream)
    return PackedWeights(data, W.gs, N, K)


def quantize_alloc(x: torch.Tensor, gs=None, amax_in=None, stream=None) -> NVFP4Tensor:
    rows, cols = x.shape
    q = torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device)
    sf = torch.empty(rows, cols // 16, dtype=torch.uint8, device=x.device)
    mode = MOE_GS_STATIC if gs is not None else MOE_GS_DYNAMIC
    g = gs if gs is not None else torch.empty(1, dtype=torch.float32, device=x.device)
    moe_quantize_nvfp4(x, q, sf, g, mode, amax_in, stream=stream)
    return NVFP4Tensor(q, sf, g)


def route_permute_alloc(logits: torch.Tensor, k: int, stream=None):
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_src = torch.empty(T * k, dtype=torch.int32, device=dev)
    tsr = torch.empty(T * k, dtype=torch.int32, device=dev)
    ws = _ws(lib().moe_route_permute_workspace(T, E, k), dev)
    moe_route_permute(logits, k, ids, w, off, row_src, tsr, ws, stream)
    return ids, w, off, row_src, tsr


def _gemm_args_for(A: NVFP4Tensor, B, expert_offsets, R, epilogue, D, A_rows):
    if isinstance(B, PackedWeights):
        return make_gemm_args(A.q, A.sf, A.gs, B.data, None, B.gs, expert_offsets, R, epilogue, D,
                              None, A_rows, N=B.N, K=B.K)
    return make_gemm_args(A.q, A.sf, A.gs, B.q, B.sf, B.gs, expert_offsets, R, epilogue, D, None, A_rows)


def grouped_gemm_alloc(A: NVFP4Tensor, B, expert_offsets, R, epilogue=MOE_EPI_NONE,
                       A_rows=None, stream=None, D_gs=None):
    """B: NVFP4Tensor (row-major) or PackedWeights.  Returns D (and the partial-maxima tensor
    for SWIGLU; an NVFP4Tensor with global scale D_gs for SWIGLU_NVFP4)."""
    N = B.N if isinstance(B, PackedWeights) else B.q.shape[1]
    dev = A.q.device
    if epilogue == MOE_EPI_SWIGLU_NVFP4:
        I = N // 2
        Dq = NVFP4Tensor(torch.empty(int(R), I // 2, dtype=torch.uint8, device=dev),
                         torch.empty(int(R), I // 16, dtype=torch.uint8, device=dev), D_gs)
        a = _gemm_args_for(A, B, expert_offsets, R, epilogue, Dq.q, A_rows)
        a.D_sf, a.D_gs = _p(Dq.sf), _p(D_gs)
        _check("moe_grouped_gemm_nvfp4_can_implement", moe_grouped_gemm_nvfp4_can_implement(a))
        moe_grouped_gemm_nvfp4(a, _ws(moe_grouped_gemm_nvfp4_workspace(a), dev), stream)
        return Dq
    cols = N if epilogue == MOE_EPI_NONE else N // 2
    D = torch.empty(int(R), cols, dtype=torch.bfloat16, device=dev)
    a = _gemm_args_for(A, B, expert_offsets, R, epilogue, D, A_rows)
    amax = None
    if epilogue == MOE_EPI_SWIGLU:
        amax = torch.empty(max(moe_grouped_gemm_nvfp4_amax_slots(a), 1), dtype=torch.float32, device=dev)
        a.amax_out = _p(amax)
    _check("moe_grouped_gemm_nvfp4_can_implement", moe_grouped_gemm_nvfp4_can_implement(a))
    ws = _ws(moe_grouped_gemm_nvfp4_workspace(a), dev)
    moe_grouped_gemm_nvfp4(a, ws, stream)
    return (D, amax) if epilogue == MOE_EPI_SWIGLU else D


class MoELayerPlan:
    """Pre-allocated buffers and argument blocks for repeated forward passes of one layer
    shape (what a serving loop or a benchmark reuses): no allocation per call."""

    def __init__(self, T: int, E: int, k: int, H: int, I: int, W1, W2, device="cuda", static_g2=None):
        """W1 / W2: NVFP4Tensor (row-major) or PackedWeights (the fast decode layout).
        static_g2: a caller-calibrated global scale (one-element f32 device tensor) for the
        SwiGLU output; with it the gate/up GEMM requantises in its epilogue
        (MOE_EPI_SWIGLU_NVFP4) and requantize() does nothing."""
        self.T, self.E, self.k, self.H, self.I = T, E, k, H, I
        R = T * k
        self.R = R
        dev = torch.device(device)
        z = lambda *s, dt: torch.empty(*s, dtype=dt, device=dev)
        self.ids, self.w = z(T, k, dt=torch.int32), z(T, k, dt=torch.float32)
        self.off, self.row_src, self.tsr = z(E + 1, dt=torch.int32), z(R, dt=torch.int32), z(R, dt=torch.int32)
        self.xq = NVFP4Tensor(z(T, H // 2, dt=torch.uint8), z(T, H // 16, dt=torch.uint8), z(1, dt=torch.float32))
        self.act = z(R, I, dt=torch.bfloat16)
        self.actq = NVFP4Tensor(z(R, I // 2, dt=torch.uint8), z(R, I // 16, dt=torch.uint8), z(1, dt=torch.float32))
        self.Y = z(R, H, dt=torch.bfloat16)
        self.out = z(T, H, dt=torch.bfloat16)
        self.W1, self.W2 = W1, W2
        self.fused = static_g2 is not None
        if self.fused:
            self.actq.gs.copy_(static_g2.reshape(1))
            self.args1 = _gemm_args_for(self.xq, W1, self.off, R, MOE_EPI_SWIGLU_NVFP4, self.actq.q, self.row_src)
            self.args1.D_sf, self.args1.D_gs = _p(self.actq.sf), _p(self.actq.gs)
        else:
            self.args1 = _gemm_args_for(self.xq, W1, self.off, R, MOE_EPI_SWIGLU, self.act, self.row_src)
            self.amax = z(max(moe_grouped_gemm_nvfp4_amax_slots(self.args1), 1), dt=torch.float32)
            self.args1.amax_out = _p(self.amax)
        self.args2 = _gemm_args_for(self.actq, W2, self.off, R, MOE_EPI_NONE, self.Y, None)
        for a in (self.args1, self.args2):
            _check("moe_grouped_gemm_nvfp4_can_implement", moe_grouped_gemm_nvfp4_can_implement(a))
        L = lib()
        self.ws_route = _ws(L.moe_route_permute_workspace(T, E, k), dev)
        self.ws_q1 = _ws(L.moe_quantize_nvfp4_workspace(T, H), dev)
        self.ws_q2 = _ws(L.moe_quantize_nvfp4_workspace(R, I), dev)
        self.ws_g1 = _ws(moe_grouped_gemm_nvfp4_workspace(self.args1), dev)
        self.ws_g2 = _ws(moe_grouped_gemm_nvfp4_workspace(self.args2), dev)

    # the six calls of the layer, individually (the benchmark times them one by one)
    def route(self, logits, stream=None):
        moe_route_permute(logits, self.k, self.ids, self.w, self.off, self.row_src, self.tsr,
                          self.ws_route, stream)

    def quantize_input(self, x, stream=None):
        moe_quantize_nvfp4(x, self.xq.q, self.xq.sf, self.xq.gs, MOE_GS_DYNAMIC, None, self.ws_q1, stream)

    def gemm1(self, stream=None):
        moe_grouped_gemm_nvfp4(self.args1, self.ws_g1, stream)

    def requantize(self, stream=None):
        if self.fused:   # done in the gate/up GEMM's epilogue
            return
        moe_quantize_nvfp4(self.act, self.actq.q, self.actq.sf, self.actq.gs, MOE_GS_DYNAMIC, self.amax,
                           self.ws_q2, stream)

    def gemm2(self, stream=None):
        moe_grouped_gemm_nvfp4(self.args2, self.ws_g2, stream)

    def finalize(self, stream=None):
        moe_finalize(self.Y, self.w, self.tsr, self.out, stream)

    def forward(self, logits, x, stream=None):
        # One stream.  Routing (logits) and token quantisation (x) are independent, but running
        # the quantiser on a second stream beside the routing kernels made the layer slower:
        # the two cross-stream waits cost more than the ~15 us the overlap saves.
        main = stream if stream is not None else torch.cuda.current_stream()
        self.route(logits, main)
        self.quantize_input(x, main)
        self.gemm1(main)
        self.requantize(main)
        self.gemm2(main)
        self.finalize(main)
        return self.out

    def graph(self, logits, x) -> "torch.cuda.CUDAGraph":
        """Capture one forward pass over the input buffers `logits` and `x` into a HIP graph.
        replay() reruns the whole layer on whatever those buffers hold at the time, writing
        the same output buffers; a serving loop copies each batch into them first.  The pass
        allocates nothing and records no memory-set node: every buffer is cleared or written
        by the library's own kernels."""
        self.forward(logits, x)              # one eager pass first (lazy initialisation)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(logits, x)
        torch.cuda.synchronize()
        return g


def quantize_experts(W: torch.Tensor, stream=None) -> NVFP4Tensor:
    """NVFP4-quantise stacked expert weights W [E, rows, cols] (f32 or bf16), one dynamic
    global scale per expert, into one contiguous [E, rows, cols/2] tensor."""
    E, rows, cols = W.shape
    dev = W.device
    q = torch.empty(E, rows, cols // 2, dtype=torch.uint8, device=dev)
    sf = torch.empty(E, rows, cols // 16, dtype=torch.uint8, device=dev)
    gs = torch.empty(E, dtype=torch.float32, device=dev)
    ws = _ws(lib().moe_quantize_nvfp4_workspace(rows, cols), dev)
    for e in range(E):
        moe_quantize_nvfp4(W[e], q[e], sf[e], gs[e:e + 1], MOE_GS_DYNAMIC, None, ws, stream)
    return NVFP4Tensor(q, sf, gs)
