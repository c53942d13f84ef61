"""GPU parity: every entry point of libmoe_nvfp4, called through the C ABI, against the CPU
oracle on the same seeded inputs.  Oracle-side inputs are uploaded to the GPU; the GPU's
outputs are compared with what the oracle computes from the same inputs.  One test also
feeds a GPU output back to the oracle: the fused SwiGLU + NVFP4 epilogue is checked byte for
byte against the oracle's quantisation of the GPU's own SwiGLU output (the same decision in
the same precision), and separately, block by block, against the oracle's own pipeline.

Sizes: the small cases span several tiles and ragged tails; the full-size cases use the
decode layer (1024 tokens, 256 experts, top-8, hidden 6144, intermediate 2048), the
skewed decode layer (512 tokens, Zipf-biased router) and the prefill layer (16384
tokens), in the launch configuration the benchmark times.  The prefill layer is compared
in full up to the requantised activations and on 128 sampled tokens after that (the
oracle's down GEMM over every row would take minutes).
"""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.parity import (bf16_values, check_bf16, dev, dev_bf16, host_bits, np_bf16_round,
                          swiglu_ref_and_bound)

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("block_scaled_fp4_02_amd")


def log(msg):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------
# weights shared by the full-size layers (same seed and expert count -> same weights)

_WEIGHTS = {}


def layer_weights(L: synth.Layer):
    """Oracle-quantised NVFP4 weights of all experts, host and device copies (cached)."""
    key = (L.E, L.H, L.I)
    if key not in _WEIGHTS:
        log(f"generating + oracle-quantising weights E={L.E} H={L.H} I={L.I}")
        W1 = synth.per_expert(lambda e: oracle.quantize(synth.layer_w1(L, e)), range(L.E))
        W2 = synth.per_expert(lambda e: oracle.quantize(synth.layer_w2(L, e)), range(L.E))
        d1 = _weights(*stack(W1), packed=True)
        d2 = _weights(*stack(W2), packed=True)
        torch.cuda.synchronize()
        _WEIGHTS[key] = (W1, W2, d1, d2)
        log("weights ready")
    return _WEIGHTS[key]


def stack(W):
    return (np.stack([w.q for w in W]), np.stack([w.sf for w in W]),
            np.array([w.g for w in W], np.float32))


# ---------------------------------------------------------------------------------------
# routing and permutation: bit-exact

def _check_route(logits: np.ndarray, k: int):
    T, E = logits.shape
    log(f"route_permute T={T} E={E} k={k}")
    ids_o, w_o = oracle.route(logits, k) if T else (np.zeros((0, k), np.int32), np.zeros((0, k)))
    off_o, rs_o, tsr_o = oracle.permute(ids_o, E)
    ids, w, off, rs, tsr = moe.route_permute_alloc(dev(logits) if T else torch.empty(0, E, device="cuda"), k)
    torch.cuda.synchronize()
    assert np.array_equal(off.cpu().numpy(), off_o)
    if T:
        assert np.array_equal(ids.cpu().numpy(), ids_o)
        assert np.array_equal(rs.cpu().numpy(), rs_o)
        assert np.array_equal(tsr.cpu().numpy(), tsr_o)
        wg = w.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(wg - w_o) <= 1e-6 * w_o + 1e-30)  # exact zeros for -inf logits


@pytest.mark.parametrize("L", [synth.TINY, synth.LAYER_DECODE, synth.LAYER_SKEWED, synth.LAYER_PREFILL],
                         ids=lambda L: L.name)
def test_route_permute_workloads(L):
    _check_route(synth.router_logits(L), L.k)


@pytest.mark.parametrize("T,E,k", [(0, 8, 2), (1, 1, 1), (37, 1024, 32), (100, 8, 8), (300, 3, 2), (257, 256, 8),
                                   (50, 100, 4), (40, 300, 6), (33, 513, 8), (65, 64, 3), (129, 128, 2),
                                   # 10 chunks, and the largest batch whose workgroups histogram all
                                   # ids themselves; then 17 chunks through the count table (three
                                   # count batches, a one-token last chunk)
                                   (2305, 160, 8), (4096, 256, 8), (4097, 160, 8)])   # 1..16 logits per lane
def test_route_permute_edges(T, E, k):
    rng = np.random.default_rng(T * 7 + E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    _check_route(logits, k)


def test_route_permute_ties_and_infinities():
    rng = np.random.default_rng(3)
    logits = rng.integers(-2, 3, (513, 64)).astype(np.float32)  # heavy ties
    logits[5, :] = 0.0
    logits[6, 10] = -0.0
    logits[7, :] = -np.inf
    logits[7, 3] = 1.0
    _check_route(logits, 8)


# ---------------------------------------------------------------------------------------
# quantisation: bit-exact

def _check_quant(x32: np.ndarray, bf16: bool, g=None, partials=None):
    rows, cols = x32.shape
    log(f"quantize rows={rows} C={cols} bf16={bf16} static={g is not None} partials={partials is not None}")
    ref = oracle.quantize(x32, g)
    xt = dev_bf16(synth.bf16_bits(x32)) if bf16 else dev(x32)
    gs = dev(np.array([g], np.float32)) if g is not None else None
    amax_in = dev(partials) if partials is not None else None
    t = moe.quantize_alloc(xt, gs=gs, amax_in=amax_in)
    torch.cuda.synchronize()
    assert np.array_equal(t.q.cpu().numpy(), ref.q)
    assert np.array_equal(t.sf.cpu().numpy(), ref.sf)
    assert t.gs.cpu().numpy().view(np.uint32)[0] == np.float32(ref.g).view(np.uint32)


def test_quantize_activations_bf16():
    L = synth.LAYER_DECODE
    x = synth.bf16_to_f32(synth.layer_activations(L))
    _check_quant(x, bf16=True)


def test_quantize_weights_f32():
    L = synth.LAYER_DECODE
    _check_quant(synth.layer_w1(L, 3), bf16=False)


def test_quantize_static_and_partials():
    rng = np.random.default_rng(1)
    x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((300, 2048)).astype(np.float32) * 3))
    _check_quant(x, bf16=True, g=0.0123)
    parts = np.zeros(997, np.float32)
    parts[17] = np.abs(x).max()
    parts[3] = np.abs(x).max() / 2
    _check_quant(x, bf16=True, partials=parts)


@pytest.mark.parametrize("n", [1, 63, 64, 997, 1024, 1025, 4096])
@pytest.mark.parametrize("where", ["first", "last"])
def test_quantize_partial_maxima_counts(n, where):
    """Dynamic scale from n caller-provided maxima: up to 1024 the quantiser reduces them
    itself (no partial-maxima launch), above it a reduction launch comes first; the largest
    one first or last (the last lane's clamped loads), the others random and smaller."""
    rng = np.random.default_rng(n)
    x = synth.bf16_to_f32(synth.bf16_bits(rng.standard_normal((64, 512)).astype(np.float32)))
    m = np.float32(np.abs(x).max())
    parts = (rng.uniform(0, 1, n) * m * np.float32(0.9)).astype(np.float32)
    parts[0 if where == "first" else n - 1] = m
    _check_quant(x, bf16=True, partials=parts)


@pytest.mark.parametrize("case", ["zeros", "tiny_block", "wide_range", "one_block", "negzero", "subnormal_dynamic",
                                  "subnormal_static"])
def test_quantize_edges(case):
    rng = np.random.default_rng(5)
    g = None
    if case.startswith("subnormal"):
        # all-subnormal values with zeros among them: the dynamic g (amax / 2688) underflows to
        # 0, or a static g = 2^-149 makes s g underflow in the small blocks -- zero elements
        # and zero blocks must stay zero (0 / 0 counts as 0), the rest saturate
        tiny = np.float32(2.0 ** -149)
        x = (rng.integers(-40, 41, (6, 64)) * tiny).astype(np.float32)
        x[1, 16:32] = 0.0
        x[2, 5] = -0.0
        x[3, :16] = np.array([3, 0, -1, 0] * 4, np.float32) * tiny
        if case == "subnormal_static":
            g = float(tiny)
            x[4, :] = rng.standard_normal(64).astype(np.float32)
        _check_quant(x, bf16=False, g=g)
        return
    if case == "zeros":
        x = np.zeros((4, 64), np.float32)
    elif case == "tiny_block":
        x = rng.standard_normal((8, 64)).astype(np.float32)
        x[3, 16:32] *= 1e-7
    elif case == "wide_range":
        x = (rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    elif case == "one_block":
        x = rng.standard_normal((1, 16)).astype(np.float32)
    else:
        x = -np.zeros((3, 32), np.float32)
        x[1, 5] = 2.0
    _check_quant(x, bf16=False)


def test_quantize_rounding_thresholds():
    """Element quotients |x| / (s g) exactly on, and within 4 ulps of, every E2M1 rounding
    threshold and grid value, for block scales across the E4M3 range (static g).  The first
    element of each block fixes the block maximum at 6 s g."""
    g = np.float32(0.0123)
    six_g = np.float32(np.float32(6.0) * g)
    svals = np.array([6 * 2.0 ** -9, 0.375, 1.0, 2.5, 13.0, 104.0, 448.0], np.float32)
    targets = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 0.125],
                       np.float32)
    blocks = []
    for sv in svals:
        sg = np.float32(sv * g)
        amax = np.float32(sv * six_g)
        for k in range(-4, 5):
            vals = (targets * sg).astype(np.float32)
            vals = (vals.view(np.int32) + np.int32(k)).view(np.float32)
            vals = np.minimum(vals, amax)
            blk = np.concatenate([[amax], vals]).astype(np.float32)
            blk[1::2] *= -1
            blocks.append(blk)
    x = np.stack(blocks).reshape(len(svals), -1)
    _check_quant(x, bf16=False, g=float(g))


# ---------------------------------------------------------------------------------------
# grouped GEMM, NONE epilogue

def _gemm_case(sizes, K, N, gather, seed):
    rng = np.random.default_rng(seed)
    E = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(off[-1])
    T = max(R, 1) + 5
    A = oracle.quantize_bf16(synth.bf16_bits(rng.standard_normal((T, K)).astype(np.float32)))
    Bs = [oracle.quantize((rng.standard_normal((N, K)) * 0.02).astype(np.float32)) for _ in range(E)]
    A_rows = rng.integers(0, T, R).astype(np.int32) if gather else None
    return A, Bs, off, A_rows, R


def _weights(Bq, Bsf, gB, packed):
    dB = moe.NVFP4Tensor(dev(Bq), dev(Bsf), dev(gB))
    return moe.pack_weights(dB) if packed else dB


def _run_gemm_none(A, Bs, off, A_rows, R, label, packed=False):
    label = f"{label} {'packed' if packed else 'row-major'}"
    log(f"gemm NONE {label}: E={len(Bs)} R={R} N={Bs[0].q.shape[0]} K={A.q.shape[1] * 2}")
    Bq, Bsf, gB = stack(Bs)
    ref = oracle.grouped_gemm(A, Bq, Bsf, gB, off, A_rows=A_rows)
    dA = moe.NVFP4Tensor(dev(A.q), dev(A.sf), dev(np.array([A.g], np.float32)))
    dB = _weights(Bq, Bsf, gB, packed)
    D = moe.grouped_gemm_alloc(dA, dB, dev(off), R, moe.MOE_EPI_NONE,
                               A_rows=dev(A_rows) if A_rows is not None else None)
    torch.cuda.synchronize()
    got = host_bits(D)
    if R:
        check_bf16(got, ref, f"gemm NONE {label}")
        exact = (got == np_bf16_round(ref)).mean()
        print(f"  bf16-exact fraction {exact:.5f}", flush=True)
        assert exact > 0.98


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("sizes,K,N,gather", [
    ([8, 6, 9, 9], 256, 512, True),                       # tiny layer shape, gate/up as one GEMM
    ([0, 1, 31, 32, 33, 64, 65, 130, 0], 512, 256, True),  # ragged groups, empty groups, tails
    ([40, 0, 3], 1536, 256, False),                       # K split 2 ways inside a workgroup
    ([7, 25], 1024, 512, False),                          # K split 4 ways
    ([45, 3], 2048, 256, True),                           # K split 8 ways, 32 + 13 row chunks
    ([33] * 14, 2048, 2048, True),                        # K split 8 ways: 896 items looped over 256 workgroups
    ([20, 7, 32], 4096, 256, True),                       # K split 8 ways, 5 and 3 half steps per wave
    ([33] * 32, 512, 2048, False),                        # K split 2 ways: 1024 items looped over 512 workgroups
    ([1] * 60 + [0, 40, 2] + [1] * 37, 2048, 256, True),  # 100 experts, K split 8 ways: listed items looped
    ([1] * 60 + [0, 40, 2] + [1] * 37, 512, 256, True),   # 100 experts, K split 2 ways: listed items looped
    ([0, 3, 17, 48, 49, 1] * 42 + [5, 0, 60, 2], 1024, 1024, True),  # 256 experts, four-wave kernel, in-kernel lookup
    ([96, 130, 0, 250, 97] * 40, 1024, 512, False),       # 200 experts, eight-wave kernel, in-kernel lookup
    # expert counts that leave the in-kernel lookup's last lane part-filled (four experts per
    # lane): 127 experts in the four-wave kernel, 101 in the eight-wave kernel
    ([0, 3, 17, 48, 49, 1, 30] * 18 + [5], 1024, 1536, True),
    ([96, 130, 0, 250, 97] * 20 + [150], 1024, 512, True),
    ([0, 1, 2, 3, 5, 8, 13] * 150 + [40, 0], 256, 256, True),  # 1052 experts: two scan blocks in the schedule
    ([0, 0, 0], 256, 256, False),                         # no rows at all
    ([300], 256, 768, True),                              # one big group: several row chunks
    ([33] * 250 + [0, 64, 5] + [20] * 10, 256, 1024, True),  # enough groups for 4 tiles per wave
    # hundreds of rows per expert (several row chunks each, every remainder 1..47 rows) and,
    # in the second case, an odd number of 256-wide K steps
    ([0, 1, 96, 127, 128, 129, 300, 513], 512, 512, True),
    ([100, 200, 57, 0], 768, 256, True),
    # 32 experts x 16 n tiles with tens of rows each: the 64-row four-wave kernel (two items per
    # CU), every token-tile count 1..4 and an expert of 65 rows (two chunks)
    ([0, 1, 15, 16, 17, 31, 32, 33, 47, 48, 49, 63, 64, 65, 40, 20] + [30] * 16, 512, 4096, True),
    # >= 96 rows per expert and N % 512 == 0: the 8-wave kernel with 96-row chunks; the groups
    # end in every token-tile count 1..6
    ([1, 17, 33, 49, 65, 81, 95, 96, 97, 200, 600], 512, 512, True),
    # the 8-wave kernel with a single K step (only the loop's odd-step tail runs)
    ([96, 130, 200, 0, 60], 256, 1024, True),
])
def test_gemm_none_shapes(sizes, K, N, gather, packed):
    A, Bs, off, A_rows, R = _gemm_case(sizes, K, N, gather, seed=sum(sizes) + K + N)
    _run_gemm_none(A, Bs, off, A_rows, R, f"sizes={sizes}", packed)


def _random_gemm_shape(seed):
    """A seeded random grouped-GEMM shape: expert count on both sides of the in-kernel item
    lookup threshold (64) and of the K-split choice, ragged and empty groups, K and N in the
    supported multiples; bounded so that the oracle finishes in about a second."""
    rng = np.random.default_rng(9000 + seed)
    E = int(rng.choice([1, 3, 8, 24, 64, 65, 100, 257]))
    K = int(rng.choice([256, 512, 1024, 2048]))
    N = int(rng.choice([256, 512, 768, 1024]))
    while E * N * K > 48 * 2 ** 20 and N > 256:
        N = 256 if N == 768 else N // 2
    while E * N * K > 48 * 2 ** 20 and K > 256:
        K //= 2
    mode = rng.integers(0, 3)   # few rows, tens of rows, or a mix with large groups
    hi = {0: 4, 1: 70, 2: 300}[int(mode)]
    sizes = [0 if rng.random() < 0.25 else int(rng.integers(1, hi + 1)) for _ in range(E)]
    while sum(sizes) * N * K > 600 * 2 ** 20:
        sizes = [v // 2 for v in sizes]
    return sizes, K, N, bool(rng.random() < 0.6)


def test_gemm_none_single_k_step_several_n_tiles():
    """K = 256 with the NONE epilogue and enough items: each work item of the four-wave kernel
    covers two 256-row n tiles that share one dequantised activation tile (192 experts,
    ragged and empty groups, gathered rows, N 6144)."""
    rng = np.random.default_rng(4242)
    sizes = [0 if rng.random() < 0.1 else int(rng.integers(1, 61)) for _ in range(192)]
    A, Bs, off, A_rows, R = _gemm_case(sizes, 256, 6144, True, seed=4242)
    _run_gemm_none(A, Bs, off, A_rows, R, "single K step, two n tiles per item", True)


@pytest.mark.parametrize("seed", range(24))
def test_gemm_random_shapes(seed):
    """Seeded random shapes through the packed kernels (NONE on even seeds, SWIGLU on odd),
    and every fourth one on row-major weights as well."""
    sizes, K, N, gather = _random_gemm_shape(seed)
    A, Bs, off, A_rows, R = _gemm_case(sizes, K, N, gather, seed=seed)
    label = f"random seed={seed} E={len(sizes)} R={R} K={K} N={N} gather={gather}"
    for packed in ([True, False] if seed % 4 == 0 else [True]):
        if seed % 2 == 0:
            _run_gemm_none(A, Bs, off, A_rows, R, label, packed)
        else:
            _run_gemm_swiglu(A, Bs, off, A_rows, R, label, packed=packed)


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_gemm_none_decode_grouped_gemm_full(packed):
    """8 groups x 32 rows, K 6144, N 2048, NONE epilogue -- the single grouped GEMM."""
    G = synth.GEMM_DECODE
    A = oracle.quantize_bf16(synth.gemm_a_bf16(G))
    Bs = synth.per_expert(lambda e: oracle.quantize(synth.gemm_b(G, e)), range(G.E))
    off = np.arange(0, (G.E + 1) * G.M, G.M, dtype=np.int32)
    _run_gemm_none(A, Bs, off, None, G.E * G.M, "decode 8x32x6144x2048", packed)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("E,N,K,rows,packed", [
    # four-wave kernel: each expert's packed weights just under the 2^31-byte reach of its
    # 32-bit buffer descriptor (2,146,959,360 B), the second expert starting past 2^31 bytes
    (2, 116480, 32768, 16, True),
    # eight-wave kernel (>= 96 rows per expert, N % 512 == 0), likewise at the limit
    (2, 116224, 32768, 100, True),
    # K-split kernel: one 256-row expert with 7281 K steps of 2048 (2,147,254,272 B)
    (1, 256, 14911488, 16, True),
    # row-major weights (64-bit addressing, no such limit): 4.3 GB of codes, the second
    # expert starting past 2^32 bytes
    (2, 131072, 32768, 16, False),
], ids=["four_wave", "eight_wave", "k_split", "row_major"])
def test_gemm_largest_experts(E, N, K, rows, packed):
    """The largest experts the kernels address: random codes and scales (every E2M1 code,
    E4M3 scales 0.5-1.875), NONE epilogue, the first and last row of every expert against
    the oracle's rows (all N columns each)."""
    if packed:
        assert moe.lib().moe_pack_weights_nvfp4_bytes(N, K) <= (1 << 31) - 4096
    rng = np.random.default_rng(N + K + rows)
    R = E * rows
    log(f"gemm NONE largest experts: E={E} N={N} K={K} rows={rows}: generating")
    Bq = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    Bsf = rng.integers(0x30, 0x40, (E, N, K // 16), dtype=np.uint8)
    gB = np.full(E, 1.0 / 64, np.float32)
    A = oracle.NVFP4(rng.integers(0, 256, (R, K // 2), dtype=np.uint8),
                     rng.integers(0x30, 0x40, (R, K // 16), dtype=np.uint8), 1.0 / 8)
    off = np.arange(0, R + 1, rows, dtype=np.int32)
    dA = moe.NVFP4Tensor(dev(A.q), dev(A.sf), dev(np.array([A.g], np.float32)))
    dB = moe.NVFP4Tensor(dev(Bq), dev(Bsf), dev(gB))
    if packed:
        dB = moe.pack_weights(dB)
    torch.cuda.synchronize()
    log("gemm NONE largest experts: GPU")
    D = moe.grouped_gemm_alloc(dA, dB, dev(off), R, moe.MOE_EPI_NONE)
    torch.cuda.synchronize()
    sample = np.array(sorted({e * rows + d for e in range(E) for d in (0, rows - 1)}), np.int32)
    got = host_bits(D)[sample]
    del dA, dB, D
    torch.cuda.empty_cache()
    log(f"gemm NONE largest experts: oracle rows {sample.tolist()}")
    ref = oracle.grouped_gemm(A, Bq, Bsf, gB, off, rows=sample)
    check_bf16(got, ref, f"gemm NONE largest experts E={E} N={N} K={K} {'packed' if packed else 'row-major'}")


def test_gemm_dense_small_full():
    """One group (a plain dense GEMM): every output element against the oracle."""
    A, Bs, off, A_rows, R = _gemm_case([512], 1024, 512, False, seed=11)
    _run_gemm_none(A, Bs, off, A_rows, R, "dense 512x512x1024", packed=True)


@pytest.mark.timeout(600)
def test_gemm_dense_full_size_sampled():
    """The dense 8192^3 case in the benchmark's launch configuration, on sampled rows."""
    G = synth.GEMM_DENSE
    log("dense 8192^3: quantising operands (oracle)")
    A = oracle.quantize_bf16(synth.gemm_a_bf16(G))
    B = oracle.quantize(synth.gemm_b(G, 0))
    Bq, Bsf, gB = stack([B])
    off = np.array([0, G.M], np.int32)
    dA = moe.NVFP4Tensor(dev(A.q), dev(A.sf), dev(np.array([A.g], np.float32)))
    D = moe.grouped_gemm_alloc(dA, _weights(Bq, Bsf, gB, True), dev(off), G.M, moe.MOE_EPI_NONE)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(5).choice(G.M, 48, replace=False)).astype(np.int32)
    log("dense 8192^3: oracle on sampled rows")
    ref = oracle.grouped_gemm(A, Bq, Bsf, gB, off, rows=rows)
    check_bf16(host_bits(D)[rows], ref, "dense 8192^3 sampled rows")


def _pack_reference(q: np.ndarray, sf: np.ndarray) -> np.ndarray:
    """The packed layout written out from its definition in the header (byte moves only)."""
    rows, half_k = q.shape
    K = 2 * half_k
    steps = K // 256
    out = np.empty(rows * K * 9 // 16, np.uint8)
    for T in range(rows // 16):
        for s in range(steps):
            blk = out[(T * steps + s) * 2304:(T * steps + s + 1) * 2304]
            for l in range(64):
                r, g = l & 15, l >> 4
                for qq in range(2):
                    blk[qq * 1024 + l * 16: qq * 1024 + l * 16 + 16] = q[16 * T + r, s * 128 + 32 * g + 16 * qq:][:16]
                blk[2048 + l * 4: 2048 + l * 4 + 4] = sf[16 * T + r, s * 16 + 4 * g:][:4]
    return out


@pytest.mark.parametrize("rows,K", [(16, 256), (32, 256), (96, 768), (64, 1024)])
def test_pack_weights_bit_exact(rows, K):
    rng = np.random.default_rng(rows + K)
    q = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    sf = rng.integers(0, 127, (rows, K // 16), dtype=np.uint8)
    packed = torch.empty(rows * K * 9 // 16, dtype=torch.uint8, device="cuda")
    moe.moe_pack_weights_nvfp4(dev(q), dev(sf), packed)
    torch.cuda.synchronize()
    assert np.array_equal(packed.cpu().numpy(), _pack_reference(q, sf))


# ---------------------------------------------------------------------------------------
# grouped GEMM, SwiGLU epilogue, and the requantisation that consumes it

def _run_gemm_swiglu(A, Bs, off, A_rows, R, label, rows=None, packed=False):
    label = f"{label} {'packed' if packed else 'row-major'}"
    log(f"gemm SWIGLU {label}: E={len(Bs)} R={R}")
    Bq, Bsf, gB = stack(Bs)
    dA = moe.NVFP4Tensor(dev(A.q), dev(A.sf), dev(np.array([A.g], np.float32)))
    dB = _weights(Bq, Bsf, gB, packed)
    act, amax = moe.grouped_gemm_alloc(dA, dB, dev(off), R, moe.MOE_EPI_SWIGLU,
                                       A_rows=dev(A_rows) if A_rows is not None else None)
    torch.cuda.synchronize()
    got_all = host_bits(act)
    # partial maxima: their maximum is max |act| (a property of the kernel's own output)
    assert amax.max().item() == np.abs(bf16_values(got_all)).max(initial=0.0)
    rows = np.arange(R, dtype=np.int32) if rows is None else rows
    y1 = oracle.grouped_gemm(A, Bq, Bsf, gB, off, A_rows=A_rows, rows=rows)
    ref, bound = swiglu_ref_and_bound(y1, np_bf16_round)
    got = bf16_values(got_all[rows])
    diff = np.abs(got - ref)
    print(f"  act: max diff {diff.max():.3e}, max bound-ratio {(diff / bound).max():.3f}, "
          f"exact {(got_all[rows] == oracle.swiglu(y1)).mean():.5f}", flush=True)
    assert (diff <= bound).all()
    check_bf16(got_all[rows], ref, f"gemm SWIGLU {label} (bf16 output bar)")


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("sizes,K,I", [([8, 6, 9, 9], 256, 256), ([0, 17, 33, 64, 65, 1], 512, 384),
                                       ([40] * 256 + [3, 0, 64], 256, 512),
                                       ([0, 130, 255, 97], 768, 256),    # several chunks, odd K steps
                                       ([20, 32], 2048, 256),            # K split 8 ways
                                       ([33] * 14, 2048, 1024),          # K split 8 ways, items looped
                                       ([20, 32], 6144, 256),            # K split 8 ways, 7 and 5 half steps
                                       # 256 experts x 2 n tiles, 0-65 rows each: the 64-row kernel
                                       ([int(v) for v in np.random.default_rng(5).integers(0, 66, 256)], 512, 256),
                                       # 131 experts at K 1024: in-kernel lookup, last lane part-filled
                                       ([int(v) for v in np.random.default_rng(6).integers(0, 60, 131)], 1024, 768),
                                       # 8-wave kernel, one K step
                                       ([100, 150, 200, 3], 256, 256)])
def test_gemm_swiglu_shapes(sizes, K, I, packed):
    A, Bs, off, A_rows, R = _gemm_case(sizes, K, 2 * I, True, seed=7 + K + I)
    _run_gemm_swiglu(A, Bs, off, A_rows, R, f"sizes={sizes}", packed=packed)


@pytest.mark.parametrize("sizes,K,I,g_div", [([8, 6, 9, 9], 256, 256, 1.0), ([0, 17, 33, 64, 65, 1], 512, 384, 4.0),
                                             ([8, 6, 9, 9], 256, 256, np.inf),           # g2 = 0: s g2 = 0
                                             ([40] * 256 + [3, 0, 64], 256, 512, 1.0),   # LDS kernel
                                             ([20, 32], 2048, 256, 1.0),                 # K split 8 ways
                                             ([33] * 14, 2048, 1024, 1.0),               # K split, items looped
                                             ([0, 130, 255, 97], 768, 256, 2.0),         # 8-wave kernel
                                             # 256 experts x 2 n tiles, 0-65 rows: 64-row kernel
                                             ([int(v) for v in np.random.default_rng(5).integers(0, 66, 256)],
                                              512, 256, 1.0)])
def test_gemm_swiglu_nvfp4_fused(sizes, K, I, g_div):
    """SwiGLU + NVFP4 epilogue with a static global scale g2: codes and scales equal the
    oracle's static-scale quantisation of the GPU's own SwiGLU output byte for byte (same
    decision in the same precision); against the oracle's own FP64 pipeline only elements
    whose bf16 act differs by an ulp may change code.  g_div > 1 makes g2 small enough
    that some blocks saturate; g_div = inf gives g2 = 0, where every non-zero block saturates
    its scale, every non-zero element its code, and zero elements stay zero."""
    A, Bs, off, A_rows, R = _gemm_case(sizes, K, 2 * I, True, seed=17 + K + I)
    Bq, Bsf, gB = stack(Bs)
    dA = moe.NVFP4Tensor(dev(A.q), dev(A.sf), dev(np.array([A.g], np.float32)))
    dB = _weights(Bq, Bsf, gB, True)
    act, _ = moe.grouped_gemm_alloc(dA, dB, dev(off), R, moe.MOE_EPI_SWIGLU, A_rows=dev(A_rows))
    act_bits = host_bits(act)
    g2 = np.float32(max(np.abs(bf16_values(act_bits)).max(initial=0.0), 1e-30) / 2688.0 / g_div)
    log(f"gemm SWIGLU_NVFP4 sizes={sizes} K={K} I={I} g2={g2:.4g}")
    fused = moe.grouped_gemm_alloc(dA, dB, dev(off), R, moe.MOE_EPI_SWIGLU_NVFP4, A_rows=dev(A_rows),
                                   D_gs=dev(np.array([g2], np.float32)))
    torch.cuda.synchronize()
    ref = oracle.quantize_bf16(act_bits, g=float(g2))
    assert np.array_equal(fused.q.cpu().numpy(), ref.q)
    assert np.array_equal(fused.sf.cpu().numpy(), ref.sf)
    # the oracle's own pipeline: FP64 GEMM, SwiGLU, then the same static quantisation; every
    # 16-element block whose act values agree with it must agree bit for bit (a block holding a
    # one-ulp act difference may round differently)
    y1 = oracle.grouped_gemm(A, Bq, Bsf, gB, off, A_rows=A_rows)
    act64 = oracle.swiglu(y1)
    ref64 = oracle.quantize_bf16(act64, g=float(g2))
    same_blk = (act_bits == act64).reshape(R, I // 16, 16).all(axis=2)
    fq, fsf = fused.q.cpu().numpy().reshape(R, I // 16, 8), fused.sf.cpu().numpy()
    assert np.array_equal(fq[same_blk], ref64.q.reshape(R, I // 16, 8)[same_blk])
    assert np.array_equal(fsf[same_blk], ref64.sf[same_blk])
    print(f"  blocks compared with the FP64 pipeline: {same_blk.mean():.5f}", flush=True)
    assert same_blk.mean() > 0.9


def test_requantize_bit_exact_from_partials():
    rng = np.random.default_rng(9)
    act = synth.bf16_bits((rng.standard_normal((8192, 2048)) * 2).astype(np.float32))
    x = synth.bf16_to_f32(act)
    parts = np.zeros(4096, np.float32)
    parts[rng.integers(0, 4096, 50)] = np.abs(x).max() * rng.uniform(0, 1, 50).astype(np.float32)
    parts[1234] = np.abs(x).max()
    _check_quant(x, bf16=True, partials=parts)


# ---------------------------------------------------------------------------------------
# FINALIZE

@pytest.mark.parametrize("T,E,k,H", [(16, 4, 2, 256), (1024, 256, 8, 6144), (5, 3, 3, 8), (64, 32, 1, 512),
                                     (37, 64, 32, 264),    # k = 32, the largest the call takes
                                     (3, 32, 32, 8),       # k = E = 32, one 8-column chunk
                                     (9, 16, 4, 2056)])    # 257 column chunks: a second, ragged round of threads
def test_finalize(T, E, k, H):
    log(f"finalize T={T} k={k} H={H}")
    rng = np.random.default_rng(T + H)
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    off, rs, tsr = oracle.permute(ids, E)
    w32 = w.astype(np.float32)
    Y = synth.bf16_bits((rng.standard_normal((T * k, H)) * 3).astype(np.float32))
    ref64, _ = oracle.finalize(bf16_values(Y), w32.astype(np.float64), tsr)
    out = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    moe.moe_finalize(dev_bf16(Y), dev(w32), dev(tsr), out)
    torch.cuda.synchronize()
    got = host_bits(out)
    check_bf16(got, ref64, f"finalize T={T} k={k} H={H}")
    assert (got == np_bf16_round(ref64)).mean() > 0.99


def test_finalize_no_tokens():
    """T = 0: nothing to combine; the call succeeds and launches nothing (empty tensors)."""
    Y = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    w = torch.empty(0, 2, dtype=torch.float32, device="cuda")
    tsr = torch.empty(0, dtype=torch.int32, device="cuda")
    out = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    moe.moe_finalize(Y, w, tsr, out)
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


# ---------------------------------------------------------------------------------------
# the whole layer, end to end

def _layer_gpu(L, logits, x_bits, d1, d2):
    plan = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, d1, d2)
    out = plan.forward(dev(logits), dev_bf16(x_bits))
    torch.cuda.synchronize()
    return plan, host_bits(out)


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
def test_layer_tiny_end_to_end(packed):
    L = synth.TINY
    logits, x = synth.router_logits(L), synth.layer_activations(L)
    W1 = [oracle.quantize(synth.layer_w1(L, e)) for e in range(L.E)]
    W2 = [oracle.quantize(synth.layer_w2(L, e)) for e in range(L.E)]
    r = oracle.moe_layer(logits, x, W1, W2, L.k)
    q1, q2 = stack(W1), stack(W2)
    d1 = _weights(*q1, packed)
    d2 = _weights(*q2, packed)
    plan, got = _layer_gpu(L, logits, x, d1, d2)
    assert np.array_equal(plan.off.cpu().numpy(), r.offsets)
    assert np.array_equal(plan.xq.q.cpu().numpy(), r.xq.q)
    check_bf16(got, r.out64, "layer tiny")


# 131 experts (not a multiple of four) with K = 1024 in both GEMMs: every GEMM of the layer
# looks its work items up in the kernel with the lookup's last lane part-filled
LAYER_E131 = synth.Layer("layer_t512_e131_k8_h1024_i1024", T=512, E=131, k=8, H=1024, I=1024)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("L", [synth.LAYER_DECODE, synth.LAYER_SKEWED, synth.LAYER_EP8, synth.LAYER_TP8, LAYER_E131],
                         ids=lambda L: L.name)
def test_layer_full_size_end_to_end(L):
    W1, W2, d1, d2 = layer_weights(L)
    logits, x = synth.router_logits(L), synth.layer_activations(L)
    log(f"layer {L.name}: GPU forward")
    plan, got = _layer_gpu(L, logits, x, d1, d2)
    log(f"layer {L.name}: oracle")
    r = oracle.moe_layer(logits, x, W1, W2, L.k)
    log(f"layer {L.name}: compare")
    sizes = np.diff(r.offsets)
    print(f"  rows per expert: min {sizes.min()} median {int(np.median(sizes))} max {sizes.max()} "
          f"empty {(sizes == 0).sum()}", flush=True)
    assert np.array_equal(plan.off.cpu().numpy(), r.offsets)
    assert np.array_equal(plan.row_src.cpu().numpy(), r.row_src)
    assert np.array_equal(plan.xq.q.cpu().numpy(), r.xq.q) and np.array_equal(plan.xq.sf.cpu().numpy(), r.xq.sf)
    check_bf16(got, r.out64, f"layer {L.name} out")


@pytest.mark.timeout(600)
def test_layer_decode_fused_static_scale_end_to_end():
    """The decode layer with the SwiGLU output requantised in the gate/up GEMM's epilogue under
    a static global scale (calibrated from the oracle's dynamic scale of the same act), against
    the oracle layer with that static scale."""
    L = synth.LAYER_DECODE
    W1, W2, d1, d2 = layer_weights(L)
    logits, x = synth.router_logits(L), synth.layer_activations(L)
    r_dyn = oracle.moe_layer(logits, x, W1, W2, L.k)
    g2 = float(r_dyn.actq.g)
    plan = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, d1, d2, static_g2=dev(np.array([g2], np.float32)))
    got = host_bits(plan.forward(dev(logits), dev_bf16(x)))
    torch.cuda.synchronize()
    r = oracle.moe_layer(logits, x, W1, W2, L.k, act_g=g2)
    check_bf16(got, r.out64, "layer decode, fused static-scale requantisation")


@pytest.mark.timeout(900)
def test_layer_prefill_end_to_end():
    """Prefill layer (16384 tokens, ~512 rows per expert) in the benchmark's launch
    configuration, against the oracle's own pipeline:
      * routing, permutation, offsets and the token quantisation (codes, scales, g bits)
        bit-exact;
      * the oracle's gate/up GEMM over all 131,072 rows (in whole-expert chunks), its SwiGLU
        output against the GPU's act element by element within the derived one-ulp bound;
      * the dynamic requantisation scale g2 bit-exact, and the requantised codes and scales
        bit-exact in every 16-element block whose act values agree (a block with a one-ulp
        act difference may round differently);
      * the down GEMM and FINALIZE on 128 sampled tokens, all k rows each: the layer's bf16
        output and those rows of the Y workspace under the bf16 bar."""
    L = synth.LAYER_PREFILL
    W1, W2, d1, d2 = layer_weights(L)
    logits, x = synth.router_logits(L), synth.layer_activations(L)
    ids_o, w_o = oracle.route(logits, L.k)
    off_o, rs_o, tsr_o = oracle.permute(ids_o, L.E)
    xq_o = oracle.quantize_bf16(x)
    log("prefill: GPU forward")
    plan, got_out = _layer_gpu(L, logits, x, d1, d2)
    assert np.array_equal(plan.ids.cpu().numpy(), ids_o)
    assert np.array_equal(plan.off.cpu().numpy(), off_o)
    assert np.array_equal(plan.row_src.cpu().numpy(), rs_o)
    assert np.array_equal(plan.tsr.cpu().numpy(), tsr_o)
    assert np.array_equal(plan.xq.q.cpu().numpy(), xq_o.q)
    assert np.array_equal(plan.xq.sf.cpu().numpy(), xq_o.sf)
    assert plan.xq.gs.cpu().numpy().view(np.uint32)[0] == np.float32(xq_o.g).view(np.uint32)
    act_gpu = host_bits(plan.act)
    actq_gpu = (plan.actq.q.cpu().numpy(), plan.actq.sf.cpu().numpy(), plan.actq.gs.cpu().numpy())

    # the oracle's gate/up GEMM and SwiGLU over every row, whole experts at a time
    B1 = stack(W1)
    act_o = np.empty((L.R, L.I), np.uint16)
    worst = 0.0
    t0 = time.time()
    for e0 in range(0, L.E, 16):
        lo, hi = int(off_o[e0]), int(off_o[min(e0 + 16, L.E)])
        rows = np.arange(lo, hi, dtype=np.int32)
        y1 = oracle.grouped_gemm(xq_o, *B1, off_o, A_rows=rs_o, rows=rows)
        act_o[lo:hi] = oracle.swiglu(y1)
        ref, bound = swiglu_ref_and_bound(y1, np_bf16_round)
        diff = np.abs(bf16_values(act_gpu[lo:hi]) - ref)
        worst = max(worst, float((diff / bound).max(initial=0.0)))
        assert (diff <= bound).all(), (e0, worst)
        log(f"prefill: oracle gate/up + SwiGLU experts {e0}..{min(e0 + 16, L.E) - 1} "
            f"({time.time() - t0:.0f} s, worst act bound ratio {worst:.3f})")
    same_act = act_gpu == act_o
    print(f"  act bf16 identical in {same_act.mean():.6f} of the elements", flush=True)
    actq_o = oracle.quantize_bf16(act_o)
    assert actq_gpu[2].view(np.uint32)[0] == np.float32(actq_o.g).view(np.uint32), (actq_gpu[2], actq_o.g)
    same_blk = same_act.reshape(L.R, L.I // 16, 16).all(axis=2)
    codes_gpu = actq_gpu[0].reshape(L.R, L.I // 16, 8)
    codes_o = actq_o.q.reshape(L.R, L.I // 16, 8)
    assert np.array_equal(actq_gpu[1][same_blk], actq_o.sf[same_blk])
    assert np.array_equal(codes_gpu[same_blk], codes_o[same_blk])
    print(f"  requantised blocks compared bit for bit: {same_blk.mean():.6f}; blocks differing "
          f"{(~(codes_gpu == codes_o).all(axis=2) | (actq_gpu[1] != actq_o.sf)).mean():.2e}", flush=True)

    # down GEMM and FINALIZE for sampled tokens, all k rows of each
    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(L.T, 128, replace=False))
    rows = tsr_o.reshape(L.T, L.k)[toks].reshape(-1).astype(np.int32)
    log("prefill: oracle down GEMM on the sampled tokens' rows")
    y2 = oracle.grouped_gemm(actq_o, *stack(W2), off_o, rows=rows)
    check_bf16(host_bits(plan.Y)[rows], y2, "prefill down GEMM, sampled tokens' rows")
    out64, _ = oracle.finalize(y2, w_o[toks], np.arange(len(rows), dtype=np.int32))
    check_bf16(got_out[toks], out64, "prefill layer output, sampled tokens")


# ---------------------------------------------------------------------------------------
# determinism: identical bytes on a repeated run (no float atomics anywhere)

def test_layer_deterministic():
    L = synth.Layer("mid_t256_e32_k4_h512_i256", T=256, E=32, k=4, H=512, I=256)
    rng = np.random.default_rng(2)
    W1 = [oracle.quantize((rng.standard_normal((2 * L.I, L.H)) * 0.02).astype(np.float32)) for _ in range(L.E)]
    W2 = [oracle.quantize((rng.standard_normal((L.H, L.I)) * 0.02).astype(np.float32)) for _ in range(L.E)]
    d1 = _weights(*stack(W1), packed=True)
    d2 = _weights(*stack(W2), packed=True)
    logits = rng.standard_normal((L.T, L.E)).astype(np.float32)
    x = synth.bf16_bits(rng.standard_normal((L.T, L.H)).astype(np.float32))
    plan = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, d1, d2)
    outs = []
    for _ in range(3):
        o = plan.forward(dev(logits), dev_bf16(x))
        torch.cuda.synchronize()
        outs.append((host_bits(o).copy(), host_bits(plan.act).copy(), plan.actq.q.cpu().numpy().copy()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    r = oracle.moe_layer(logits, x, W1, W2, L.k)
    check_bf16(outs[0][0], r.out64, "layer mid (E=32)")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("L", [synth.LAYER_DECODE, synth.LAYER_TP8, synth.LAYER_PREFILL], ids=lambda L: L.name)
def test_layer_deterministic_full_size(L):
    """The benchmark's kernel paths at full size, run three times on the same inputs with the
    outputs overwritten in between: every intermediate is identical byte for byte.  Decode:
    the four-wave LDS kernels with their items looked up in the kernel (256 experts, four per
    lane); TP8 share: the schedule kernel and items of several n tiles (K = 256); prefill:
    the eight-wave kernel over ~512 rows per expert."""
    _, _, d1, d2 = layer_weights(L)
    plan = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, d1, d2)
    logits, x = dev(synth.router_logits(L)), dev_bf16(synth.layer_activations(L))
    outs = [plan.out, plan.act, plan.Y, plan.actq.q, plan.actq.sf, plan.actq.gs, plan.xq.q, plan.xq.sf, plan.off,
            plan.row_src, plan.tsr, plan.ids, plan.w]
    snaps = []
    for run in range(3):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5 + run)
        plan.forward(logits, x)
        torch.cuda.synchronize()
        snaps.append([t.clone() for t in outs])
        log(f"{L.name}: run {run} done")
    for s in snaps[1:]:
        for a, b in zip(snaps[0], s):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
