"""Pins of the oracle's grouped NVFP4 GEMM.  CPU only.

(1) Against numpy's FP64 matmul of operands dequantised independently of the oracle (golden
E2M1 table, torch's float8_e4m3fn cast), over the grouped shapes with empty, single-row and
ragged groups.  (2) Closed forms: all-ones operands give y = K; a single 16-block by hand.
(3) The gather map equals an explicit gather.  A transposed operand, a wrong group offset,
a dropped block scale or a sign slip all fail (1).
"""
import numpy as np
import pytest
import torch

import oracle

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dq(q, sf, g):
    lo, hi = q & 15, q >> 4
    c = np.stack([lo, hi], axis=-1).reshape(*q.shape[:-1], -1)
    return E2M1[c] * np.repeat(e4m3(sf), 16, axis=-1) * np.float64(g)


def make_case(rng, sizes, K, N, gather):
    E = len(sizes)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    R = int(offsets[-1])
    T = max(R, 1) + 3
    A = oracle.quantize((rng.standard_normal((T, K)) * 1.7).astype(np.float32))
    Bq, Bs, gB = [], [], []
    for e in range(E):
        t = oracle.quantize((rng.standard_normal((N, K)) * 0.02 * (e + 1)).astype(np.float32))
        Bq.append(t.q); Bs.append(t.sf); gB.append(t.g)
    A_rows = rng.integers(0, T, R).astype(np.int32) if gather else None
    return A, np.stack(Bq), np.stack(Bs), np.array(gB, np.float32), offsets, A_rows


def reference(A, Bq, Bs, gB, offsets, A_rows):
    a = dq(A.q, A.sf, A.g)
    R = int(offsets[-1])
    rows = A_rows if A_rows is not None else np.arange(R)
    y = np.zeros((R, Bq.shape[1]))
    for e in range(len(gB)):
        lo, hi = offsets[e], offsets[e + 1]
        if hi > lo:
            y[lo:hi] = a[rows[lo:hi]] @ dq(Bq[e], Bs[e], gB[e]).T
    return y


@pytest.mark.parametrize("sizes", [[5], [0, 3], [1, 0, 15, 16], [17, 33, 0, 1]])
@pytest.mark.parametrize("K", [16, 32, 256])
@pytest.mark.parametrize("N", [16, 64])
@pytest.mark.parametrize("gather", [False, True])
def test_matches_dequantised_matmul(sizes, K, N, gather):
    rng = np.random.default_rng(hash((tuple(sizes), K, N, gather)) % 2**32)
    A, Bq, Bs, gB, off, A_rows = make_case(rng, sizes, K, N, gather)
    y = oracle.grouped_gemm(A, Bq, Bs, gB, off, A_rows=A_rows)
    ref = reference(A, Bq, Bs, gB, off, A_rows)
    assert y.shape == ref.shape
    if ref.size:
        err = np.abs(y - ref).max() / max(np.abs(ref).max(), 1e-300)
        assert err <= 1e-12, err


def test_row_subset_matches_full():
    rng = np.random.default_rng(11)
    A, Bq, Bs, gB, off, A_rows = make_case(rng, [4, 9, 0, 6], 64, 32, True)
    full = oracle.grouped_gemm(A, Bq, Bs, gB, off, A_rows=A_rows)
    pick = np.array([18, 0, 5, 12, 3], np.int32)
    sub = oracle.grouped_gemm(A, Bq, Bs, gB, off, A_rows=A_rows, rows=pick)
    assert np.array_equal(sub, full[pick])


def test_all_ones_gives_K():
    K, N, M = 256, 16, 8
    q = np.full((M, K // 2), 0x22, np.uint8)          # every code 2 (= 1.0)
    s = np.full((M, K // 16), 0x38, np.uint8)         # every scale 0x38 (= 1.0)
    A = oracle.NVFP4(q, s, 1.0)
    Bq = np.full((1, N, K // 2), 0x22, np.uint8)
    Bs = np.full((1, N, K // 16), 0x38, np.uint8)
    y = oracle.grouped_gemm(A, Bq, Bs, np.ones(1, np.float32), np.array([0, M], np.int32))
    assert np.all(y == K)


def test_single_block_by_hand():
    # a = [6, -1.5, 0.5, 0 ...], b = [2, 4, -3, 1 ...] with scales 2 and 0.5, g = 0.25 and 4:
    # y = 0.25 * 4 * 2 * 0.5 * (12 - 6 - 1.5 + 0) = 4.5
    # A byte 0: low nibble 7 (6.0), high nibble 0xB (-1.5); byte 1: low 1 (0.5), high 0
    A = oracle.NVFP4(np.array([[0x07 | (0xB << 4), 0x01, 0, 0, 0, 0, 0, 0]], np.uint8),
                     np.array([[0x40]], np.uint8), 0.25)   # scale 0x40 = 2.0
    Bq = np.zeros((1, 1, 8), np.uint8)
    Bq[0, 0, 0] = 0x04 | (0x6 << 4)                   # 2.0, 4.0
    Bq[0, 0, 1] = 0x0D | (0x2 << 4)                   # -3.0, 1.0
    Bs = np.array([[[0x30]]], np.uint8)               # 0.5
    y = oracle.grouped_gemm(A, Bq, Bs, np.array([4.0], np.float32), np.array([0, 1], np.int32))
    assert y[0, 0] == 0.25 * 4 * 2 * 0.5 * (6 * 2 - 1.5 * 4 + 0.5 * -3 + 0 * 1)


def test_empty_groups_and_no_rows():
    rng = np.random.default_rng(12)
    A, Bq, Bs, gB, off, A_rows = make_case(rng, [0, 0, 0], 32, 16, False)
    y = oracle.grouped_gemm(A, Bq, Bs, gB, off)
    assert y.shape == (0, 16)
