"""Pins of the oracle's NVFP4 quantiser: exact round trips, the normal-scale block maximum,
sign, monotonicity, the rounding-error bound and the degenerate tensors.  CPU only.

The quantiser reading (decode-direction global scale g = amax / (6 * 448); block scale
e4m3(amax_b / (6 g)); element e2m1(|x| / (s g)), both round-to-nearest-even and saturating)
is fixed in the design notes.  Values are decoded here with the golden E2M1 table and torch's
float8_e4m3fn cast, not with the oracle's own decode.
"""
import numpy as np
import pytest
import torch

import oracle

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6], np.float64)


def e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def codes_of(q):
    lo = q & 15
    hi = q >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.shape[0], -1)


def dequant(t: oracle.NVFP4):
    c = codes_of(t.q)
    s = np.repeat(e4m3(t.sf), 16, axis=1)
    return E2M1[c] * s * np.float64(t.g)


def test_exact_inputs_round_trip():
    rng = np.random.default_rng(0)
    rows, C = 24, 256
    g = np.float32(2.0 ** -7)
    codes = rng.integers(0, 16, (rows, C))
    scales = rng.integers(1, 0x7F, (rows, C // 16))      # every finite positive e4m3
    codes[:, ::16] = 7                                   # each block holds a 6.0 ...
    scales[0, 0] = 0x7E                                  # ... and one block the largest scale 448
    x = E2M1[codes] * np.repeat(e4m3(scales), 16, axis=1) * float(g)
    assert np.all(x.astype(np.float32) == x)             # exactly representable in binary32
    t = oracle.quantize(x.astype(np.float32))
    assert t.g == g                                      # amax = 6 * 448 * g exactly
    assert np.array_equal(t.sf, scales.astype(np.uint8))
    got = codes_of(t.q)
    # equal values may differ only in the sign of zero
    assert np.array_equal(E2M1[got], E2M1[codes])
    assert np.array_equal(dequant(t), x)


def test_normal_scale_blocks_reach_six_and_signs_kept():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 512)) * np.exp(rng.uniform(-6, 6, (64, 1)))).astype(np.float32)
    x[3, 17] = -0.0
    t = oracle.quantize(x)
    c = codes_of(t.q)
    mag = c & 7
    blk_max = mag.reshape(64, -1, 16).max(axis=2)
    normal = t.sf >= 0x08
    assert normal.sum() > 0.5 * normal.size
    assert np.all(blk_max[normal] == 7)
    assert np.array_equal((c >> 3).astype(bool), np.signbit(x))


def test_monotone_within_blocks_and_error_bound():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((32, 1024)).astype(np.float32)
    t = oracle.quantize(x)
    c = codes_of(t.q)
    dq = dequant(t)
    s = np.repeat(e4m3(t.sf), 16, axis=1) * np.float64(t.g)
    u = np.abs(x.astype(np.float64)) / s
    mags = np.abs(E2M1[c])
    # half the E2M1 spacing around u, plus the clip at 6
    half_step = np.where(u <= 2, 0.25, np.where(u <= 4, 0.5, 1.0)) + np.maximum(u - 6, 0) + 1e-6
    assert np.all(np.abs(u - mags) <= half_step)
    xb, mb = np.abs(x).reshape(32, -1, 16), mags.reshape(32, -1, 16)
    order = np.argsort(xb, axis=2, kind="stable")
    assert np.all(np.diff(np.take_along_axis(mb, order, axis=2), axis=2) >= 0)
    rel = np.linalg.norm(dq - x) / np.linalg.norm(x)
    assert rel < 0.12


def test_zero_and_tiny_blocks():
    x = np.zeros((2, 32), np.float32)
    x[1, 16:] = -0.0
    t = oracle.quantize(x)
    assert t.g == 1.0
    assert np.all(t.sf == 0)
    assert np.all(codes_of(t.q)[0] == 0) and np.all(codes_of(t.q)[1, 16:] == 8)
    # a block far below the tensor's amax gets scale 0 and signed-zero codes
    y = np.zeros((1, 32), np.float32)
    y[0, 0] = 1000.0
    y[0, 16] = -1e-6
    t = oracle.quantize(y)
    assert t.sf[0, 1] == 0 and codes_of(t.q)[0, 16] == 8


def test_static_global_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    t = oracle.quantize(x, g=0.25)
    assert t.g == np.float32(0.25)
    # block scale decision: t_b = amax_b / 1.5 rounded to e4m3
    amax_b = np.abs(x).reshape(4, -1, 16).max(axis=2)
    want = torch.from_numpy((amax_b / np.float32(1.5)).astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(t.sf, want)


def test_saturation_at_448():
    x = np.zeros((1, 32), np.float32)
    x[0, :16] = 1.0
    x[0, 16] = 1e6
    t = oracle.quantize(x, g=1e-3)
    assert t.sf[0, 1] == 0x7E           # amax_b / (6 g) far above 448 -> 448
    assert codes_of(t.q)[0, 16] == 7    # |x| / (448 g) far above 6 -> 6


def test_underflowed_global_scale_keeps_zeros():
    """An all-subnormal tensor whose global scale amax / 2688 underflows to 0 in binary32
    (numpy's own float32 division says so): 6 g = 0, so a block with a non-zero maximum gets
    t = +inf -> scale 448 (0x7E) and its non-zero elements saturate at 6 (code 7 with their
    sign), while zero stays zero -- a zero block keeps scale 0 and a zero element code 0
    (0 / 0 counts as 0 in the reading)."""
    tiny = np.float32(2.0 ** -149)
    x = np.zeros((2, 48), np.float32)
    x[0, :16] = tiny * np.arange(-8, 8, dtype=np.float32)     # zeros among small values
    x[1, 32:48] = -tiny * 40
    x[1, 33] = -0.0
    amax = np.abs(x).max()
    assert np.float32(amax) / np.float32(2688.0) == 0.0
    t = oracle.quantize(x)
    assert t.g == 0.0
    c = codes_of(t.q)
    assert t.sf[0, 0] == 0x7E and t.sf[1, 2] == 0x7E
    assert np.all(t.sf[0, 1:] == 0) and np.all(t.sf[1, :2] == 0)
    row0 = x[0, :16]
    want = np.where(row0 == 0, 0, 7) | np.where(np.signbit(row0), 8, 0)
    assert np.array_equal(c[0, :16], want)
    assert np.all(c[0, 16:] == 0) and np.all(c[1, :32] == 0)
    assert c[1, 33] == 8 and np.all(np.delete(c[1, 32:48], 1) == 15)


def test_underflowed_block_divisor_keeps_zeros():
    """Static g = 2^-149: a block with maximum 3 * 2^-149 gets t = 0.5 exactly, scale 0.5
    (0x30), and s g = 2^-150 rounds to 0 in binary32 (numpy).  Its zero elements keep code 0
    (0 / 0 counts as 0), its non-zero ones saturate at 6; a block of ordinary values under the
    same g saturates its scale at 448 and is quantised normally."""
    g = np.float32(2.0 ** -149)
    assert np.float32(0.5) * g == 0.0
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = np.array([3, 0, -1, -0.0], np.float32) * g
    x[0, 16:32] = np.float32(1.0)
    t = oracle.quantize(x, g=float(g))
    c = codes_of(t.q)
    assert t.sf[0, 0] == 0x30 and t.sf[0, 1] == 0x7E
    assert list(c[0, :4]) == [7, 0, 15, 8] and np.all(c[0, 4:16] == 0)
    assert np.all(c[0, 16:32] == 7)   # 1 / (448 g) is far above 6
