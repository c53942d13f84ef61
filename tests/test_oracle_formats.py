"""Pins of the oracle's element formats against the published encodings and library casts.

CPU only.  Each check is independent of the oracle's own code: values come from the
golden tables (OCP MX v1.0 / IEEE 754 round-to-nearest-even) or from torch's float8 and
bfloat16 casts.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_e2m1_value_table():
    for code, val in _table("e2m1_values.txt"):
        got = oracle.e2m1_value(int(code))
        want = float(val)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)


def test_e4m3_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = oracle.e4m3_value(c)
        if np.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == float(ref[c]) and math.copysign(1, got) == math.copysign(1, float(ref[c])), c
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert math.isnan(oracle.e4m3_value(0x7F)) and math.isnan(oracle.e4m3_value(0xFF))


def _torch_e4m3_code(t):
    return int(torch.tensor([t], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def test_e4m3_round_matches_torch_cast():
    vals = [oracle.e4m3_value(c) for c in range(127)]
    pts = set(vals)
    for a, b in zip(vals[:-1], vals[1:]):
        mid = np.float32((a + b) / 2)  # exact: neighbours differ by one binary32-representable step
        pts.update([float(mid), float(np.nextafter(mid, np.float32(0))), float(np.nextafter(mid, np.float32(1e9)))])
    rng = np.random.default_rng(5)
    pts.update(rng.uniform(0, 448, 20000).astype(np.float32).tolist())
    pts.update((2.0 ** rng.uniform(-14, 8.8, 20000)).astype(np.float32).tolist())
    pts = [p for p in pts if 0 <= p <= 448]
    t = torch.tensor(pts, dtype=torch.float32)
    ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for p, r in zip(pts, ref):
        assert oracle.e4m3_round(p) == int(r), (p, oracle.e4m3_round(p), int(r))


def test_e4m3_round_ties_go_to_even_code():
    # 2^-10 lies halfway between 0 (code 0) and 2^-9 (code 1): even code 0.
    assert oracle.e4m3_round(2.0 ** -10) == 0
    # 1.5 * 2^-9 lies halfway between codes 1 and 2: code 2.
    assert oracle.e4m3_round(1.5 * 2.0 ** -9) == 2
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even code 0x38.
    assert oracle.e4m3_round(1.0625) == 0x38
    # 432 lies halfway between 416 (0x7D) and 448 (0x7E): even code 0x7E.
    assert oracle.e4m3_round(432.0) == 0x7E


def test_e2m1_rounding_table():
    for u, code in _table("e2m1_rounding.txt"):
        assert oracle.e2m1_round(float(u)) == int(code), (u, oracle.e2m1_round(float(u)), code)


def test_bf16_round_matches_torch_on_binary32_inputs():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-30,
                        rng.standard_normal(2000) * 1e30]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for xi, r in zip(x.tolist(), ref.tolist()):
        assert oracle.bf16_round(xi) == r, (xi, oracle.bf16_round(xi), r)


def test_bf16_round_is_direct_not_double_rounded():
    # 1 + 2^-8 is the midpoint of bf16 neighbours 1 and 1 + 2^-7; a value just above it must
    # round up, although going through binary32 first would land on the tie and round down.
    assert oracle.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert oracle.bf16_round(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.bf16_round(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.bf16_round(-0.0) == 0x8000
    assert oracle.bf16_value(0x3F80) == 1.0
