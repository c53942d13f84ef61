"""Pins of the oracle's routing, permutation, SwiGLU, FINALIZE and layer wiring.  CPU only.

Routing against numpy's lexsort (descending logit, ascending id) and scipy's softmax;
permutation against numpy's stable argsort and bincount; SwiGLU against torch's silu with
special values; FINALIZE against its invariants (k = 1, constant expert outputs, expert
relabelling, linearity); the layer against a brute-force per-token loop.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth


@pytest.mark.parametrize("T,E,k", [(16, 4, 2), (64, 256, 8), (5, 8, 8), (33, 7, 1)])
def test_route_matches_lexsort_and_softmax(T, E, k):
    rng = np.random.default_rng(T * E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, ::3] = np.round(logits[:, ::3])          # plenty of ties
    ids, w = oracle.route(logits, k)
    for t in range(T):
        order = np.lexsort((np.arange(E), -logits[t].astype(np.float64)))
        assert np.array_equal(ids[t], order[:k])
        ref = scipy.special.softmax(logits[t, order[:k]].astype(np.float64))
        assert np.allclose(w[t], ref, rtol=1e-13, atol=0)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_route_all_equal_logits_and_full_sort():
    ids, w = oracle.route(np.zeros((3, 6), np.float32), 6)
    assert np.array_equal(ids, np.tile(np.arange(6), (3, 1)))
    assert np.allclose(w, 1 / 6, rtol=1e-15)


@pytest.mark.parametrize("T,E,k", [(16, 4, 2), (512, 256, 8), (7, 300, 3)])
def test_permute_matches_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    off, row_src, tsr = oracle.permute(ids, E)
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(row_src, order // k)
    inv = np.empty_like(order)
    inv[order] = np.arange(len(order))
    assert np.array_equal(tsr, inv)


def test_swiglu_special_values_and_torch_silu():
    I = 5
    y1 = np.zeros((3, 2 * I))
    y1[0, :I] = [0.0, 1.0, -1.0, 50.0, -50.0]
    y1[0, I:] = [3.0, 1.0, 1.0, 2.0, 7.0]
    act = oracle.swiglu(y1)
    v = [oracle.bf16_value(int(b)) for b in act[0]]
    assert v[0] == 0.0                      # silu(0) = 0
    assert v[3] == 100.0                    # silu(50) = 50 to bf16 precision
    assert abs(v[4]) < 1e-18                # silu(-50) ~ -1e-20
    assert np.all(act[1:] == 0)
    rng = np.random.default_rng(4)
    y1 = rng.standard_normal((64, 2 * 32)) * 3
    act = oracle.swiglu(y1)
    gate = torch.from_numpy(y1[:, :32].astype(np.float32)).to(torch.bfloat16).to(torch.float64)
    up = torch.from_numpy(y1[:, 32:].astype(np.float32)).to(torch.bfloat16).to(torch.float64)
    ref = (torch.nn.functional.silu(gate) * up).numpy()
    got = np.vectorize(oracle.bf16_value)(act)
    # bf16 rounding of the FP64 product: within half a bf16 ulp (2^-9 relative)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0 ** -8 + 1e-30)
    # y1 values already bf16 in this draw for the rounding of halves: exact match in >99%
    exact = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert (got == exact).mean() > 0.99


def _finalize_case(rng, T, E, k, H):
    ids, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    off, row_src, tsr = oracle.permute(ids, E)
    y2 = rng.standard_normal((T * k, H))
    return ids, w, off, row_src, tsr, y2


def test_finalize_invariants():
    rng = np.random.default_rng(9)
    T, E, k, H = 12, 6, 3, 40
    ids, w, off, row_src, tsr, y2 = _finalize_case(rng, T, E, k, H)
    o64, o16 = oracle.finalize(y2, w, tsr)
    # brute force: sum over slots of weight x the permuted row of that (token, slot)
    ref = np.zeros((T, H))
    for t in range(T):
        for j in range(k):
            ref[t] += w[t, j] * y2[tsr[t * k + j]]
    assert np.allclose(o64, ref, rtol=1e-14, atol=1e-15)
    # constant expert outputs c: out = c (weights sum to one)
    c = np.full_like(y2, 0.37)
    o64c, _ = oracle.finalize(c, w, tsr)
    assert np.allclose(o64c, 0.37, rtol=1e-14)
    # linearity
    y2b = rng.standard_normal(y2.shape)
    o_b, _ = oracle.finalize(y2b, w, tsr)
    o_ab, _ = oracle.finalize(y2 + y2b, w, tsr)
    assert np.allclose(o_ab, o64 + o_b, rtol=1e-12, atol=1e-14)
    # k = 1: out = bf16 of the routed row
    ids1, w1 = oracle.route(rng.standard_normal((T, E)).astype(np.float32), 1)
    _, _, tsr1 = oracle.permute(ids1, E)
    y21 = rng.standard_normal((T, H))
    o64_1, o16_1 = oracle.finalize(y21, w1, tsr1)
    assert np.all(w1 == 1.0)
    assert np.array_equal(o64_1, y21[tsr1])
    ref16 = torch.from_numpy(y21[tsr1].astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (o16_1 == ref16).mean() > 0.999


def test_finalize_relabelling_experts_leaves_output_unchanged():
    rng = np.random.default_rng(10)
    T, E, k, H = 20, 8, 2, 16
    logits = rng.standard_normal((T, E)).astype(np.float32)
    perm = rng.permutation(E)
    ids, w = oracle.route(logits, k)
    ids_p, w_p = oracle.route(logits[:, np.argsort(perm)], k)   # expert e renamed perm[e]
    assert np.array_equal(perm[ids], ids_p)
    # per-expert output function: row value depends only on (token, expert)
    f = rng.standard_normal((T, E, H))
    def outputs(ids_, naming):
        off, row_src, tsr = oracle.permute(ids_, E)
        y2 = np.zeros((T * k, H))
        for t in range(T):
            for j in range(k):
                y2[tsr[t * k + j]] = f[t, naming[ids_[t, j]]]
        return oracle.finalize(y2, w if naming is ident else w_p, tsr)[0]
    ident = np.arange(E)
    inv = np.argsort(perm)
    assert np.allclose(outputs(ids, ident), outputs(ids_p, inv), rtol=1e-15, atol=1e-15)


def test_layer_wiring_matches_per_token_loop():
    L = synth.TINY
    logits = synth.router_logits(L)
    x = synth.layer_activations(L)
    W1 = [oracle.quantize(synth.layer_w1(L, e)) for e in range(L.E)]
    W2 = [oracle.quantize(synth.layer_w2(L, e)) for e in range(L.E)]
    r = oracle.moe_layer(logits, x, W1, W2, L.k)
    E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])

    def dq(t):
        c = np.stack([t.q & 15, t.q >> 4], -1).reshape(t.q.shape[0], -1)
        s = torch.from_numpy(t.sf).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return E2M1[c] * np.repeat(s, 16, 1) * np.float64(t.g)

    xd = dq(r.xq)
    ad = dq(r.actq)
    for t in range(L.T):
        acc = np.zeros(L.H)
        order = np.lexsort((np.arange(L.E), -logits[t].astype(np.float64)))[:L.k]
        assert np.array_equal(order, r.ids[t])
        for j, e in enumerate(order):
            p = r.token_slot_row[t * L.k + j]
            assert r.row_src[p] == t and r.offsets[e] <= p < r.offsets[e + 1]
            y1 = xd[t] @ dq(W1[e]).T
            assert np.allclose(r.y1[p], y1, rtol=1e-12, atol=1e-12)
            acc += r.w[t, j] * (ad[p] @ dq(W2[e]).T)
        assert np.allclose(r.out64[t], acc, rtol=1e-12, atol=1e-12)
    assert np.isfinite(r.out64).all() and np.abs(r.out64).max() > 0.01
