"""A layer's forward pass captured in a HIP graph (MoELayerPlan.graph) replays to exactly the
bytes of the eager pass.

Every replay is checked against an eager pass of its own inputs, with eager work (fills of
the outputs, a whole eager pass of another plan) and device synchronisations between the
replays; odd replays run on new inputs copied into the captured input buffers.  Every
intermediate is compared byte for byte (routing, permutation, quantised tokens, act, its
requantisation, Y, the output): the pass is deterministic, so any difference is a capture
error.  Layers: a 32-expert layer (K-split kernels, items looked up in the kernel), the TP8
share (its down GEMM's schedule kernel writes the item list inside the graph) and the decode
layer (four-wave kernels)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

MID = synth.Layer("mid_t256_e32_k4_h512_i256", T=256, E=32, k=4, H=512, I=256)


def _inputs(L, seed):
    rng = np.random.default_rng(seed)
    logits = torch.from_numpy(rng.standard_normal((L.T, L.E)).astype(np.float32)).cuda()
    x = torch.from_numpy(synth.bf16_bits(rng.standard_normal((L.T, L.H)).astype(np.float32)).view(np.int16))
    return logits, x.cuda().view(torch.bfloat16)


def _buffers(plan):
    return [plan.ids, plan.w, plan.off, plan.row_src, plan.tsr, plan.xq.q, plan.xq.sf, plan.xq.gs, plan.act,
            plan.actq.q, plan.actq.sf, plan.actq.gs, plan.Y, plan.out]


def _snapshot(plan):
    return [b.clone() for b in _buffers(plan)]


def _fill(plan, v):
    for b in _buffers(plan):
        b.view(torch.uint8).fill_(v)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("L", [MID, synth.LAYER_TP8, synth.LAYER_DECODE], ids=lambda L: L.name)
def test_graph_replays_match_eager(L):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    import block_scaled_fp4_02_amd as moe
    torch.cuda.set_device(0)
    print(f"graph: {L.name}: weights", flush=True)
    W1, W2 = bench.make_weights(L, moe, torch)
    eager = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, W1, W2)
    graphed = moe.MoELayerPlan(L.T, L.E, L.k, L.H, L.I, W1, W2)
    ins = [_inputs(L, 10), _inputs(L, 11)]
    refs = []
    for logits, x in ins:
        eager.forward(logits, x)
        torch.cuda.synchronize()
        refs.append(_snapshot(eager))
    static_logits, static_x = ins[0][0].clone(), ins[0][1].clone()
    print(f"graph: {L.name}: capture", flush=True)
    g = graphed.graph(static_logits, static_x)
    for r in range(4):
        which = r % 2
        _fill(graphed, 0xA5 + r)
        static_logits.copy_(ins[which][0])
        static_x.copy_(ins[which][1])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(graphed)
        for i, (a, b) in enumerate(zip(refs[which], got)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), (L.name, r, i)
        print(f"graph: {L.name}: replay {r} (inputs {which}) matches the eager pass", flush=True)
        # eager work between replays
        eager.forward(*ins[1 - which])
        torch.cuda.synchronize()
