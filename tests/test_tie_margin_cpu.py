"""Derivation of the top-k margin that the backward pass's FarSkip stack test keeps (BWD_TIE_MARGIN).

In that test the library and the oracle each run the stack forward themselves, so their layer inputs
drift apart by bf16 rounding flips (an fp32 sum on the GPU and an fp64 sum in the oracle falling on
opposite sides of a bf16 midpoint), and the drift compounds through the layers.  Every weight
gradient sums over all tokens, so the test needs every token routed alike on both sides at every
layer.  Here the kernels' arithmetic is emulated on the CPU (tests/kernel_emulation.py) and run
free beside the store-mirrored oracle, for the test's shapes, modes and masks and four seeded
inputs.  The largest logit drift among tokens still routed alike is measured; two logits can swap
order only when they are closer than twice it.  The margin must be at least four times the drift
(a factor of two beyond that), and every token whose oracle top-k gap exceeds the margin at every
layer must be routed identically by the emulation at every layer.
"""
import numpy as np
import pytest

import moe_inputs as mi
import oracle
from tests.helpers import BWD_STACK, BWD_STACK_CASES, BWD_TIE_MARGIN, make_layer
from tests.kernel_emulation import emulated_layer_fns

rnd = oracle.round_to_bf16
SEEDS = range(4)


def _weights():
    s = BWD_STACK
    layers = [make_layer(mi.seed_for(87, j, 1), s["T"], s["d"], s["E"], s["c"], s["cs"], bias=(j == 1))[1]
              for j in range(s["L"])]
    as_np = lambda W, dt: {key: (None if v is None else v.to(dt).numpy()) for key, v in W.items()}
    import torch
    return [as_np(W, torch.float64) for W in layers], [as_np(W, torch.float32) for W in layers]


@pytest.mark.parametrize("mode,mask", BWD_STACK_CASES)
def test_backward_stack_tie_margin(mode, mask):
    s = BWD_STACK
    W64, W32 = _weights()
    k, gate, renorm = s["k"], s["gate"], s["renorm"]
    drift = 0.0
    for seed in SEEDS:
        o0 = mi.normal((s["T"], s["d"]), 1.0, mi.seed_for(87, seed, 9)).numpy().astype(np.float64)
        rec_ref, rec_emu = [], []
        oracle.moe_stack(o0, W64, k, gate, renorm, mode, mask, 1, s["cs"], rnd, rec_ref, rnd)
        oracle.farskip_stack(o0, [emulated_layer_fns(W, k, gate, renorm) for W in W32], mode, mask, rnd, rec_emu)
        alike = np.ones(s["T"], bool)       # routed identically at every earlier layer
        clear = np.ones(s["T"], bool)       # oracle gap above the margin at every layer so far
        for j in range(s["L"]):
            L_ref = oracle.router_logits(rec_ref[j][0], W64[j]["W_R"], W64[j]["bias"])
            L_emu = oracle.router_logits(rec_emu[j][0], W64[j]["W_R"], W64[j]["bias"])
            if alike.any():
                drift = max(drift, float(np.abs(L_ref - L_emu).max(axis=1)[alike].max()))
            clear &= oracle.topk_gap(L_ref, k) >= BWD_TIE_MARGIN
            same = np.all(oracle.select_topk(L_ref, k) == oracle.select_topk(L_emu, k), axis=1)
            assert same[clear].all(), f"seed {seed} layer {j}: a token beyond the margin routed differently"
            alike &= same
    print(f"{mode} {mask}: largest logit drift {drift:.3e}, margin {BWD_TIE_MARGIN} = {BWD_TIE_MARGIN / drift:.1f} x drift")
    assert drift > 0.0          # the emulation does differ from the mirrored oracle
    assert 4.0 * drift <= BWD_TIE_MARGIN
