"""GPU parity of the MoE sublayer backward (moe_layer_backward) against the backward oracle.

The forward pieces the backward takes (selection, permutation, expert outputs Y) come from the
library's own forward calls; the router logits are computed on the host from the same bf16 inputs
and handed to the selection, so the selection is the oracle's (asserted).  The oracle runs the
forward and backward in float64 with bf16 rounding at the points the library keeps bf16
intermediates; every gradient must meet the bf16 bar max|err| <= 2e-2 * max|ref|.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
import oracle.moe_backward as ob
from tests.helpers import BWD_STACK, BWD_STACK_CASES, BWD_TIE_MARGIN, assert_parity, make_layer, to_np

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF = torch.bfloat16


@pytest.fixture(scope="module")
def ops():
    from mixture_experts_layer_sum_amd import ops as _ops
    return _ops


def run_backward(ops, A, W, dOut, k, gate, renorm, cs, with_dbias=True):
    T, d = A.shape
    E, c = W["W1"].shape[0], W["W1"].shape[1]
    Wd = {key: (v.to(DEV) if v is not None else None) for key, v in W.items()}
    Ad, dOutd = A.to(DEV), dOut.to(DEV)
    # logits from the same bf16 values, in float64 on the host, handed over in float32
    L = to_np(A).astype(np.float64) @ to_np(W["W_R"]).astype(np.float64).T
    if W["bias"] is not None:
        L = L + W["bias"].numpy().astype(np.float64)
    Ld = torch.from_numpy(L.astype(np.float32)).to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ops.moe_route_from_logits(Ld, k, gate, renorm, idx, w)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    src = torch.empty(T * k, dtype=torch.int32, device=DEV)
    dest = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ops.moe_permute(idx, E, off, src, dest)
    Y = torch.empty((T * k, d), dtype=BF, device=DEV)
    ops.moe_grouped_swiglu_gathered(Ad, src, k, off, Wd["W1"], Wd["W2"], Wd["W3"], Y)
    f32 = lambda *shape: torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    grads = {"dA": f32(T, d), "dW_R": f32(E, d), "dbias": f32(E) if with_dbias else None,
             "dW1": f32(E, c, d), "dW2": f32(E, c, d), "dW3": f32(E, d, c)}
    if cs:
        grads.update(dWs1=f32(cs, d), dWs2=f32(cs, d), dWs3=f32(d, cs))
    cfg = ops.stack_cfg(T, d, c, cs, E, k, gate, renorm, BF)
    ops.moe_layer_backward(Wd, cfg, Ad, Ld, idx, w, off, src, dest, Y, dOutd, grads)
    torch.cuda.synchronize()
    ref_idx = oracle.select_topk(L, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
    return {key: (to_np(v) if v is not None else None) for key, v in grads.items()}


def oracle_weights64(W):
    return {key: (to_np(v).astype(np.float64) if isinstance(v, torch.Tensor) else v) for key, v in W.items()}


CASES = [
    # T, d, E, k, c, cs, gate, renorm, bias, empty experts
    (256, 128, 8, 2, 128, 128, "softmax", True, False, ()),
    (500, 256, 16, 4, 192, 0, "sigmoid", True, True, ()),           # E padded to 64 for the router
    (333, 192, 8, 1, 64, 64, "softmax", False, True, (3, 5)),       # empty experts, top-1
    (2048, 1024, 64, 6, 512, 1024, "softmax", False, False, ()),    # several tiles in every dimension
    (700, 256, 24, 3, 256, 128, "sigmoid", False, True, ()),
]


@pytest.mark.parametrize("T,d,E,k,c,cs,gate,renorm,bias,empty", CASES)
def test_layer_backward_matches_oracle(ops, T, d, E, k, c, cs, gate, renorm, bias, empty):
    seed = mi.seed_for(88, T, d, E, k)
    A, W, dOut = make_layer(seed, T, d, E, c, cs, bias, empty)
    got = run_backward(ops, A, W, dOut, k, gate, renorm, cs)
    W64 = oracle_weights64(W)
    ref = ob.moe_layer_backward(to_np(A).astype(np.float64), W64, k, gate, renorm, dOut.numpy().astype(np.float64),
                                n_shared=1 if cs else 0, c_shared=cs, store=oracle.round_to_bf16)
    keys = ["dA", "dW_R", "dW1", "dW2", "dW3"] + (["dbias"] if bias else []) + (["dWs1", "dWs2", "dWs3"] if cs else [])
    for key in keys:
        assert_parity(got[key], ref[key], BF, key)
    for e in empty:
        assert not got["dW1"][e].any() and not got["dW2"][e].any() and not got["dW3"][e].any()


def test_layer_backward_dsv3_dims(ops):
    """The DeepSeek-V3 layer's widths (d = 7168, c = 2048, one 2048-wide shared expert, sigmoid
    renormalised top-8) over 16 experts and 128 tokens."""
    T, d, E, k, c, cs = 128, 7168, 16, 8, 2048, 2048
    A, W, dOut = make_layer(mi.seed_for(88, T, d, E, k), T, d, E, c, cs, bias=False)
    got = run_backward(ops, A, W, dOut, k, "sigmoid", True, cs, with_dbias=False)
    ref = ob.moe_layer_backward(to_np(A).astype(np.float64), oracle_weights64(W), k, "sigmoid", True,
                                dOut.numpy().astype(np.float64), n_shared=1, c_shared=cs, store=oracle.round_to_bf16)
    for key in ("dA", "dW_R", "dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3"):
        assert_parity(got[key], ref[key], BF, key)


def test_layer_backward_is_deterministic(ops):
    T, d, E, k, c, cs = 300, 128, 8, 2, 128, 64
    A, W, dOut = make_layer(7, T, d, E, c, cs, bias=True)
    g1 = run_backward(ops, A, W, dOut, k, "softmax", True, cs)
    g2 = run_backward(ops, A, W, dOut, k, "softmax", True, cs)
    for key in g1:
        if g1[key] is not None:
            np.testing.assert_array_equal(g1[key], g2[key])


def test_layer_backward_dsv3_full_size_sampled(ops):
    """The DeepSeek-V3-shaped layer at full size (65536 tokens, 256 experts, top-8 sigmoid
    renormalised, d = 7168, c = 2048, one 2048-wide shared expert): dA of 256 sampled tokens (their
    2048 slots reach nearly every expert) and the weight gradients of eight experts over all of their
    rows (the first and the last, the largest and the smallest group, four seeded others) against
    the oracle, composed from its per-token and per-expert steps.  The oracle runs expert-major: each
    expert the samples need is fetched once, its contributions to every sampled token routed to it
    are added, and its weight gradients are checked if it is one of the eight.  The selection is
    checked for every token."""
    cfg = {c.name: c for c in mi.CONFIGS}["dsv3-stack"]
    T, d, E, k, c, cs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.c, cfg.shared_width
    W = mi.layer_weights(cfg, 0, DEV)
    A = mi.activations(cfg, DEV)
    dOut = mi.normal((T, d), 1.0, mi.seed_for(cfg.cfg_id, 0, mi.T_MISC, 0, 31), DEV)
    A64 = to_np(A).astype(np.float64)
    WR64 = to_np(W["W_R"]).astype(np.float64)
    L = A64 @ WR64.T
    if W.get("bias") is not None:
        L = L + W["bias"].cpu().numpy().astype(np.float64)
    Ld = torch.from_numpy(L.astype(np.float32)).to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ops.moe_route_from_logits(Ld, k, cfg.gate, cfg.renormalize, idx, w)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    src = torch.empty(T * k, dtype=torch.int32, device=DEV)
    dest = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ops.moe_permute(idx, E, off, src, dest)
    Y = torch.empty((T * k, d), dtype=BF, device=DEV)
    ops.moe_grouped_swiglu_gathered(A, src, k, off, W["W1"], W["W2"], W["W3"], Y)
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=DEV)
    grads = {"dA": f32(T, d), "dW_R": f32(E, d), "dW1": f32(E, c, d), "dW2": f32(E, c, d), "dW3": f32(E, d, c),
             "dWs1": f32(cs, d), "dWs2": f32(cs, d), "dWs3": f32(d, cs)}
    bcfg = ops.stack_cfg(T, d, c, cs, E, k, cfg.gate, cfg.renormalize, BF)
    ops.moe_layer_backward(W, bcfg, A, Ld, idx, w, off, src, dest, Y, dOut, grads)
    torch.cuda.synchronize()
    idx_np = idx.cpu().numpy()
    ref_idx = oracle.select_topk(L, k)
    np.testing.assert_array_equal(idx_np, ref_idx)
    ref_w = oracle.gate_weights(L, ref_idx, cfg.gate, cfg.renormalize)
    dOut64 = dOut.cpu().numpy().astype(np.float64)
    st = oracle.round_to_bf16

    counts = np.bincount(ref_idx.ravel(), minlength=E)
    others = np.random.default_rng(mi.seed_for(cfg.cfg_id, 0, mi.T_SAMPLE, 1, 31)).permutation(E)
    sel = {0, E - 1, int(np.argmax(counts)), int(np.argmin(counts))}
    for e in others:
        if len(sel) == 8:
            break
        sel.add(int(e))
    rows_t = mi.sample_rows(T, 256, mi.seed_for(cfg.cfg_id, 0, mi.T_SAMPLE, 0, 31)).numpy()
    n = len(rows_t)
    x_s, dOut_s, idx_s = A64[rows_t], dOut64[rows_t], ref_idx[rows_t]
    dX = np.zeros((n, d))          # the routed experts' input gradients of the sampled tokens
    dw = np.zeros((n, k))          # dLoss / d(gate weight) per sampled slot
    for e in sorted(set(idx_s.ravel().tolist()) | sel):
        W1e, W2e, W3e = (to_np(W[key][e]).astype(np.float64) for key in ("W1", "W2", "W3"))
        tt, ii = np.nonzero(idx_s == e)       # a token lists an expert at most once
        if len(tt):
            y = oracle.mlp(x_s[tt], W1e, W2e, W3e, store=st)
            dw[tt, ii] = np.sum(dOut_s[tt] * y, axis=1)
            dX[tt] += ob.mlp_backward(x_s[tt], W1e, W2e, W3e, ref_w[rows_t[tt], ii][:, None] * dOut_s[tt],
                                      store=st)[0]
        if e in sel:   # the weight gradients over all of the expert's rows
            tok, slot = np.nonzero(ref_idx == e)
            dY = ref_w[tok, slot][:, None] * dOut64[tok]
            _, dW1, dW2, dW3 = ob.mlp_backward(A64[tok], W1e, W2e, W3e, dY, store=st)
            for key, ref in (("dW1", dW1), ("dW2", dW2), ("dW3", dW3)):
                assert_parity(grads[key][e].cpu().numpy(), ref, BF, f"{key} of expert {e} ({counts[e]} rows)")
    Ws = [to_np(W[key]).astype(np.float64) for key in ("Ws1", "Ws2", "Ws3")]
    dL = ob.gate_backward(L[rows_t], idx_s, dw, cfg.gate, cfg.renormalize)
    ref_dA = dX + ob.router_backward(x_s, WR64, dL, store=st)[0] + ob.mlp_backward(x_s, *Ws, dOut_s, store=st)[0]
    got_dA = grads["dA"][torch.from_numpy(rows_t).to(DEV)].cpu().numpy()
    assert_parity(got_dA, ref_dA, BF, f"dA of {n} sampled tokens ({len(set(idx_s.ravel().tolist()))} experts)")
    for key in ("dA", "dW_R", "dWs1", "dWs2", "dWs3"):
        assert torch.isfinite(grads[key]).all().item(), key


# =================================================================================================
# FarSkip stack backward
# =================================================================================================
def clean_stack_input(o0, layers64, k, gate, renorm, mode, mask, cs, delta=BWD_TIE_MARGIN, seed=0):
    """Redraw the token rows whose top-k choice is within delta of a tie at any layer of the
    oracle's forward (tokens are independent through the stack), so that both sides choose alike:
    every weight gradient sums over all tokens, so one token routed differently would move it.
    delta is derived in tests/test_tie_margin_cpu.py."""
    o0 = o0.copy()
    rng = np.random.default_rng(seed)
    for _ in range(30):
        rec = []
        oracle.moe_stack(o0, layers64, k, gate, renorm, mode, mask, 1 if cs else 0, cs, oracle.round_to_bf16, rec,
                         oracle.round_to_bf16)
        gap = np.full(o0.shape[0], np.inf)
        for j, (x, *_rest) in enumerate(rec):
            L = oracle.router_logits(x, layers64[j]["W_R"], layers64[j].get("bias"))
            gap = np.minimum(gap, oracle.topk_gap(L, k))
        bad = gap < delta
        if not bad.any():
            return o0
        o0[bad] = rng.standard_normal((int(bad.sum()), o0.shape[1]))
    raise AssertionError("could not draw a stack input without near-ties")


@pytest.mark.parametrize("mode,mask", BWD_STACK_CASES)
def test_stack_backward_matches_oracle(ops, mode, mask):
    T, d, E, k, c, cs, L = (BWD_STACK[key] for key in ("T", "d", "E", "k", "c", "cs", "L"))
    gate, renorm = BWD_STACK["gate"], BWD_STACK["renorm"]
    layers = [make_layer(mi.seed_for(87, j, 1), T, d, E, c, cs, bias=(j == 1))[1] for j in range(L)]
    layers64 = [oracle_weights64(W) for W in layers]
    o0 = clean_stack_input(mi.normal((T, d), 1.0, mi.seed_for(87, 0, 9)).numpy().astype(np.float64), layers64, k, gate,
                           renorm, mode, mask, cs, seed=mi.seed_for(87, 0, 10))
    dOL = mi.normal((T, d), 1.0, mi.seed_for(87, 0, 11)).numpy().astype(np.float64)
    Wd = [{key: (v.to(DEV) if v is not None else None) for key, v in W.items()} for W in layers]
    f32 = lambda *shape: torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)
    grads = [{"dA": f32(T, d), "dW_R": f32(E, d), "dbias": f32(E) if W["bias"] is not None else None,
              "dW1": f32(E, c, d), "dW2": f32(E, c, d), "dW3": f32(E, d, c), "dWs1": f32(cs, d), "dWs2": f32(cs, d),
              "dWs3": f32(d, cs)} for W in layers]
    o0d = torch.from_numpy(o0.astype(np.float32)).to(DEV)
    dOLd = torch.from_numpy(dOL.astype(np.float32)).to(DEV)
    dO0 = f32(T, d)
    cfg = ops.stack_cfg(T, d, c, cs, E, k, gate, renorm, BF)
    ops.farskip_stack_backward(Wd, cfg, mode, o0d, dOLd, dO0, grads, skip_mask=mask)
    torch.cuda.synchronize()
    ref = ob.moe_stack_backward(o0, layers64, k, gate, renorm, mode, dOL, mask, n_shared=1, c_shared=cs,
                                round_inputs=oracle.round_to_bf16, store=oracle.round_to_bf16)
    assert_parity(to_np(dO0), ref["do0"], BF, "dO0")
    for j in range(L):
        for key in ("dA", "dW_R", "dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3") + (("dbias",) if j == 1 else ()):
            assert_parity(to_np(grads[j][key]), ref["layers"][j][key], BF, f"layer {j} {key}")
