"""Planted mistakes in the oracle must make its pins fail.

Each case swaps one oracle function for a plausibly wrong variant (on the CPU, inside this test
only) and runs the pins that should catch it.
"""
import numpy as np
import pytest

import oracle
import oracle.moe_oracle as om
from tests import test_oracle_pins as pins


def _mlp_gate_up_swapped(X, W1, W2, W3, store=None):
    X = np.asarray(X, np.float64)
    return ((X @ np.asarray(W2, np.float64).T) * om.silu(X @ np.asarray(W1, np.float64).T)) @ np.asarray(W3, np.float64).T


def _mlp_w3_untransposed(X, W1, W2, W3, store=None):
    X = np.asarray(X, np.float64)
    H = (X @ np.asarray(W1, np.float64).T) * om.silu(X @ np.asarray(W2, np.float64).T)
    return H @ np.asarray(W3, np.float64)


def _mlp_sigmoid_not_silu(X, W1, W2, W3, store=None):
    X = np.asarray(X, np.float64)
    G = X @ np.asarray(W2, np.float64).T
    H = (X @ np.asarray(W1, np.float64).T) * (1 / (1 + np.exp(-G)))
    return H @ np.asarray(W3, np.float64).T


def _scores_softmax_wrong_sign(logits, gate):
    L = np.asarray(logits, np.float64)
    if gate == "softmax":
        e = np.exp(-(L - L.min(1, keepdims=True)))
        return e / e.sum(1, keepdims=True)
    return 1 / (1 + np.exp(-L))


def _weights_softmax_over_k(logits, idx, gate, renormalize):
    sel = np.take_along_axis(np.asarray(logits, np.float64), np.asarray(idx, np.int64), 1)
    p = om.gate_scores(sel, gate)
    return p / p.sum(1, keepdims=True) if renormalize else p


def _topk_ties_to_higher_index(logits, k):
    L = np.asarray(logits, np.float64)
    E = L.shape[1]
    order = np.argsort(-L[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _topk_unordered(logits, k):
    return np.sort(ORIG["select_topk"](logits, k), axis=1)


def _permute_unstable(topk_idx, E):
    off, src, dest = ORIG["permute"](topk_idx, E)
    src = src.copy()
    for e in range(E):
        src[off[e]:off[e + 1]] = src[off[e]:off[e + 1]][::-1]
    dest = np.empty_like(src)
    dest[src] = np.arange(src.size)
    return off, src, dest


def _permute_offsets_shifted(topk_idx, E):
    off, src, dest = ORIG["permute"](topk_idx, E)
    return np.concatenate([[0], off[:-1]]).astype(np.int32), src, dest


def _combine_weight_index_reversed(Y, topk_w, dest_row, addend=None, residual=None):
    return ORIG["combine"](Y, np.asarray(topk_w)[:, ::-1], dest_row, addend, residual)


def _combine_dropped_last_slot(Y, topk_w, dest_row, addend=None, residual=None):
    w = np.array(topk_w, np.float64, copy=True)
    w[:, -1] = 0
    return ORIG["combine"](Y, w, dest_row, addend, residual)


def _stack_partial_without_residual(o0, layers, mode, mask=None, round_inputs=None, record=None):
    # partial input taken as S_k alone (o_{k-1} dropped)
    n = len(layers)
    mask = [1] * n if mask is None else list(mask)
    o_prev = np.asarray(o0, np.float64)
    x = o_prev
    for j, (sf, rf) in enumerate(layers):
        S, R = sf(x), rf(x)
        o = o_prev + S + R
        x_next = o if (mode == "none" or not mask[j]) else (S if mode == "partial" else o_prev)
        o_prev, x = o, x_next
    return o_prev


def _stack_outdated_as_current(o0, layers, mode, mask=None, round_inputs=None, record=None):
    return ORIG["farskip_stack"](o0, layers, "none" if mode == "outdated" else mode, mask, round_inputs, record)


def _stack_dropped_o0(o0, layers, mode, mask=None, round_inputs=None, record=None):
    return ORIG["farskip_stack"](o0, layers, mode, mask, round_inputs, record) - np.asarray(o0, np.float64)


def _attn_input_not_skipped(o0, layers, mode, round_inputs=None, record=None):
    # attention fed the full o_{k-1} (the routed output not skipped), MoE input as the page's
    o_prev = np.asarray(o0, np.float64)
    for af, sf, rf in layers:
        A = af(o_prev)
        S, R = sf(o_prev), rf(o_prev)
        o_prev = o_prev + A + S + R
    return o_prev


def _mlp_input_without_routed(o0, layers, mode, round_inputs=None, record=None):
    # MoE fed the partial activation too (routed-out_{k-1} dropped from mlp-in_k)
    o_prev = np.asarray(o0, np.float64)
    partial = o_prev
    for af, sf, rf in layers:
        A = af(partial)
        S, R = sf(partial), rf(partial)
        o = o_prev + A + S + R
        partial = o_prev + A + S
        o_prev = o
    return o_prev


def _attn_partial_with_routed_not_shared(o0, layers, mode, round_inputs=None, record=None):
    # the partial activation built from the routed output instead of the shared one
    o_prev = np.asarray(o0, np.float64)
    partial = o_prev
    for af, sf, rf in layers:
        A = af(partial if mode == "farskip" else o_prev)
        m = o_prev if mode == "farskip" else o_prev + A
        S, R = sf(m), rf(m)
        o = o_prev + A + S + R
        partial = o_prev + A + R
        o_prev = o
    return o_prev


ORIG = {name: getattr(om, name) for name in ("select_topk", "permute", "combine", "farskip_stack", "mlp",
                                            "gate_scores", "gate_weights", "attn_moe_stack")}

GOLDEN_ROUTED = [lambda c=c: pins.test_routed_layer_golden(c) for c in range(6)]
GOLDEN_STACK = [lambda c=c: pins.test_stack_golden_scalar(c) for c in range(5)]
GOLDEN_ATTN = [lambda c=c: pins.test_attn_moe_stack_golden_scalar(c) for c in range(2)]

CASES = [
    ("mlp", _mlp_gate_up_swapped, [pins.test_mlp_golden]),
    ("mlp", _mlp_w3_untransposed, [pins.test_mlp_golden]),
    ("mlp", _mlp_sigmoid_not_silu, [pins.test_mlp_golden]),
    ("gate_scores", _scores_softmax_wrong_sign, [pins.test_softmax_scores_sum_to_one_and_k_equals_E] + GOLDEN_ROUTED),
    ("gate_weights", _weights_softmax_over_k, GOLDEN_ROUTED),
    ("select_topk", _topk_ties_to_higher_index, [lambda: pins.test_topk_exhaustive_small(3)]),
    ("select_topk", _topk_unordered, [lambda: pins.test_topk_exhaustive_small(4)]),
    ("permute", _permute_unstable, [pins.test_permute_bruteforce_all_maps_T2_k2_E3]),
    ("permute", _permute_offsets_shifted, [pins.test_permute_bruteforce_all_maps_T2_k2_E3]),
    ("combine", _combine_weight_index_reversed, GOLDEN_ROUTED + [pins.test_combine_is_linear_in_weights_and_uses_dest_rows]),
    ("combine", _combine_dropped_last_slot, GOLDEN_ROUTED + [pins.test_topk_equals_E_softmax_is_the_full_weighted_sum]),
    ("farskip_stack", _stack_partial_without_residual, GOLDEN_STACK),
    ("farskip_stack", _stack_outdated_as_current, GOLDEN_STACK),
    ("farskip_stack", _stack_dropped_o0, GOLDEN_STACK),
    ("attn_moe_stack", _attn_input_not_skipped, GOLDEN_ATTN),
    ("attn_moe_stack", _mlp_input_without_routed, GOLDEN_ATTN),
    ("attn_moe_stack", _attn_partial_with_routed_not_shared, GOLDEN_ATTN),
]


# ---- MXFP8 oracle (oracle/mxfp8.py) ----------------------------------------------------------
from tests import test_oracle_mxfp8_pins as mxpins  # noqa: E402

mx = oracle.mxfp8
MX_ORIG = {name: getattr(mx, name) for name in ("block_exponent", "e4m3_encode", "mx_quantize", "mlp_mxfp8")}


def _scale_floor_rule(amax):          # the clipping rule floor(log2(amax)) - 8
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(amax)
    return np.clip(np.where(amax > 0, e - 9, 0), -127, 127).astype(np.int64)


def _scale_one_too_large(amax):
    return MX_ORIG["block_exponent"](amax) + 1


def _encode_truncating(x):
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    code = np.maximum(np.searchsorted(mx._POS_VALS, a, side="right") - 1, 0)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _encode_ties_away(x):
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), 448.0)
    hi = np.minimum(np.searchsorted(mx._POS_VALS, a, side="left"), 0x7E)
    lo = np.maximum(hi - 1, 0)
    code = np.where((mx._POS_VALS[hi] - a) <= (a - mx._POS_VALS[lo]), hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def _quantize_blocks_of_16(X, block=32):
    return MX_ORIG["mx_quantize"](X, 16)


def _mlp_hidden_not_quantised(X, W1q, W2q, W3q, hidden_store=None):
    Xd = mx.mx_dequantize(*mx.mx_quantize(X))
    H = (Xd @ mx.mx_dequantize(*W1q).T) * mx.silu(Xd @ mx.mx_dequantize(*W2q).T)
    return H @ mx.mx_dequantize(*W3q).T


def _mlp_gate_up_swapped_fp8(X, W1q, W2q, W3q, hidden_store=None):
    return MX_ORIG["mlp_mxfp8"](X, W2q, W1q, W3q, hidden_store)


MX_CASES = [
    ("block_exponent", _scale_floor_rule, [mxpins.test_mx_block_scale_rule]),
    ("block_exponent", _scale_one_too_large, [mxpins.test_mx_representable_blocks_quantize_exactly]),
    ("e4m3_encode", _encode_truncating, [mxpins.test_e4m3_ties_to_even_and_saturation]),
    ("e4m3_encode", _encode_ties_away, [mxpins.test_e4m3_ties_to_even_and_saturation]),
    ("mx_quantize", _quantize_blocks_of_16, [mxpins.test_mx_block_scale_rule]),
    ("mlp_mxfp8", _mlp_hidden_not_quantised, [mxpins.test_mlp_mxfp8_hand_example_quantises_the_hidden]),
    ("mlp_mxfp8", _mlp_gate_up_swapped_fp8, [mxpins.test_mlp_mxfp8_equals_the_mlp_on_representable_operands]),
]


@pytest.mark.parametrize("i", range(len(MX_CASES)), ids=[c[1].__name__.lstrip("_") for c in MX_CASES])
def test_planted_mxfp8_mistake_is_caught(i, monkeypatch):
    name, bad, pin_fns = MX_CASES[i]
    monkeypatch.setattr(mx, name, bad)
    caught = 0
    for fn in pin_fns:
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {bad.__name__}"


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[1].__name__.lstrip("_") for c in CASES])
def test_planted_mistake_is_caught(i, monkeypatch):
    name, bad, pin_fns = CASES[i]
    monkeypatch.setattr(om, name, bad)
    monkeypatch.setattr(oracle, name, bad)
    caught = 0
    for fn in pin_fns:
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake {bad.__name__}"


# ---- backward oracle --------------------------------------------------------------------------
import oracle.moe_backward as ob  # noqa: E402
from tests import test_oracle_backward_pins as bpins  # noqa: E402

BWD_ORIG = {n: getattr(ob, n) for n in ("silu_grad", "gate_backward", "mlp_backward", "unpermute_sum",
                                        "router_backward", "combine_backward")}


def _silu_grad_sigmoid_only(g):
    return 1.0 / (1.0 + np.exp(-np.asarray(g, np.float64)))


def _gate_backward_no_renorm_term(logits, topk_idx, dw, gate, renormalize):
    return BWD_ORIG["gate_backward"](logits, topk_idx, dw, gate, False)


def _mlp_backward_dw3_from_u(X, W1, W2, W3, dY, store=None):
    dX, dW1, dW2, dW3 = BWD_ORIG["mlp_backward"](X, W1, W2, W3, dY, store)
    U = np.asarray(X, np.float64) @ np.asarray(W1, np.float64).T
    return dX, dW1, dW2, np.asarray(dY, np.float64).T @ U


def _unpermute_by_sorted_src(dXp, dest_row, k):
    inv = np.empty_like(np.asarray(dest_row))
    inv[np.asarray(dest_row)] = np.arange(len(dest_row))
    return BWD_ORIG["unpermute_sum"](dXp, inv, k)


def _router_backward_no_input_gradient(A, W_R, dlogits, store=None):
    dA, dW_R, db = BWD_ORIG["router_backward"](A, W_R, dlogits, store)
    return np.zeros_like(dA), dW_R, db


def _combine_backward_unweighted(dOut, Y, topk_w, dest_row):
    return BWD_ORIG["combine_backward"](dOut, Y, np.ones_like(np.asarray(topk_w, np.float64)), dest_row)


def _fd_cases():
    bpins.test_gradients_match_finite_differences("softmax", True, 2)
    bpins.test_gradients_match_finite_differences("sigmoid", True, 2)


BWD_CASES = [
    ("silu_grad", _silu_grad_sigmoid_only),
    ("gate_backward", _gate_backward_no_renorm_term),
    ("mlp_backward", _mlp_backward_dw3_from_u),
    ("unpermute_sum", _unpermute_by_sorted_src),
    ("router_backward", _router_backward_no_input_gradient),
    ("combine_backward", _combine_backward_unweighted),
]


@pytest.mark.parametrize("i", range(len(BWD_CASES)), ids=[c[1].__name__.lstrip("_") for c in BWD_CASES])
def test_planted_backward_mistake_is_caught(i, monkeypatch):
    name, bad = BWD_CASES[i]
    monkeypatch.setattr(ob, name, bad)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _fd_cases()


# ---- the stack's gradient routing -----------------------------------------------------------------
def _stack_backward_without_shared_feed(o0, layer_weights, k, gate, renormalize, mode, dOL, mask=None, n_shared=0,
                                        c_shared=0, round_inputs=None, store=None):
    # "partial" treated like "outdated" in the reverse pass: S_j no longer receives dLoss/dx_{j+1}
    m = "outdated" if mode == "partial" else mode
    g = STACK_ORIG(o0, layer_weights, k, gate, renormalize, m, dOL, mask, n_shared, c_shared, round_inputs, store)
    return g


def _stack_backward_skip_to_wrong_output(o0, layer_weights, k, gate, renormalize, mode, dOL, mask=None, n_shared=0,
                                         c_shared=0, round_inputs=None, store=None):
    # the skipped input's gradient sent to o_{j-1} as if there were no skip
    return STACK_ORIG(o0, layer_weights, k, gate, renormalize, "none", dOL, mask, n_shared, c_shared, round_inputs,
                      store)


STACK_ORIG = ob.moe_stack_backward


@pytest.mark.parametrize("bad", [_stack_backward_without_shared_feed, _stack_backward_skip_to_wrong_output],
                         ids=["without_shared_feed", "skip_to_wrong_output"])
def test_planted_stack_backward_mistake_is_caught(bad, monkeypatch):
    monkeypatch.setattr(ob, "moe_stack_backward", bad)
    with pytest.raises(AssertionError):
        bpins.test_stack_gradients_match_finite_differences("partial", None)
