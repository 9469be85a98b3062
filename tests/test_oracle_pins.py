"""Pins for the CPU oracle: it is checked against brute force, hand-derived worked examples,
closed forms and special cases of the pages' equations, never against itself.

Each test names the plausible oracle mistake it would catch.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import moe_inputs as mi

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))
LN2, LN3 = math.log(2.0), math.log(3.0)


def frac(pq):
    return float(Fraction(int(pq[0]), int(pq[1])))


# ------------------------------------------------------------------------------------------
# top-k selection: exhaustive enumeration (catches wrong tie order, off-by-one k, ascending sort)
# ------------------------------------------------------------------------------------------
def brute_topk(vec, k):
    """Among all k-subsets, the one with the largest sum; among equal sums, the lexicographically
    smallest index tuple.  Slot order: descending value, then ascending index."""
    best, best_key = None, None
    for sub in itertools.combinations(range(len(vec)), k):
        key = (-sum(vec[j] for j in sub), sub)
        if best_key is None or key < best_key:
            best_key, best = key, sub
    return sorted(best, key=lambda j: (-vec[j], j))


@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 6])
def test_topk_exhaustive_small(E):
    vals = [0.0, 0.5, 1.0]
    vecs = np.array(list(itertools.product(vals, repeat=E)), dtype=np.float32)
    for k in range(1, E + 1):
        got = oracle.select_topk(vecs, k)
        for t, v in enumerate(vecs):
            assert list(got[t]) == brute_topk(list(map(float, v)), k), (E, k, v)


def test_topk_exhaustive_e8_selected_k():
    vals = [0.0, 0.5, 1.0]
    vecs = np.array(list(itertools.product(vals, repeat=8)), dtype=np.float32)
    for k in (2, 5, 7):
        got = oracle.select_topk(vecs, k)
        rows = np.random.default_rng(7).choice(len(vecs), 600, replace=False)
        for t in rows:
            assert list(got[t]) == brute_topk(list(map(float, vecs[t])), k)


def test_topk_signed_zero_is_a_tie():
    L = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]], dtype=np.float32)
    assert oracle.select_topk(L, 1).tolist() == [[0], [0]]


# ------------------------------------------------------------------------------------------
# gate weights: closed forms (catches softmax over k instead of E, wrong sign, missing renorm)
# ------------------------------------------------------------------------------------------
def test_softmax_scores_sum_to_one_and_k_equals_E():
    L = mi.logits(50, 9, 3).numpy()
    p = oracle.gate_scores(L, "softmax")
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
    idx = oracle.select_topk(L, 9)
    w = oracle.gate_weights(L, idx, "softmax", renormalize=False)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-14)


def test_renormalised_softmax_equals_softmax_over_selected():
    L = mi.logits(40, 16, 4).numpy().astype(np.float64)
    k = 4
    idx = oracle.select_topk(L, k)
    w = oracle.gate_weights(L, idx, "softmax", renormalize=True)
    sel = np.take_along_axis(L, idx.astype(np.int64), 1)
    # w_i = 1 / sum_j exp(l_j - l_i): a different formula for the same closed form
    ref = 1.0 / np.exp(sel[:, None, :] - sel[:, :, None]).sum(axis=2)
    np.testing.assert_allclose(w, ref, rtol=1e-13)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)


def test_sigmoid_scores_match_tanh_identity_and_renorm():
    L = mi.logits(30, 12, 5).numpy().astype(np.float64) * 4
    p = oracle.gate_scores(L, "sigmoid")
    np.testing.assert_allclose(p, 0.5 * (1.0 + np.tanh(0.5 * L)), rtol=1e-13)
    assert np.all((p > 0) & (p < 1))
    idx = oracle.select_topk(L, 3)
    w = oracle.gate_weights(L, idx, "sigmoid", renormalize=True)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)
    wn = oracle.gate_weights(L, idx, "sigmoid", renormalize=False)
    np.testing.assert_allclose(wn, 0.5 * (1.0 + np.tanh(0.5 * np.take_along_axis(L, idx.astype(np.int64), 1))),
                               rtol=1e-13)


def test_router_logits_library_matmul_and_bias():
    A = mi.normal((7, 5), 1.0, 11).numpy()
    W = mi.normal((3, 5), 1.0, 12).numpy()
    b = np.array([0.5, -1.0, 2.0])
    L = oracle.router_logits(A, W, b)
    ref = np.einsum("td,ed->te", A.astype(np.float64), W.astype(np.float64)) + b
    np.testing.assert_allclose(L, ref, rtol=1e-14, atol=1e-14)


# ------------------------------------------------------------------------------------------
# permutation: brute force over all maps (catches unstable order, off-by-one offsets, inverse swap)
# ------------------------------------------------------------------------------------------
def check_perm(idx, E):
    flat = [int(e) for e in np.asarray(idx).reshape(-1)]
    n = len(flat)
    offsets, sorted_src, dest_row = oracle.permute(idx, E)
    ref_src = sorted(range(n), key=lambda f: (flat[f], f))
    assert list(sorted_src) == ref_src
    ref_dest = [0] * n
    for r, f in enumerate(ref_src):
        ref_dest[f] = r
    assert list(dest_row) == ref_dest
    ref_off = [0] + list(itertools.accumulate(sum(1 for x in flat if x == e) for e in range(E)))
    assert list(offsets) == ref_off


def test_permute_bruteforce_all_maps_T2_k2_E3():
    n_cases = 0
    for flat in itertools.product(range(3), repeat=4):
        check_perm(np.array(flat, dtype=np.int32).reshape(2, 2), 3)
        n_cases += 1
    assert n_cases == 81
    # the 36 maps with distinct experts per token are among them
    distinct = [f for f in itertools.product(range(3), repeat=4) if f[0] != f[1] and f[2] != f[3]]
    assert len(distinct) == 36


def test_permute_random_matches_stable_argsort_and_inverse():
    idx = mi.topk_assignments(300, 17, 5, seed=21, zipf=1.2).numpy()
    offsets, sorted_src, dest_row = oracle.permute(idx, 17)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(sorted_src, np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(sorted_src[dest_row], np.arange(flat.size))
    np.testing.assert_array_equal(np.diff(offsets), np.bincount(flat, minlength=17))
    A = mi.normal((300, 4), 1.0, 22).numpy()
    Ap = oracle.permute_rows(A, sorted_src, 5)
    for f in range(flat.size):
        np.testing.assert_array_equal(Ap[dest_row[f]], A[f // 5])


# ------------------------------------------------------------------------------------------
# MLP: hand-derived example (catches gate/up swap, W3 transposed, SiLU vs sigmoid)
# ------------------------------------------------------------------------------------------
def test_silu_closed_forms():
    np.testing.assert_allclose(oracle.silu(np.array([0.0, LN3, -LN3, 40.0])),
                               [0.0, 0.75 * LN3, -0.25 * LN3, 40.0], rtol=1e-15, atol=0)


def test_mlp_golden():
    g = GOLDEN["mlp"]
    A = np.array(g["A"])
    W1 = np.array(g["W1"])
    W2 = np.array(g["W2_times_ln3"]) * LN3
    W3 = np.array(g["W3"])
    Y = oracle.mlp(A, W1, W2, W3)
    ref = np.array([[frac(pq) * LN3 for pq in row] for row in g["Y_times_ln3"]])
    np.testing.assert_allclose(Y, ref, rtol=1e-15, atol=1e-15)


# ------------------------------------------------------------------------------------------
# Routed layer: hand-derived example through routing, permutation, experts and combine
# ------------------------------------------------------------------------------------------
def golden_layer_weights():
    g = GOLDEN["routed_layer"]
    lnv = {"0": 0.0, "ln2": LN2, "ln3": LN3}
    W = dict(W_R=np.array([[lnv[v] for v in row] for row in g["W_R_times_ln"]]), bias=None,
             W1=np.array(g["W1"]), W2=np.array(g["W2_times_ln3"]) * LN3, W3=np.array(g["W3"]))
    return np.array(g["A"]), W


@pytest.mark.parametrize("case", range(len(GOLDEN["routed_layer"]["cases"])))
def test_routed_layer_golden(case):
    c = GOLDEN["routed_layer"]["cases"][case]
    A, W = golden_layer_weights()
    out = oracle.moe_layer(A, W, c["k"], c["gate"], c["renormalize"])
    assert out["topk_idx"].tolist() == c["topk_idx"]
    np.testing.assert_allclose(out["topk_w"], [[frac(pq) for pq in row] for row in c["weights"]], rtol=1e-14)
    np.testing.assert_allclose(out["R"][:, 0], [frac(pq) * LN3 for pq in c["R_times_ln3"]], rtol=1e-14)


# ------------------------------------------------------------------------------------------
# Closed forms of the MoE equation (catch combine using the wrong row/weight, dropped experts)
# ------------------------------------------------------------------------------------------
def small_weights(E, d, c, seed, std=0.3):
    return dict(W_R=mi.normal((E, d), std, seed).double().numpy(), bias=None,
                W1=mi.normal((E, c, d), std, seed + 1).double().numpy(),
                W2=mi.normal((E, c, d), std, seed + 2).double().numpy(),
                W3=mi.normal((E, d, c), std, seed + 3).double().numpy())


def test_single_expert_top1_is_the_dense_mlp():
    A = mi.normal((23, 6), 1.0, 31).double().numpy()
    W = small_weights(1, 6, 10, 32)
    for gate, renorm in (("softmax", False), ("softmax", True), ("sigmoid", True)):
        out = oracle.moe_layer(A, W, 1, gate, renorm)
        np.testing.assert_allclose(out["R"], oracle.mlp(A, W["W1"][0], W["W2"][0], W["W3"][0]), rtol=1e-12)


def test_topk_equals_E_softmax_is_the_full_weighted_sum():
    E, d, c = 5, 6, 7
    A = mi.normal((19, d), 1.0, 41).double().numpy()
    W = small_weights(E, d, c, 42)
    out = oracle.moe_layer(A, W, E, "softmax", False)
    L = A @ W["W_R"].T
    G = np.exp(L - L.max(1, keepdims=True))
    G = G / G.sum(1, keepdims=True)
    dense = sum(G[:, j:j + 1] * oracle.mlp(A, W["W1"][j], W["W2"][j], W["W3"][j]) for j in range(E))
    np.testing.assert_allclose(out["R"], dense, rtol=1e-11, atol=1e-13)


def test_combine_is_linear_in_weights_and_uses_dest_rows():
    T, k, d = 11, 3, 4
    Y = mi.normal((T * k, d), 1.0, 51).double().numpy()
    w = mi.uniform((T, k), 0.1, 1.0, 52).double().numpy()
    dest = mi.randperm(T * k, 53).numpy()
    out = oracle.combine(Y, w, dest)
    np.testing.assert_allclose(oracle.combine(Y, 2.5 * w, dest), 2.5 * out, rtol=1e-14)
    for t in range(T):
        ref = sum(w[t, i] * Y[dest[t * k + i]] for i in range(k))
        np.testing.assert_allclose(out[t], ref, rtol=1e-14)


def test_two_shared_experts_equal_one_concatenated():
    d, h = 6, 5
    Ws1 = mi.normal((2 * h, d), 0.4, 61).double().numpy()
    Ws2 = mi.normal((2 * h, d), 0.4, 62).double().numpy()
    Ws3 = mi.normal((d, 2 * h), 0.4, 63).double().numpy()
    A = mi.normal((9, d), 1.0, 64).double().numpy()
    two = oracle.shared_mlp(A, Ws1, Ws2, Ws3, 2, h)
    one = oracle.shared_mlp(A, Ws1, Ws2, Ws3, 1, 2 * h)
    np.testing.assert_allclose(two, one, rtol=1e-12)
    sep = oracle.mlp(A, Ws1[:h], Ws2[:h], Ws3[:, :h]) + oracle.mlp(A, Ws1[h:], Ws2[h:], Ws3[:, h:])
    np.testing.assert_allclose(two, sep, rtol=1e-12)


# ------------------------------------------------------------------------------------------
# FarSkip stack: hand-derived scalar example and special cases of section 3
# ------------------------------------------------------------------------------------------
@pytest.mark.parametrize("case", range(len(GOLDEN["stack"]["cases"])))
def test_stack_golden_scalar(case):
    g = GOLDEN["stack"]
    c = g["cases"][case]
    layers = [(lambda x, a=a: a * x, lambda x, b=b: b * x) for a, b in zip(g["a"], g["b"])]
    oL = oracle.farskip_stack(np.array([[g["o0"]]]), layers, c["mode"], c["mask"])
    assert float(oL[0, 0]) == c["oL"]


def moe_stack_setup(L=3, T=13, d=6, E=4, c=5, k=2, seed=70):
    o0 = mi.normal((T, d), 1.0, seed).double().numpy()
    Ws = []
    for j in range(L):
        W = small_weights(E, d, c, seed + 10 * (j + 1))
        W["Ws1"] = mi.normal((c, d), 0.3, seed + 10 * j + 5).double().numpy()
        W["Ws2"] = mi.normal((c, d), 0.3, seed + 10 * j + 6).double().numpy()
        W["Ws3"] = mi.normal((d, c), 0.3, seed + 10 * j + 7).double().numpy()
        Ws.append(W)
    return o0, Ws, dict(k=k, gate="sigmoid", renormalize=True, n_shared=1, c_shared=c)


def f_layer(W, kw):
    def f(x):
        return (oracle.moe_layer(x, W, kw["k"], kw["gate"], kw["renormalize"])["R"]
                + oracle.shared_mlp(x, W["Ws1"], W["Ws2"], W["Ws3"], 1, kw["c_shared"]))
    return f


def test_stack_L1_all_modes_equal():
    o0, Ws, kw = moe_stack_setup(L=1)
    outs = [oracle.moe_stack(o0, Ws, mode=m, **kw) for m in ("none", "partial", "outdated")]
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_stack_none_and_zero_mask_are_the_standard_residual_sum():
    o0, Ws, kw = moe_stack_setup(L=3)
    o = o0.copy()
    for W in Ws:  # o_k = o_{k-1} + f_k(o_{k-1}), summed out: o_L = o_0 + sum_i f_i(o_{i-1})
        o = o + f_layer(W, kw)(o)
    np.testing.assert_allclose(oracle.moe_stack(o0, Ws, mode="none", **kw), o, rtol=1e-12)
    np.testing.assert_allclose(oracle.moe_stack(o0, Ws, mode="partial", mask=[0, 0, 0], **kw), o, rtol=1e-12)


def test_stack_outdated_L2_closed_form():
    o0, Ws, kw = moe_stack_setup(L=2)
    ref = o0 + f_layer(Ws[0], kw)(o0) + f_layer(Ws[1], kw)(o0)
    np.testing.assert_allclose(oracle.moe_stack(o0, Ws, mode="outdated", **kw), ref, rtol=1e-12)


def test_stack_partial_L2_closed_form():
    o0, Ws, kw = moe_stack_setup(L=2)
    S1 = oracle.shared_mlp(o0, Ws[0]["Ws1"], Ws[0]["Ws2"], Ws[0]["Ws3"], 1, kw["c_shared"])
    ref = o0 + f_layer(Ws[0], kw)(o0) + f_layer(Ws[1], kw)(o0 + S1)
    np.testing.assert_allclose(oracle.moe_stack(o0, Ws, mode="partial", **kw), ref, rtol=1e-12)


def test_stack_partial_equals_none_when_routed_output_is_zero():
    o0, Ws, kw = moe_stack_setup(L=3)
    for W in Ws:
        W["W3"] = np.zeros_like(W["W3"])
    np.testing.assert_allclose(oracle.moe_stack(o0, Ws, mode="partial", **kw),
                               oracle.moe_stack(o0, Ws, mode="none", **kw), rtol=1e-13)


def test_stack_record_has_the_layer_inputs():
    o0, Ws, kw = moe_stack_setup(L=3)
    rec = []
    oracle.moe_stack(o0, Ws, mode="partial", record=rec, **kw)
    (x1, S1, R1, o1), (x2, S2, R2, o2), (x3, S3, R3, o3) = rec
    np.testing.assert_array_equal(x1, o0)
    np.testing.assert_allclose(x2, o0 + S1, rtol=1e-14)
    np.testing.assert_allclose(x3, o1 + S2, rtol=1e-14)
    np.testing.assert_allclose(o3, o0 + S1 + R1 + S2 + R2 + S3 + R3, rtol=1e-12)


# ------------------------------------------------------------------------------------------
# Attention + MoE wiring of section 3 (attn-in_k partial, mlp-in_k outdated)
# ------------------------------------------------------------------------------------------
def _scalar_attn_layers(g):
    return [(lambda x, v=v: v * x, lambda x, a=a: a * x, lambda x, b=b: b * x)
            for v, a, b in zip(g["alpha"], g["a"], g["b"])]


@pytest.mark.parametrize("case", range(len(GOLDEN["attn_moe_stack"]["cases"])))
def test_attn_moe_stack_golden_scalar(case):
    g = GOLDEN["attn_moe_stack"]
    c = g["cases"][case]
    rec = []
    oL = oracle.attn_moe_stack(np.array([[g["o0"]]]), _scalar_attn_layers(g), c["mode"], record=rec)
    assert [float(r[0][0, 0]) for r in rec] == c["attn_in"]
    assert [float(r[1][0, 0]) for r in rec] == c["mlp_in"]
    assert [float(r[5][0, 0]) for r in rec] == c["o"]
    assert float(oL[0, 0]) == c["o"][-1]


def attn_setup(L=3, T=11, d=6, E=4, c=5, k=2, seed=90):
    o0, Ws, kw = moe_stack_setup(L=L, T=T, d=d, E=E, c=c, k=k, seed=seed)
    Wa = [(mi.normal((c, d), 0.3, seed + 100 + 3 * j).double().numpy(),
           mi.normal((c, d), 0.3, seed + 101 + 3 * j).double().numpy(),
           mi.normal((d, c), 0.3, seed + 102 + 3 * j).double().numpy()) for j in range(L)]
    return o0, Ws, Wa, kw


def _attn_fn(Wa):
    return lambda x: oracle.mlp(x, *Wa)


def test_attn_moe_none_is_the_residual_sum_over_interleaved_sub_blocks():
    """Mode none is section 3's first equation over the 2L sub-blocks attn_1, moe_1, attn_2, ...:
    the (already pinned) MoE-only stack with skipping disabled, fed the interleaved blocks."""
    o0, Ws, Wa, kw = attn_setup()
    zero = lambda x: np.zeros_like(np.asarray(x, np.float64))  # noqa: E731
    blocks = []
    for W, A in zip(Ws, Wa):
        blocks.append((_attn_fn(A), zero))
        blocks.append((lambda x, W=W: oracle.shared_mlp(x, W["Ws1"], W["Ws2"], W["Ws3"], 1, kw["c_shared"]),
                       lambda x, W=W: oracle.moe_layer(x, W, kw["k"], kw["gate"], kw["renormalize"])["R"]))
    ref = oracle.farskip_stack(o0, blocks, "none")
    got = oracle.attn_moe_layer_stack(o0, Ws, Wa, kw["k"], kw["gate"], kw["renormalize"], "none", 1, kw["c_shared"])
    np.testing.assert_allclose(got, ref, rtol=1e-12)


def test_attn_moe_farskip_without_attention_is_the_standard_moe_stack():
    """With every attention output zero, mlp-in_k = o_{k-1} is the full residual: the MoE-only
    stack with skipping disabled."""
    o0, Ws, Wa, kw = attn_setup()
    Wa0 = [(a, b, np.zeros_like(c)) for a, b, c in Wa]
    got = oracle.attn_moe_layer_stack(o0, Ws, Wa0, kw["k"], kw["gate"], kw["renormalize"], "farskip", 1,
                                      kw["c_shared"])
    np.testing.assert_allclose(got, oracle.moe_stack(o0, Ws, mode="none", **kw), rtol=1e-12)


def test_attn_moe_farskip_without_routed_experts_is_parallel_blocks():
    """With every routed output zero, attn-in_k = mlp-in_k = o_{k-1}: each layer adds the attention
    and the shared experts of the same input, o_k = o_{k-1} + A_k(o_{k-1}) + S_k(o_{k-1})."""
    o0, Ws, Wa, kw = attn_setup()
    for W in Ws:
        W["W3"] = np.zeros_like(W["W3"])
    o = o0.copy()
    for W, A in zip(Ws, Wa):
        o = o + oracle.mlp(o, *A) + oracle.shared_mlp(o, W["Ws1"], W["Ws2"], W["Ws3"], 1, kw["c_shared"])
    got = oracle.attn_moe_layer_stack(o0, Ws, Wa, kw["k"], kw["gate"], kw["renormalize"], "farskip", 1,
                                      kw["c_shared"])
    np.testing.assert_allclose(got, o, rtol=1e-12)


def test_attn_moe_farskip_inputs_follow_the_page():
    """attn-in_k = o_{k-2} + attn-out_{k-1} + shared-out_{k-1}, mlp-in_k = o_{k-1}, and the page's
    decomposition mlp-in_k = attn-in_k + routed-out_{k-1}; every sub-block output enters o_L."""
    o0, Ws, Wa, kw = attn_setup(L=3)
    rec = []
    oracle.attn_moe_layer_stack(o0, Ws, Wa, kw["k"], kw["gate"], kw["renormalize"], "farskip", 1, kw["c_shared"],
                                record=rec)
    np.testing.assert_array_equal(rec[0][0], o0)
    np.testing.assert_array_equal(rec[0][1], o0)
    o_prev = o0
    for j in range(1, 3):
        a_in, m_in = rec[j][0], rec[j][1]
        A, S, R, o = rec[j - 1][2], rec[j - 1][3], rec[j - 1][4], rec[j - 1][5]
        np.testing.assert_allclose(a_in, o_prev + A + S, rtol=1e-14)
        np.testing.assert_array_equal(m_in, o)
        np.testing.assert_allclose(m_in, a_in + R, rtol=1e-12, atol=1e-14)
        o_prev = o
    total = o0 + sum(r[2] + r[3] + r[4] for r in rec)
    np.testing.assert_allclose(rec[-1][5], total, rtol=1e-12)


def test_attn_moe_one_layer():
    o0, Ws, Wa, kw = attn_setup(L=1)
    W = Ws[0]
    moe = oracle.moe_layer(o0, W, kw["k"], kw["gate"], kw["renormalize"])["R"] + \
        oracle.shared_mlp(o0, W["Ws1"], W["Ws2"], W["Ws3"], 1, kw["c_shared"])
    A = oracle.mlp(o0, *Wa[0])
    far = oracle.attn_moe_layer_stack(o0, Ws, Wa, kw["k"], kw["gate"], kw["renormalize"], "farskip", 1,
                                      kw["c_shared"])
    np.testing.assert_allclose(far, o0 + A + moe, rtol=1e-12)


# ------------------------------------------------------------------------------------------
# Precision helpers
# ------------------------------------------------------------------------------------------
def test_round_to_bf16_matches_torch():
    x = mi.normal((4096,), 3.0, 81).numpy()
    edge = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 1e-30, 0.0, -0.0, 65504.0],
                    dtype=np.float32)
    x = np.concatenate([x, edge])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(x).view(np.uint32), ref.view(np.uint32))


def test_topk_gap():
    L = np.array([[3.0, 1.0, 2.0, 2.0], [0.0, 5.0, 1.0, -1.0]])
    np.testing.assert_array_equal(oracle.topk_gap(L, 2), [0.0, 1.0])
    np.testing.assert_array_equal(oracle.topk_gap(L, 4), [np.inf, np.inf])


def test_store_hook_identity_and_rounding_bound():
    o0, Ws, kw = moe_stack_setup(L=2)
    exact = oracle.moe_stack(o0, Ws, mode="partial", **kw)
    ident = oracle.moe_stack(o0, Ws, mode="partial", store=lambda v: v, **kw)
    np.testing.assert_array_equal(exact, ident)
    A = o0
    W = Ws[0]
    Y = oracle.mlp(A, W["W1"][0], W["W2"][0], W["W3"][0])
    Yr = oracle.mlp(A, W["W1"][0], W["W2"][0], W["W3"][0], store=oracle.round_to_bf16)
    np.testing.assert_array_equal(Yr, oracle.round_to_bf16(Yr))  # stored values are bf16 values
    assert np.max(np.abs(Yr - Y)) <= 2 ** -7 * np.max(np.abs(Y))
