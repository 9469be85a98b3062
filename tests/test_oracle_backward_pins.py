"""Pins of the backward oracle (oracle/moe_backward.py) to the forward definition: every gradient is
checked against central finite differences of oracle.moe_layer in float64, plus closed forms.
CPU only."""
import numpy as np
import pytest

import oracle.moe_backward as ob
import oracle.moe_oracle as om

EPS = 1e-5
PARAMS = ["A", "W_R", "bias", "W1", "W2", "W3", "Ws1", "Ws2", "Ws3"]


def make_case(seed, T=5, d=8, c=6, E=5, k=2, n_shared=0, c_shared=4, bias=False):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((T, d))
    W = {
        "W_R": rng.standard_normal((E, d)),
        "bias": rng.standard_normal(E) if bias else None,
        "W1": rng.standard_normal((E, c, d)) * 0.5,
        "W2": rng.standard_normal((E, c, d)) * 0.5,
        "W3": rng.standard_normal((E, d, c)) * 0.5,
    }
    if n_shared:
        W["Ws1"] = rng.standard_normal((n_shared * c_shared, d)) * 0.5
        W["Ws2"] = rng.standard_normal((n_shared * c_shared, d)) * 0.5
        W["Ws3"] = rng.standard_normal((d, n_shared * c_shared)) * 0.5
    dOut = rng.standard_normal((T, d))
    return rng, A, W, dOut


def loss(A, W, k, gate, renorm, dOut, n_shared, c_shared):
    out = om.moe_layer(A, W, k, gate, renorm, n_shared=n_shared, c_shared=c_shared)
    return float(np.sum(dOut * out["out"])), out["topk_idx"]


def check_fd(seed, gate, renorm, k=2, n_shared=0, bias=False, E=5):
    c_shared = 4
    rng, A, W, dOut = make_case(seed, k=k, n_shared=n_shared, c_shared=c_shared, bias=bias, E=E)
    g = ob.moe_layer_backward(A, W, k, gate, renorm, dOut, n_shared=n_shared, c_shared=c_shared)
    names = [p for p in PARAMS if (p == "A" or (W.get(p) is not None))]
    grad_key = {"A": "dA", "W_R": "dW_R", "bias": "dbias", "W1": "dW1", "W2": "dW2", "W3": "dW3",
                "Ws1": "dWs1", "Ws2": "dWs2", "Ws3": "dWs3"}
    for name in names:
        base = A if name == "A" else W[name]
        V = rng.standard_normal(base.shape)
        vals, sels = [], []
        for s in (+1, -1):
            if name == "A":
                l, sel = loss(A + s * EPS * V, W, k, gate, renorm, dOut, n_shared, c_shared)
            else:
                W2 = dict(W)
                W2[name] = W[name] + s * EPS * V
                l, sel = loss(A, W2, k, gate, renorm, dOut, n_shared, c_shared)
            vals.append(l)
            sels.append(sel)
        assert np.array_equal(sels[0], sels[1]), "selection changed under the perturbation (pick another seed)"
        fd = (vals[0] - vals[1]) / (2 * EPS)
        an = float(np.sum(g[grad_key[name]] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: finite difference {fd!r} vs analytic {an!r}"


@pytest.mark.parametrize("gate,renorm", [("softmax", False), ("softmax", True), ("sigmoid", True),
                                         ("sigmoid", False)])
@pytest.mark.parametrize("k", [1, 2, 3])
def test_gradients_match_finite_differences(gate, renorm, k):
    check_fd(100 + 7 * k, gate, renorm, k=k)


@pytest.mark.parametrize("gate,renorm", [("softmax", True), ("sigmoid", True)])
def test_gradients_with_shared_experts_and_bias(gate, renorm):
    check_fd(5, gate, renorm, k=2, n_shared=2, bias=True)


def test_top_k_equal_to_e_softmax():
    check_fd(9, "softmax", False, k=4, E=4)


def test_expert_without_rows_gets_zero_weight_gradients():
    rng, A, W, dOut = make_case(3, bias=True)
    W["bias"][2] = -1e3                                                  # expert 2 never wins
    L = om.router_logits(A, W["W_R"], W["bias"])
    idx = om.select_topk(L, 2)
    assert not (idx == 2).any()
    g = ob.moe_layer_backward(A, W, 2, "softmax", True, dOut)
    assert not g["dW1"][2].any() and not g["dW2"][2].any() and not g["dW3"][2].any()


def test_single_expert_top1_softmax_passes_no_router_gradient():
    rng, A, W, dOut = make_case(4, E=1, k=1)
    g = ob.moe_layer_backward(A, W, 1, "softmax", False, dOut)
    assert np.all(g["dlogits"] == 0) and np.all(g["dW_R"] == 0)
    # the layer is then the dense MLP: its input gradient is the MLP's
    dX, dW1, dW2, dW3 = ob.mlp_backward(A, W["W1"][0], W["W2"][0], W["W3"][0], dOut)
    np.testing.assert_allclose(g["dA"], dX, rtol=1e-12, atol=1e-12)


def test_zero_output_gradient_and_linearity():
    rng, A, W, d1 = make_case(6, n_shared=1)
    d2 = rng.standard_normal(d1.shape)
    kw = dict(n_shared=1, c_shared=4)
    g0 = ob.moe_layer_backward(A, W, 2, "sigmoid", True, np.zeros_like(d1), **kw)
    assert all(not np.any(g0[key]) for key in ("dA", "dW_R", "dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3"))
    g1 = ob.moe_layer_backward(A, W, 2, "sigmoid", True, d1, **kw)
    g2 = ob.moe_layer_backward(A, W, 2, "sigmoid", True, d2, **kw)
    g12 = ob.moe_layer_backward(A, W, 2, "sigmoid", True, 2 * d1 - d2, **kw)
    for key in ("dA", "dW_R", "dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3"):
        np.testing.assert_allclose(g12[key], 2 * g1[key] - g2[key], rtol=1e-10, atol=1e-10)


# ---- the FarSkip stack ----------------------------------------------------------------------------
def stack_case(seed, L=3, T=4, d=8, c=6, E=4, k=2, cs=4):
    rng = np.random.default_rng(seed)
    layers = []
    for _ in range(L):
        layers.append({"W_R": rng.standard_normal((E, d)), "bias": None,
                       "W1": rng.standard_normal((E, c, d)) * 0.4, "W2": rng.standard_normal((E, c, d)) * 0.4,
                       "W3": rng.standard_normal((E, d, c)) * 0.4, "Ws1": rng.standard_normal((cs, d)) * 0.4,
                       "Ws2": rng.standard_normal((cs, d)) * 0.4, "Ws3": rng.standard_normal((d, cs)) * 0.4})
    return rng, rng.standard_normal((T, d)), layers, rng.standard_normal((T, d))


@pytest.mark.parametrize("mode,mask", [("none", None), ("partial", None), ("outdated", None),
                                       ("partial", [1, 0, 1]), ("outdated", [0, 1, 1])])
def test_stack_gradients_match_finite_differences(mode, mask):
    rng, o0, layers, dOL = stack_case(21)
    k, gate, renorm = 2, "softmax", True
    kw = dict(mask=mask, n_shared=1, c_shared=4)
    g = ob.moe_stack_backward(o0, layers, k, gate, renorm, mode, dOL, **kw)

    def loss(o, lays):
        return float(np.sum(dOL * om.moe_stack(o, lays, k, gate, renorm, mode, **kw)))

    V = rng.standard_normal(o0.shape)
    fd = (loss(o0 + EPS * V, layers) - loss(o0 - EPS * V, layers)) / (2 * EPS)
    an = float(np.sum(g["do0"] * V))
    assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"do0: {fd!r} vs {an!r}"
    for j in range(len(layers)):
        for name, key in (("W_R", "dW_R"), ("W1", "dW1"), ("W3", "dW3"), ("Ws2", "dWs2"), ("Ws3", "dWs3")):
            V = rng.standard_normal(layers[j][name].shape)
            plus = [dict(l) for l in layers]
            minus = [dict(l) for l in layers]
            plus[j][name] = layers[j][name] + EPS * V
            minus[j][name] = layers[j][name] - EPS * V
            fd = (loss(o0, plus) - loss(o0, minus)) / (2 * EPS)
            an = float(np.sum(g["layers"][j][key] * V))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"layer {j} {name}: {fd!r} vs {an!r}"


def test_stack_of_one_layer_is_the_layer_plus_identity():
    rng, o0, layers, dOL = stack_case(22, L=1)
    for mode in ("none", "partial", "outdated"):
        g = ob.moe_stack_backward(o0, layers, 2, "sigmoid", True, mode, dOL, n_shared=1, c_shared=4)
        gl = ob.moe_layer_backward(o0, layers[0], 2, "sigmoid", True, dOL, n_shared=1, c_shared=4)
        np.testing.assert_allclose(g["do0"], dOL + gl["dA"], rtol=1e-12, atol=1e-12)
