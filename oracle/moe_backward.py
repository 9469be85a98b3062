"""CPU oracle: the backward pass of one MoE sublayer, written plainly.

TEST INFRASTRUCTURE ONLY.  Like moe_oracle, only the test suite, the smoke check and the bench's
CPU-baseline leg may import it; it shares no code with the HIP kernels.

What it computes: the gradients of the sublayer output out = S(A) + R(A) of moe_oracle.moe_layer
(page "FarSkip-Collective", section 2.1: the modern MLP, the router G(A) = s(A W_R^T), Dispatch and
Combine, and the shared expert) with respect to the input A and every weight, given the gradient
dOut of a loss with respect to out.  The pages describe training with this layer (section 4.1:
the backward pass and its all-to-all overlap) but print no gradient formulas; the gradients here
are the chain rule applied to the forward definition, step by step in reverse order:
  Combine     out[t] = sum_i w[t,i] Y[dest_row[t,i]]      -> dY rows and dw
  gate        w = scores of the selected experts (renormalised or not)   -> dlogits
  router      logits = A W_R^T + b                          -> dA (router part), dW_R, db
  experts     U = X W1^T, G = X W2^T, H = U . SiLU(G), Y = H W3^T        -> dX, dW1, dW2, dW3
  Dispatch    X[r] = A[token of row r]                      -> dA[t] += sum over t's rows of dX
  shared      S = sum_s MLP_s(A)                            -> dA, dWs1, dWs2, dWs3
The selection of the top k experts is piecewise constant in the logits; as in any implementation,
no gradient flows through the choice itself, only through the selected experts' weights (reading
stated; exact wherever no two logits tie at the k-th place).

Arithmetic is float64.  An optional `store` rounding is applied where an implementation keeps an
intermediate in a narrower storage type (dY, the recomputed U and G, H, dH, dU and dG, dX, the
bf16 copy of dlogits feeding the router products, and the same for the shared expert); with
store=None everything is exact.

Pins (tests/test_oracle_backward_pins.py): central finite differences of moe_oracle.moe_layer in
float64 for every gradient separately (A, W_R, bias, W1, W2, W3, Ws1, Ws2, Ws3) over the gate
variants, plus closed forms (an expert without rows has zero weight gradients; one expert top-1
softmax passes no gradient to the router; dOut = 0 gives zero; linearity in dOut).  The stack's
backward (moe_stack_backward) is pinned by finite differences of moe_oracle.moe_stack for do_0 and
every layer's weights in all three modes and with mixed skip masks, and a one-layer stack equals
the layer plus the identity.
"""
from __future__ import annotations

import numpy as np

from . import moe_oracle as om

F64 = np.float64


def _f64(x):
    return np.asarray(x, dtype=F64)


def _st(x, store):
    return x if store is None else _f64(store(x))


def combine_backward(dOut, Y, topk_w, dest_row):
    """Combine: out[t] = sum_i w[t,i] Y[dest_row[t*k+i]].  Returns dY [N, d] (row dest_row[t*k+i]
    receives w[t,i] dOut[t]) and dw [T, k] (dw[t,i] = <dOut[t], Y[dest_row[t*k+i]]>)."""
    dOut, Y, w = _f64(dOut), _f64(Y), _f64(topk_w)
    T, k = w.shape
    dest = np.asarray(dest_row, dtype=np.int64).reshape(T, k)
    dY = np.zeros_like(Y)
    dw = np.zeros((T, k), dtype=F64)
    for i in range(k):
        dY[dest[:, i]] = w[:, i:i + 1] * dOut
        dw[:, i] = np.sum(dOut * Y[dest[:, i]], axis=1)
    return dY, dw


def gate_backward(logits, topk_idx, dw, gate, renormalize):
    """dlogits [T, E] from dw [T, k] through w = the selected experts' scores (moe_oracle.gate_weights).

    softmax over all E: p = softmax(L), d p_a / d L_j = p_a (delta_aj - p_j).
    sigmoid: p_j = 1 / (1 + e^-L_j), d p_j / d L_j = p_j (1 - p_j).
    renormalised: w_i = p_{e_i} / P with P = sum over the selected of p, so
        dL/dp_{e_i} = (dw_i - sum_m dw_m w_m) / P."""
    L = _f64(logits)
    idx = np.asarray(topk_idx, dtype=np.int64)
    dw = _f64(dw)
    T, E = L.shape
    p = om.gate_scores(L, gate)
    p_sel = np.take_along_axis(p, idx, axis=1)
    if renormalize:
        P = p_sel.sum(axis=1, keepdims=True)
        w = p_sel / P
        dp_sel = (dw - np.sum(dw * w, axis=1, keepdims=True)) / P
    else:
        dp_sel = dw
    dp = np.zeros((T, E), dtype=F64)                  # dLoss / dp_j, zero for experts not selected
    np.put_along_axis(dp, idx, dp_sel, axis=1)
    if gate == "softmax":
        return p * (dp - np.sum(dp * p, axis=1, keepdims=True))
    if gate == "sigmoid":
        return dp * p * (1.0 - p)
    raise ValueError(gate)


def router_backward(A, W_R, dlogits, store=None):
    """logits = A W_R^T + b.  Returns (dA_router [T, d], dW_R [E, d], dbias [E])."""
    A, W_R = _f64(A), _f64(W_R)
    dL = _st(_f64(dlogits), store)
    return dL @ W_R, dL.T @ A, _f64(dlogits).sum(axis=0)


def silu_grad(g):
    """d/dg of g * sigmoid(g) = sigmoid(g) (1 + g (1 - sigmoid(g)))."""
    g = _f64(g)
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def mlp_backward(X, W1, W2, W3, dY, store=None):
    """The modern MLP H = U . SiLU(G), U = X W1^T, G = X W2^T, Y = H W3^T.
    Returns (dX, dW1, dW2, dW3) for output gradient dY."""
    X, W1, W2, W3 = _f64(X), _f64(W1), _f64(W2), _f64(W3)
    dY = _st(_f64(dY), store)
    U = _st(X @ W1.T, store)
    G = _st(X @ W2.T, store)
    H = _st(U * om.silu(G), store)
    dH = _st(dY @ W3, store)
    dU = _st(dH * om.silu(G), store)
    dG = _st(dH * U * silu_grad(G), store)
    dX = _st(dU @ W1 + dG @ W2, store)
    return dX, dU.T @ X, dG.T @ X, dY.T @ H


def grouped_mlp_backward(X, offsets, W1, W2, W3, dY, store=None):
    """mlp_backward per expert over rows [offsets[e], offsets[e+1]); an expert without rows gets
    zero weight gradients.  W* index by expert.  Returns (dX [N, d], dW1 [E,c,d], dW2, dW3 [E,d,c])."""
    X, dY = _f64(X), _f64(dY)
    E = len(offsets) - 1
    c, d = np.asarray(W1[0]).shape
    dX = np.zeros_like(X)
    dW1 = np.zeros((E, c, d), dtype=F64)
    dW2 = np.zeros((E, c, d), dtype=F64)
    dW3 = np.zeros((E, d, c), dtype=F64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            dX[a:b], dW1[e], dW2[e], dW3[e] = mlp_backward(X[a:b], W1[e], W2[e], W3[e], dY[a:b], store)
    return dX, dW1, dW2, dW3


def unpermute_sum(dXp, dest_row, k):
    """Dispatch: X[r] = A[token of r], so dA[t] = sum over the slots i of dX[dest_row[t*k+i]]."""
    dXp = _f64(dXp)
    dest = np.asarray(dest_row, dtype=np.int64).reshape(-1, k)
    dA = np.zeros((dest.shape[0], dXp.shape[1]), dtype=F64)
    for i in range(k):
        dA += dXp[dest[:, i]]
    return dA


def shared_mlp_backward(A, Ws1, Ws2, Ws3, n_shared, c_shared, dS, store=None):
    """S = sum_s MLP_s(A) (moe_oracle.shared_mlp).  Returns (dA, dWs1, dWs2, dWs3)."""
    A = _f64(A)
    dA = np.zeros_like(A)
    dWs1 = np.zeros_like(_f64(Ws1))
    dWs2 = np.zeros_like(_f64(Ws2))
    dWs3 = np.zeros_like(_f64(Ws3))
    for s in range(n_shared):
        h = slice(s * c_shared, (s + 1) * c_shared)
        dXs, dWs1[h], dWs2[h], dWs3[:, h] = mlp_backward(A, _f64(Ws1)[h], _f64(Ws2)[h], _f64(Ws3)[:, h], dS, store)
        dA += dXs
    return dA, dWs1, dWs2, dWs3


def moe_layer_backward(A, W, k, gate, renormalize, dOut, n_shared=0, c_shared=0, store=None, fwd=None,
                       dOut_shared=None):
    """Gradients of out = S(A) + R(A) (moe_oracle.moe_layer) for output gradient dOut [T, d].

    W as for moe_layer.  fwd: optionally the forward's dict (moe_layer's return value; its Y then
    plays the saved expert outputs).  dOut_shared: the shared experts' own output gradient when it
    differs from the routed part's (in a FarSkip stack the shared output also feeds the next
    layer's input); default dOut.  Returns a dict with dA, dW_R, dbias, dW1, dW2, dW3 and, with
    shared experts, dWs1, dWs2, dWs3; also the intermediates dY, dw and dlogits."""
    A = _f64(A)
    if fwd is None:
        fwd = om.moe_layer(A, W, k, gate, renormalize, store=store)
    idx, w, dest = fwd["topk_idx"], fwd["topk_w"], fwd["dest_row"]
    dY, dw = combine_backward(dOut, fwd["Y"], w, dest)
    dlogits = gate_backward(fwd["logits"], idx, dw, gate, renormalize)
    dA_r, dW_R, dbias = router_backward(A, W["W_R"], dlogits, store)
    Xp = om.permute_rows(A, fwd["sorted_src"], k)
    dXp, dW1, dW2, dW3 = grouped_mlp_backward(Xp, fwd["offsets"], W["W1"], W["W2"], W["W3"], dY, store)
    dA = unpermute_sum(dXp, dest, k) + dA_r
    out = dict(dA=dA, dW_R=dW_R, dbias=dbias, dW1=dW1, dW2=dW2, dW3=dW3, dY=dY, dw=dw, dlogits=dlogits)
    if n_shared:
        dS = dOut if dOut_shared is None else dOut_shared
        dA_s, dWs1, dWs2, dWs3 = shared_mlp_backward(A, W["Ws1"], W["Ws2"], W["Ws3"], n_shared, c_shared, dS, store)
        out.update(dA=dA + dA_s, dWs1=dWs1, dWs2=dWs2, dWs3=dWs3)
    return out


# ---------------------------------------------------------------------------------------------
# The FarSkip stack (section 3): o_j = o_{j-1} + S_j(x_j) + R_j(x_j), x_1 = o_0, and the next
# input x_{j+1} = o_j (no skip), o_{j-1} + S_j(x_j) ("partial", 8b) or o_{j-1} ("outdated", 8a).
# Reverse mode through that graph: o_j feeds o_{j+1}, and x_{j+1} (no skip at layer j) or x_{j+2}
# (skip at layer j+1); S_j additionally feeds x_{j+1} under "partial".  The layer inputs' rounding
# to the activation dtype passes the gradient through unchanged (reading: the cast is treated as
# the identity, as any implementation that backpropagates through a storage cast does).
# ---------------------------------------------------------------------------------------------
def moe_stack_backward(o0, layer_weights, k, gate, renormalize, mode, dOL, mask=None, n_shared=0, c_shared=0,
                       round_inputs=None, store=None):
    """Gradients of o_L of moe_oracle.moe_stack for dOL = dLoss/do_L.  Returns a dict with do0 and
    layers (one moe_layer_backward dict per layer, in layer order)."""
    L = len(layer_weights)
    mask = [1] * L if mask is None else list(mask)
    record = []
    om.moe_stack(o0, layer_weights, k, gate, renormalize, mode, mask, n_shared, c_shared, round_inputs, record,
                 store)
    zero = np.zeros_like(_f64(o0))
    Go = [zero.copy() for _ in range(L + 1)]      # dLoss/do_j, j = 0 .. L
    Gx = [zero.copy() for _ in range(L + 2)]      # dLoss/dx_j, j = 1 .. L (+1 unused)
    Go[L] = _f64(dOL).copy()
    skip = [mode != "none" and bool(mask[j]) for j in range(L)]   # skip[j-1]: x_{j+1} bypasses o_j
    grads = [None] * L
    for j in range(L, 0, -1):
        W = layer_weights[j - 1]
        dS = Go[j] + (Gx[j + 1] if (mode == "partial" and skip[j - 1] and j < L) else 0.0)
        g = moe_layer_backward(record[j - 1][0], W, k, gate, renormalize, Go[j], n_shared, c_shared, store,
                               dOut_shared=dS)
        grads[j - 1] = g
        Gx[j] = g["dA"]
        Go[j - 1] += Go[j]
        if j == 1:
            Go[0] += Gx[1]
        elif not skip[j - 2]:
            Go[j - 1] += Gx[j]
        else:
            Go[j - 2] += Gx[j]
    return dict(do0=Go[0], layers=grads)
