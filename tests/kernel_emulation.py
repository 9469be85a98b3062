"""A CPU emulation of the kernels' arithmetic, for deriving bars and margins (test infrastructure).

Products: an fp32 running sum over 32-wide K steps of exact bf16 products (the bf16 MFMA's K per
instruction); the expert hidden H and the outputs Y, S stored as bf16; router logits summed the same
way in fp32, plus the bias in fp32; the combine summed in fp32 in slot order.  Selection and gate
weights come from the oracle applied to the fp32 logits, so the emulation differs from the oracle
only in where it rounds.
"""
import numpy as np

import oracle

rnd = oracle.round_to_bf16


def bf(x):
    return rnd(np.asarray(x, np.float32)).astype(np.float32)


def acc32(X, W, step=32):
    """X [n, K] @ W[m, K]^T as an fp32 running sum of 32-wide K steps (each step's products are
    exact in fp32 for bf16 operands)."""
    out = np.zeros((X.shape[0], W.shape[0]), np.float32)
    for k0 in range(0, X.shape[1], step):
        part = X[:, k0:k0 + step].astype(np.float64) @ W[:, k0:k0 + step].astype(np.float64).T
        out = (out + part.astype(np.float32)).astype(np.float32)
    return out


def emulated_mlp(X, W1, W2, W3):
    """The SwiGLU expert MLP as the kernels compute it; returns float64 values of the bf16 output."""
    X = np.asarray(X, np.float32)
    U, G = acc32(X, W1), acc32(X, W2)
    H = bf(U * (G / (np.float32(1) + np.exp(-G).astype(np.float32))))
    return bf(acc32(H, W3)).astype(np.float64)


def emulated_logits(x, W_R, bias=None):
    L = acc32(np.asarray(x, np.float32), W_R)
    if bias is not None:
        L = (L + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    return L


def emulated_layer_fns(W, k, gate, renormalize):
    """(shared_fn, routed_fn) of one MoE sublayer for oracle.farskip_stack, with float32 weights W
    (W_R, bias, W1-W3 per expert, Ws1-Ws3 for one shared expert or None)."""
    def shared(x):
        if W.get("Ws1") is None:
            return np.zeros(np.shape(x))
        return emulated_mlp(x, W["Ws1"], W["Ws2"], W["Ws3"])

    def routed(x):
        x = np.asarray(x, np.float32)
        L = emulated_logits(x, W["W_R"], W.get("bias")).astype(np.float64)
        idx = oracle.select_topk(L, k)
        w = oracle.gate_weights(L, idx, gate, renormalize).astype(np.float32)
        out = np.zeros(x.shape, np.float32)
        for i in range(k):
            Y = np.zeros(x.shape, np.float32)
            for e in np.unique(idx[:, i]):
                rows = idx[:, i] == e
                Y[rows] = emulated_mlp(x[rows], W["W1"][e], W["W2"][e], W["W3"][e])
            out = (out + w[:, i:i + 1] * Y).astype(np.float32)
        return out.astype(np.float64)

    return shared, routed
