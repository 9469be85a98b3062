"""CPU oracle: one MoE sublayer forward and the FarSkip-Collective residual stack, written plainly.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the HIP library.  Only the
test suite, the smoke check and the bench's CPU-baseline leg may import or call it; the product path
never does.  It shares no code with the HIP kernels and imports nothing from the product package.

Source of every step: the page "FarSkip-Collective: Unhobbling Blocking Communication in Mixture of
Experts Models" (papercache summary).  Its section 2.1 defines the modern MLP, the MoE layer sum,
the router G(A) = s(A W_R^T), Dispatch (a permutation of the token rows grouped by expert) and
Combine (aggregate and sum the routed expert outputs); its section 3 defines the residual stream
and the FarSkip inputs o*_k, "outdated" (8a) and "partial" (8b).

Arithmetic is float64 throughout.  Inputs given as float32 or bfloat16-valued float32 are upcast
exactly.  Where the pages leave a step open, the reading taken is stated at the function.  An
optional `store` rounding (off by default) can be applied to the intermediates an implementation
keeps in a narrower storage type (expert hidden, expert and shared outputs), and `round_inputs` to
the stack's layer inputs: a routing decision of a deep layer then sees inputs of the same precision
as the implementation's, so the decision is comparable; it changes no other arithmetic.

Pins (tests that tie this module to something other than itself): brute-force top-k enumeration,
brute-force stable permutation, hand-derived worked examples under tests/golden/, the closed forms
"E=1 top-1 equals the dense MLP", "top-k = E with softmax equals the full weighted sum", the stack
special cases (L=1, mode none, outdated L=2, zero routed W3) and linear-layer closed forms.  The
choice of weights that are not renormalised for softmax top-6 (DeepSeek-V2-Lite shape) and sigmoid
top-1 (Llama-4-Scout shape) is a reading of the workload descriptions: parity unpinned by the pages.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(x):
    return np.asarray(x, dtype=F64)


# ---------------------------------------------------------------------------------------------
# Step 1: router logits.  Section 2.1, MoE equation: G(A) = s(A W_R^T), a linear classifier
# followed by a sparse selection function s().  An optional per-expert bias is added to the
# logits (the skewed Qwen3-shaped workload perturbs the logits this way).
# ---------------------------------------------------------------------------------------------
def router_logits(A, W_R, bias=None):
    L = _f64(A) @ _f64(W_R).T
    if bias is not None:
        L = L + _f64(bias)[None, :]
    return L


# ---------------------------------------------------------------------------------------------
# Step 2: sparse selection s().  Reading: each token keeps the k experts with the largest logits;
# the order is descending logit and equal logits go to the lower expert index.  Selection is done
# on the logits themselves (softmax and sigmoid are monotone, so the same set is chosen).
# ---------------------------------------------------------------------------------------------
def select_topk(logits, k):
    """topk_idx [T,k] int32 in slot order (best first)."""
    logits = np.asarray(logits)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    # a stable sort of -logit keeps equal logits in increasing expert order
    order = np.argsort(-_f64(logits), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gate_scores(logits, gate):
    """Per-expert scores before selection: softmax over all E experts, or elementwise sigmoid."""
    L = _f64(logits)
    if gate == "softmax":
        m = L.max(axis=1, keepdims=True)
        e = np.exp(L - m)
        return e / e.sum(axis=1, keepdims=True)
    if gate == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-L))
    raise ValueError(gate)


def gate_weights(logits, topk_idx, gate, renormalize):
    """w[t,i] = score of the i-th selected expert; divided by the sum over the k selected ones when
    renormalising."""
    p = gate_scores(logits, gate)
    w = np.take_along_axis(p, np.asarray(topk_idx, dtype=np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def route(A, W_R, k, gate, renormalize, bias=None):
    L = router_logits(A, W_R, bias)
    idx = select_topk(L, k)
    return L, idx, gate_weights(L, idx, gate, renormalize)


# ---------------------------------------------------------------------------------------------
# Step 3: Dispatch permutation.  Section 2.1: tokens A[l,:] are grouped by the experts P_l chosen
# for them, by permuting A.  (The indicator R_i printed there is garbled; it is read as the
# B_i x T row selection of expert i's tokens.)  Every (token, slot) pair becomes one row; rows are
# ordered by expert, and inside an expert by flat slot f = t*k + i (a stable counting sort).
# ---------------------------------------------------------------------------------------------
def permute(topk_idx, E):
    """Returns (offsets [E+1], sorted_src [T*k], dest_row [T*k]) as int32.

    offsets[e] = first row of expert e; dest_row[f] = row of flat slot f; sorted_src[r] = the flat
    slot placed at row r (the inverse of dest_row)."""
    flat = np.asarray(topk_idx, dtype=np.int64).reshape(-1)
    n = flat.size
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    next_row = offsets[:-1].copy()
    dest_row = np.empty(n, dtype=np.int64)
    for f in range(n):
        e = flat[f]
        dest_row[f] = next_row[e]
        next_row[e] += 1
    sorted_src = np.empty(n, dtype=np.int64)
    sorted_src[dest_row] = np.arange(n)
    return offsets.astype(np.int32), sorted_src.astype(np.int32), dest_row.astype(np.int32)


def permute_rows(A, sorted_src, k):
    """A_perm[r] = A[token of slot sorted_src[r]]: a pure row copy (no arithmetic)."""
    A = np.asarray(A)
    return A[np.asarray(sorted_src, dtype=np.int64) // k]


# ---------------------------------------------------------------------------------------------
# Step 4: the modern MLP of section 2.1, MLP(A) = sigma(A W1^T . g(A W2^T)) W3^T with W1, W2 of
# shape c x d and W3 of shape d x c.  Readings: "." is the elementwise product (both factors are
# T x c); g = SiLU (x * sigmoid(x)) and sigma = identity (SwiGLU); W2 is the gated branch.
# ---------------------------------------------------------------------------------------------
def silu(x):
    x = _f64(x)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def mlp(X, W1, W2, W3, store=None):
    """store: optional rounding applied to the values an implementation keeps in its storage
    dtype (the hidden H and the output); None = exact."""
    X = _f64(X)
    U = X @ _f64(W1).T
    G = X @ _f64(W2).T
    H = U * silu(G)
    if store is not None:
        H = _f64(store(H))
    Y = H @ _f64(W3).T
    return Y if store is None else _f64(store(Y))


def grouped_mlp(X, offsets, W1, W2, W3, store=None):
    """Rows [offsets[e], offsets[e+1]) of X go through expert e's MLP.  W1, W2, W3 only need to
    support indexing by expert (W1[e] is expert e's c x d matrix)."""
    X = _f64(X)
    Y = np.zeros_like(X)  # the MLP maps width d back to width d
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            Y[a:b] = mlp(X[a:b], W1[e], W2[e], W3[e], store)
    return Y


def shared_mlp(A, Ws1, Ws2, Ws3, n_shared, c_shared, store=None):
    """Sum over the shared experts (each processes every token, section 2.1) with weight 1.  Shared
    expert s owns hidden rows [s*c_shared, (s+1)*c_shared) of Ws1/Ws2 and the same columns of Ws3."""
    A = _f64(A)
    S = np.zeros_like(A)
    for s in range(n_shared):
        h = slice(s * c_shared, (s + 1) * c_shared)
        H = (A @ _f64(Ws1[h]).T) * silu(A @ _f64(Ws2[h]).T)
        if store is not None:
            H = _f64(store(H))
        S += H @ _f64(Ws3[:, h]).T
    return S if store is None else _f64(store(S))


# ---------------------------------------------------------------------------------------------
# Step 5: Combine.  Section 2.1: the routed expert outputs are aggregated and summed back into
# token order.  out[t] = addend[t] + residual[t] + sum_i w[t,i] * Y[dest_row[t*k+i]], slot order.
# ---------------------------------------------------------------------------------------------
def combine(Y, topk_w, dest_row, addend=None, residual=None):
    Y = _f64(Y)
    w = _f64(topk_w)
    T, k = w.shape
    dest = np.asarray(dest_row, dtype=np.int64).reshape(T, k)
    out = np.zeros((T, Y.shape[1]), dtype=F64)
    if residual is not None:
        out += _f64(residual)
    if addend is not None:
        out += _f64(addend)
    for i in range(k):
        out += w[:, i:i + 1] * Y[dest[:, i]]
    return out


# ---------------------------------------------------------------------------------------------
# One MoE sublayer (section 2.1, MoE equation plus the shared expert): f(A) = S(A) + R(A) with
# R(A) = sum over selected experts of G(A)_j MLP_j(A).
# ---------------------------------------------------------------------------------------------
def moe_layer(A, W, k, gate, renormalize, n_shared=0, c_shared=0, store=None):
    """W: dict with W_R, bias, W1, W2, W3, Ws1, Ws2, Ws3 (numpy or None).  Returns a dict with the
    logits, topk_idx, topk_w, offsets, sorted_src, dest_row, Y, S (shared sum or zeros) and R."""
    A = _f64(A)
    E = np.asarray(W["W_R"]).shape[0]
    L, idx, w = route(A, W["W_R"], k, gate, renormalize, W.get("bias"))
    offsets, sorted_src, dest_row = permute(idx, E)
    Xp = permute_rows(A, sorted_src, k)
    Y = grouped_mlp(Xp, offsets, W["W1"], W["W2"], W["W3"], store)
    R = combine(Y, w, dest_row)
    if n_shared:
        S = shared_mlp(A, W["Ws1"], W["Ws2"], W["Ws3"], n_shared, c_shared, store)
    else:
        S = np.zeros_like(A)
    return dict(logits=L, topk_idx=idx, topk_w=w, offsets=offsets, sorted_src=sorted_src,
                dest_row=dest_row, Y=Y, S=S, R=R, out=S + R)


# ---------------------------------------------------------------------------------------------
# FarSkip stack.  Section 3: o_k = o_0 + f_1(o_0) + f_2(o*_1) + ... + f_k(o*_{k-1}), i.e.
# o_k = o_{k-1} + f_k(x_k) with x_1 = o_0 and x_{k+1} = o*_k, where
#   standard residual (no skip):  x_{k+1} = o_k
#   "outdated" (8a):              x_{k+1} = o_{k-1}
#   "partial"  (8b):              x_{k+1} = o_{k-1} + f*_k(x_k)
# and f*_k is the part of block k ready before its collective: here the shared expert S_k.
# f_k = S_k + R_k.  A per-layer mask turns the skip off for chosen layers (x_{k+1} = o_k there).
# ---------------------------------------------------------------------------------------------
def farskip_stack(o0, layers, mode, mask=None, round_inputs=None, record=None):
    """layers: list of (shared_fn, routed_fn), each mapping x [T,d] -> [T,d].
    mode: "none" | "partial" | "outdated".  mask: per-layer 0/1 (default: all 1).
    round_inputs: optional function applied to every layer input x_k (e.g. rounding to the
    workload's activation dtype).  record: optional list that receives (x_k, S_k, R_k, o_k)."""
    if mode not in ("none", "partial", "outdated"):
        raise ValueError(mode)
    n = len(layers)
    mask = [1] * n if mask is None else list(mask)
    o_prev = _f64(o0)
    x = o_prev
    for j, (shared_fn, routed_fn) in enumerate(layers):
        xin = x if round_inputs is None else _f64(round_inputs(x))
        S = _f64(shared_fn(xin))
        R = _f64(routed_fn(xin))
        o = o_prev + S + R
        if mode == "none" or not mask[j]:
            x_next = o
        elif mode == "partial":
            x_next = o_prev + S
        else:
            x_next = o_prev
        if record is not None:
            record.append((xin, S, R, o))
        o_prev, x = o, x_next
    return o_prev


def moe_stack(o0, layer_weights, k, gate, renormalize, mode, mask=None, n_shared=0, c_shared=0,
              round_inputs=None, record=None, store=None):
    """The FarSkip stack with MoE sublayers as the blocks f_k = S_k + R_k.  `store` as in mlp()."""
    layers = []
    for W in layer_weights:
        def shared_fn(x, W=W):
            if n_shared:
                return shared_mlp(x, W["Ws1"], W["Ws2"], W["Ws3"], n_shared, c_shared, store)
            return np.zeros_like(_f64(x))

        def routed_fn(x, W=W):
            return moe_layer(x, W, k, gate, renormalize, store=store)["R"]
        layers.append((shared_fn, routed_fn))
    return farskip_stack(o0, layers, mode, mask, round_inputs, record)


# ---------------------------------------------------------------------------------------------
# Section 3, the wiring of a model whose layers are an attention sub-block followed by an MoE
# sub-block (shared experts S_k and routed experts R_k).  The page gives the attention input as
# the "partial" activation of (8b), everything the residual holds after layer k-1 except that
# layer's routed-expert output,
#     attn-in_k = o_{k-2} + attn-out_{k-1} + shared-out_{k-1}        (attn-in_1 = o_0),
# and the MoE input as the "outdated" activation of (8a), the previous layer's full output, which
# lacks only layer k's own attention output,
#     mlp-in_k = o_{k-1} = attn-in_k + routed-out_{k-1}.
# Every sub-block output still enters the residual: o_k = o_{k-1} + attn-out_k + S_k + R_k, with
# S_k and R_k computed from mlp-in_k.  Mode "none" is the standard residual stream of section 3's
# first equation: attn-in_k = o_{k-1}, mlp-in_k = o_{k-1} + attn-out_k.  (The equation for mlp-in_k
# is missing from the page; its stated decomposition and the (8a) reading agree on o_{k-1}.)
# ---------------------------------------------------------------------------------------------
def attn_moe_stack(o0, layers, mode, round_inputs=None, record=None):
    """layers: list of (attn_fn, shared_fn, routed_fn), each mapping x [T,d] -> [T,d].
    mode: "farskip" (the wiring above) | "none".  round_inputs: optional function applied to every
    sub-block input (the implementation's activation dtype).  record: optional list that receives
    (attn_in, mlp_in, attn_out, S, R, o) per layer, the inputs as the sub-blocks saw them."""
    if mode not in ("farskip", "none"):
        raise ValueError(mode)
    rnd = (lambda x: x) if round_inputs is None else (lambda x: _f64(round_inputs(x)))
    o_prev = _f64(o0)
    partial = o_prev      # attn-in of the next layer: o_{k-1} without R_{k-1}
    for attn_fn, shared_fn, routed_fn in layers:
        a_in = rnd(partial if mode == "farskip" else o_prev)
        A = _f64(attn_fn(a_in))
        m_in = rnd(o_prev if mode == "farskip" else o_prev + A)
        S = _f64(shared_fn(m_in))
        R = _f64(routed_fn(m_in))
        o = o_prev + A + S + R
        partial = o_prev + A + S
        if record is not None:
            record.append((a_in, m_in, A, S, R, o))
        o_prev = o
    return o_prev


def attn_moe_layer_stack(o0, layer_weights, attn_weights, k, gate, renormalize, mode, n_shared=0, c_shared=0,
                         round_inputs=None, record=None, store=None):
    """attn_moe_stack with MoE sublayers (shared + routed experts, as moe_layer) and, standing in for
    each attention sub-block, a dense per-token SwiGLU block with its own weights: attn_weights[j] =
    (Wa1, Wa2 [c_a, d], Wa3 [d, c_a]) and attn-out = mlp(x, Wa1, Wa2, Wa3).  `store` as in mlp()."""
    layers = []
    for W, Wa in zip(layer_weights, attn_weights):
        def attn_fn(x, Wa=Wa):
            return mlp(x, Wa[0], Wa[1], Wa[2], store)

        def shared_fn(x, W=W):
            if n_shared:
                return shared_mlp(x, W["Ws1"], W["Ws2"], W["Ws3"], n_shared, c_shared, store)
            return np.zeros_like(_f64(x))

        def routed_fn(x, W=W):
            return moe_layer(x, W, k, gate, renormalize, store=store)["R"]
        layers.append((attn_fn, shared_fn, routed_fn))
    return attn_moe_stack(o0, layers, mode, round_inputs, record)


# ---------------------------------------------------------------------------------------------
# Precision helpers used by the comparisons.
# ---------------------------------------------------------------------------------------------
def round_to_bf16(x):
    """Round float32 values to the nearest bfloat16 (ties to even), returned as float32.  Finite
    inputs only."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def topk_gap(logits, k):
    """Per token: (k-th largest logit) - ((k+1)-th largest logit); +inf when k == E."""
    L = np.sort(_f64(logits), axis=1)[:, ::-1]
    if k >= L.shape[1]:
        return np.full(L.shape[0], np.inf)
    return L[:, k - 1] - L[:, k]
