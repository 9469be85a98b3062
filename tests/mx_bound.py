"""Parity bars of the MXFP8 grouped products (test infrastructure).

CDNA4's scaled fp8 matrix instruction does not form its 128-term dot products exactly.  Measured
on the device (operands of normal values and of uniformly random finite codes, single
instructions and chains of 16 and 56 into one fp32 accumulator), each instruction's result is
within 2^-10.7 of the power of two at or below max(largest |product|, |accumulator it adds to|),
and exact when all products share one binade.  The bars bound a product's error by
    instr_bound = sum over the 128-wide K chunks of E_INSTR * 2^floor(log2 max(max_k |a_k b_k|, |C|)),
C the exact partial sum before the chunk, with E_INSTR = 2^-9 (a margin of three).

Second product, Y = H W3^T in bf16, from given MXFP8 operands (check_down): element by element
    |Y - ref| <= 2^-8 |ref| + 1.01 instr_bound(H, W3);
2^-8 |ref| is Y's rounding to bf16 (half a unit in the last place is at most 2^-8 of the value).

First product, H = (X W1^T) . SiLU(X W2^T) quantised to MXFP8 (check_hidden): an implementation
forms H in fp32 from the instruction's sums U and G, so its H lies within
    dH = dU |SiLU(G)| + 1.1 |U| dG + 2^-20 |H|
of the exact H (dU, dG: instr_bound of the two products; 1.1 bounds |SiLU'|; 2^-20 covers the
fp32 SiLU and rounding).  Every dequantised H value must lie in the range that MXFP8 quantisation
reaches when each element of its block lies anywhere in [H - dH, H + dH]: where no rounding
midpoint or power-of-two scale boundary is in reach that range is the one value the oracle gives;
near one, either side is correct.  This worst-case reach grows with K (at d = 7168 it spans a
rounding midpoint for most elements), so a second bar is statistical: at most 1% of the values may
differ from the oracle's (measured: about 0.1%).

The fused call (both products, H kept in the workspace) must give the two calls' Y bit for bit.
"""
import numpy as np

import oracle

mx = oracle.mxfp8

E_INSTR = 2.0 ** -9


def instr_bound(A, B, rows_per_pass=64):
    """[R, N] bound on |(A B^T) as the chained instruction forms it - exact|, A [R, K], B [N, K]
    dequantised operands (see the module docstring)."""
    R, K = A.shape
    N = B.shape[0]
    out = np.zeros((R, N))
    Bf = np.abs(B).astype(np.float32)
    for r0 in range(0, R, rows_per_pass):
        Ar = A[r0:r0 + rows_per_pass]
        C = np.zeros((Ar.shape[0], N))
        for k0 in range(0, K, 128):
            a = np.abs(Ar[:, k0:k0 + 128]).astype(np.float32)
            m = (a[:, None, :] * Bf[None, :, k0:k0 + 128]).max(axis=2).astype(np.float64)
            top = np.maximum(m, np.abs(C))
            out[r0:r0 + rows_per_pass] += E_INSTR * np.where(top > 0, np.exp2(np.floor(np.log2(np.maximum(top, 1e-300)))), 0)
            C += Ar[:, k0:k0 + 128] @ B[:, k0:k0 + 128].T
    return out


def fp32_store(H):
    """H as an implementation that forms it in fp32 holds it before quantising."""
    return np.asarray(H, dtype=np.float32).astype(np.float64)


def hidden_reach(X, W1q, W2q):
    """Per H element [R, c]: the lowest and highest dequantised MXFP8 value an implementation's H
    can quantise to (see the module docstring)."""
    Xd = mx.mx_dequantize(*mx.mx_quantize(X))
    W1d, W2d = mx.mx_dequantize(*W1q), mx.mx_dequantize(*W2q)
    U, G = Xd @ W1d.T, Xd @ W2d.T
    H = fp32_store(U * mx.silu(G))
    dH = instr_bound(Xd, W1d) * np.abs(mx.silu(G)) + 1.1 * np.abs(U) * instr_bound(Xd, W2d) + 2.0 ** -20 * np.abs(H)
    R, C = H.shape
    B, D = H.reshape(R, C // 32, 32), dH.reshape(R, C // 32, 32)
    s_lo = mx.block_exponent(np.maximum(np.abs(B) - D, 0).max(axis=2))
    s_hi = mx.block_exponent((np.abs(B) + D).max(axis=2))
    lo, hi = np.full(B.shape, np.inf), np.full(B.shape, -np.inf)
    for ds in range(int((s_hi - s_lo).max()) + 1):      # quantisation is monotone for a fixed scale
        s = np.minimum(s_lo + ds, s_hi)[:, :, None]
        for V in (B - D, B + D):
            q = mx.e4m3_decode(mx.e4m3_encode(V / np.exp2(s))) * np.exp2(s)
            lo, hi = np.minimum(lo, q), np.maximum(hi, q)
    return lo.reshape(R, C), hi.reshape(R, C)


def check_hidden(Hq, Hs, X, W1q, W2q, what="", max_flip_frac=0.01):
    """H codes / scales of an implementation against the oracle's; returns the number of values
    that differ from the oracle's."""
    rq, rs = mx.swiglu_hidden_mxfp8(X, W1q, W2q, hidden_store=fp32_store)
    got, ref = mx.mx_dequantize(Hq, Hs), mx.mx_dequantize(rq, rs)
    lo, hi = hidden_reach(X, W1q, W2q)
    out = (got < lo) | (got > hi)
    assert not out.any(), (f"{what}: {int(out.sum())} H values outside their reach, e.g. row/col "
                           f"{np.argwhere(out)[0].tolist()} got {got[out][0]!r} ref {ref[out][0]!r}")
    flips = int((got != ref).sum())
    assert flips <= max_flip_frac * got.size, f"{what}: {flips} of {got.size} H values differ from the oracle's"
    return flips


def check_down(Y, Hq_pair, W3q, what=""):
    """Y (bf16 values as float) of the second product against the oracle's exact product."""
    ref = mx.mx_matmul(Hq_pair, W3q)
    bound = 2.0 ** -8 * np.abs(ref) + 1.01 * instr_bound(mx.mx_dequantize(*Hq_pair), mx.mx_dequantize(*W3q))
    err = np.abs(np.asarray(Y, dtype=np.float64) - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} Y elements past the bound, worst err/bound {(err / bound).max():.3f}"
    return float((err / bound).max())


def check_end_to_end(Y, X, W1q, W2q, W3q, what=""):
    """Y of the whole MLP against the oracle's: mean|err| <= 2^-8 mean|ref| (the per-element bars
    are those of check_hidden and check_down)."""
    ref = mx.mlp_mxfp8(X, W1q, W2q, W3q, hidden_store=fp32_store)
    err = np.abs(np.asarray(Y, dtype=np.float64) - ref)
    r = float(err.mean() / np.abs(ref).mean())
    assert r <= 2.0 ** -8, f"{what}: mean|err|/mean|ref| = {r:.3e}"
    return r
