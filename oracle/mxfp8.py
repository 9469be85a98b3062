"""MXFP8 numbers for the FP8 expert products, written plainly.

TEST INFRASTRUCTURE ONLY.  Like moe_oracle, this module is the correctness reference for the HIP
library; only the test suite, the smoke check and the bench's CPU-baseline leg may import it.  It
shares no code with the HIP kernels.

The pages state only that FarSkip's inference runs use FP8 quantisation together with fused MoE
forward kernels (FarSkip-Collective, papercache summary: the experimental setup, software
configuration, inference parameters); they name no format.
Reading taken (the format CDNA4's scaled matrix instructions execute natively): the OCP
microscaling format MXFP8 -- FP8 E4M3 elements, and one power-of-two E8M0 scale shared by each
block of 32 consecutive elements along the reduction dimension K.

- E4M3 (the "FN" variant): sign, 4 exponent bits (bias 7), 3 mantissa bits; subnormals at exponent
  field 0; no infinities; 0x7F / 0xFF are NaN; the largest finite magnitude is 448 (1.75 * 2^8).
- Encoding: the nearest E4M3 value, ties to the even code; magnitudes above 448 saturate to 448
  (reading: the saturating conversion); the sign of zero is kept.
- Block scale (reading): the smallest power of two 2^s with max |x| / 2^s <= 448, i.e.
  s = ceil(log2(max |x| / 448)), clamped to [-127, 127] and stored as the E8M0 byte s + 127; an
  all-zero block takes s = 0.  The elements are x / 2^s encoded as above, so the block maximum lands
  in (224, 448] and nothing saturates.  (The OCP specification's own example rule,
  floor(log2(max |x|)) - 8, puts the maximum in [256, 512) and clips block maxima with mantissas
  above 1.75 by up to 12.5%; the rule taken here trades that for one bit of headroom.)
- Decoding: e4m3(code) * 2^(scale - 127).

Parity pins: the four extreme E4M3 values of the format definition, every code's round trip, the
ties-to-even rule at midpoints, saturation, the scale rule on hand-made blocks, representable
blocks quantising exactly, and the per-element error bound 2^-4 (relative) of the normal range.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E8M0_BIAS = 127
BLOCK = 32


def e4m3_decode(codes):
    """E4M3 codes (uint8) -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    exp = (c >> 3) & 15
    man = c & 7
    mag = np.where(exp == 0, (man / 8.0) * 2.0 ** -6, (1.0 + man / 8.0) * 2.0 ** (exp - 7))
    val = np.where(sign == 1, -mag, mag)
    return np.where((exp == 15) & (man == 7), np.nan, val)


_POS = np.arange(0x7F, dtype=np.uint8)     # the non-negative finite codes, ascending in value
_POS_VALS = e4m3_decode(_POS)


def e4m3_encode(x):
    """Float values -> nearest E4M3 codes, ties to the even code, saturating at +-448.  Finite inputs."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.minimum(np.searchsorted(_POS_VALS, a, side="left"), 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALS[lo]
    d_hi = _POS_VALS[hi] - a
    code = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def block_exponent(amax):
    """Shared exponent s of a block whose largest magnitude is amax: the smallest integer with
    amax <= 448 * 2^s (E8M0 code s + 127); 0 for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    f, e = np.frexp(amax)          # amax = f * 2^e, f in [0.5, 1); 448 = 0.875 * 2^9
    s = np.where(amax > 0, e - 9 + (f > 0.875), 0)
    return np.clip(s, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def mx_quantize(X, block=BLOCK):
    """Rows of X [R, K] (K a multiple of block) -> (E4M3 codes uint8 [R, K], E8M0 scales uint8
    [R, K / block]); blocks are consecutive elements of a row."""
    X = np.asarray(X, dtype=np.float64)
    R, K = X.shape
    if K % block:
        raise ValueError("K must be a multiple of the block size")
    B = X.reshape(R, K // block, block)
    s = block_exponent(np.abs(B).max(axis=2))
    codes = e4m3_encode(B / np.exp2(s)[:, :, None]).reshape(R, K)
    return codes, (s + E8M0_BIAS).astype(np.uint8)


def mx_dequantize(codes, scales, block=BLOCK):
    codes = np.asarray(codes, dtype=np.uint8)
    R, K = codes.shape
    f = np.exp2(np.asarray(scales, dtype=np.float64) - E8M0_BIAS)
    return (e4m3_decode(codes).reshape(R, K // block, block) * f[:, :, None]).reshape(R, K)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu_hidden_mxfp8(X, W1q, W2q, hidden_store=None):
    """The first half of the expert MLP of section 2.1 with MXFP8 operands: H = (X W1^T) . SiLU(X W2^T)
    with X quantised along d and W1 / W2 given quantised ((codes, scales) pairs along d), the
    products and SiLU exact in float64; returns H quantised along c as (codes, scales).
    hidden_store (optional) rounds H to the precision an implementation forms it in before H is
    quantised (each H code is then decided in that precision)."""
    Xd = mx_dequantize(*mx_quantize(X))
    U = Xd @ mx_dequantize(*W1q).T
    G = Xd @ mx_dequantize(*W2q).T
    H = U * silu(G)
    if hidden_store is not None:
        H = hidden_store(H)
    return mx_quantize(H)


def mx_matmul(Aq, Bq):
    """A B^T exact in float64 for MXFP8 operands given as (codes, scales) pairs, both quantised
    along the shared dimension."""
    return mx_dequantize(*Aq) @ mx_dequantize(*Bq).T


def mlp_mxfp8(X, W1q, W2q, W3q, hidden_store=None):
    """The expert MLP of section 2.1 (H = (X W1^T) . SiLU(X W2^T), Y = H W3^T) with MXFP8 operands:
    H from swiglu_hidden_mxfp8 (quantised along c), then Y = mx_matmul(H, W3) (W3 given quantised
    along c)."""
    return mx_matmul(swiglu_hidden_mxfp8(X, W1q, W2q, hidden_store), W3q)


def grouped_mlp_mxfp8(X, offsets, W1q, W2q, W3q, hidden_store=None):
    """mlp_mxfp8 per group: rows [offsets[g], offsets[g+1]) use expert g's quantised weights
    (W*q[g] -> (codes, scales))."""
    X = np.asarray(X, dtype=np.float64)
    Y = np.zeros((X.shape[0], W3q[0][0].shape[0]) if len(W3q) else (X.shape[0], 0), dtype=np.float64)
    for g in range(len(offsets) - 1):
        a, b = int(offsets[g]), int(offsets[g + 1])
        if b > a:
            Y[a:b] = mlp_mxfp8(X[a:b], W1q[g], W2q[g], W3q[g], hidden_store)
    return Y
