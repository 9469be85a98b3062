"""The MXFP8 parity bars (tests/mx_bound.py) on the CPU: emulated fp32 implementations whose
matrix instruction errs at the measured level pass them, and emulations with planted mistakes
(rounding rule, block exponent, a scale taken from the wrong block, a dropped SiLU, a shifted row,
bf16 truncation) fail them."""
import numpy as np
import pytest

import oracle
from tests.mx_bound import check_down, check_end_to_end, check_hidden, instr_bound

mx = oracle.mxfp8
POS = mx.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
CHAIN_ERR = 5e-6   # a chain error of the instruction's size, relative to the sum of |products|


def block_scaled(rng, shape, std, spread):
    x = rng.standard_normal(shape) * std
    j = rng.integers(-spread, spread + 1, shape[:-1] + (shape[-1] // 32, 1))
    return (x.reshape(shape[:-1] + (shape[-1] // 32, 32)) * np.exp2(j)).reshape(shape)


def bf16(x, truncate=False):
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    if not truncate:
        b = b + 0x7FFF + ((b >> 16) & 1)
    return ((b >> 16) << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def quantize(V, mistake=None):
    """(codes, scales) of the rows of V, written independently of the oracle's encoder."""
    R, C = V.shape
    B = V.reshape(R, C // 32, 32)
    amax = np.abs(B).max(axis=2)
    f, e = np.frexp(amax)
    s = np.where(amax > 0, e - 9 + (f > 0.875), 0)
    if mistake == "exp+1":
        s = s + 1
    Y = np.abs(B) / np.exp2(s)[:, :, None]
    if mistake == "truncate":
        idx = np.searchsorted(POS, Y, side="right") - 1
    else:
        hi = np.minimum(np.searchsorted(POS, Y), len(POS) - 1)
        lo = np.maximum(hi - 1, 0)
        dlo, dhi = Y - POS[lo], POS[hi] - Y
        idx = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    codes = (idx | np.where(np.signbit(B), 0x80, 0)).astype(np.uint8).reshape(R, C)
    return codes, (s + 127).astype(np.uint8)


def deq(q):
    return mx.mx_dequantize(*q)


def noisy(rng, A, B, err):
    return A @ B.T + err * rng.uniform(-1, 1, (A.shape[0], B.shape[0])) * (np.abs(A) @ np.abs(B).T)


def emulate_hidden(X, W1q, W2q, rng, err=CHAIN_ERR, mistake=None):
    Xd = deq(quantize(X))
    if mistake == "shifted_row":
        Xd = np.roll(Xd, 1, axis=0)
    W1d = deq(W1q)
    if mistake == "scale_block":
        W1d = W1d.copy()
        W1d[:, 32:64] *= 2.0
    U, G = noisy(rng, Xd, W1d, err), noisy(rng, Xd, deq(W2q), err)
    H = U * G if mistake == "no_silu" else U * (G / (1.0 + np.exp(-G)))
    return quantize(np.asarray(H, dtype=np.float32).astype(np.float64), mistake)


def emulate_down(Hq, W3q, rng, err=CHAIN_ERR, mistake=None):
    W3d = deq(W3q)
    if mistake == "scale_block":
        W3d = W3d.copy()
        W3d[:, 32:64] *= 2.0
    return bf16(noisy(rng, deq(Hq), W3d, err), truncate=(mistake == "bf16_truncate"))


def case(seed, N=48, d=256, c=256):
    rng = np.random.default_rng(seed)
    X = bf16(block_scaled(rng, (N, d), 1.0, 3))
    W1q = mx.mx_quantize(bf16(block_scaled(rng, (c, d), d ** -0.5, 2)))
    W2q = mx.mx_quantize(bf16(block_scaled(rng, (c, d), d ** -0.5, 2)))
    W3q = mx.mx_quantize(bf16(block_scaled(rng, (d, c), c ** -0.5, 2)))
    return rng, X, W1q, W2q, W3q


def test_independent_quantizer_agrees_with_the_oracle():
    rng, X, *_ = case(5)
    q = quantize(X)
    ref = mx.mx_quantize(X)
    np.testing.assert_array_equal(q[0], ref[0])
    np.testing.assert_array_equal(q[1], ref[1])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bars_accept_an_implementation_within_the_instruction_error(seed):
    rng, X, W1q, W2q, W3q = case(seed)
    Hq = emulate_hidden(X, W1q, W2q, rng)
    flips = check_hidden(*Hq, X, W1q, W2q, f"seed {seed}")
    assert flips < 0.01 * Hq[0].size
    Y = emulate_down(Hq, W3q, rng)
    check_down(Y, Hq, W3q, f"seed {seed}")
    check_end_to_end(Y, X, W1q, W2q, W3q, f"seed {seed}")


def test_hidden_reach_covers_errors_at_the_instruction_bound():
    """Products that err by the full instr_bound (either sign) still quantise within reach,
    although they move many more codes."""
    rng, X, W1q, W2q, _ = case(7)
    Xd, W1d, W2d = deq(quantize(X)), deq(W1q), deq(W2q)
    U = Xd @ W1d.T + rng.choice([-1.0, 1.0], (X.shape[0], W1d.shape[0])) * instr_bound(Xd, W1d)
    G = Xd @ W2d.T + rng.choice([-1.0, 1.0], (X.shape[0], W2d.shape[0])) * instr_bound(Xd, W2d)
    Hq = quantize(np.asarray(U * (G / (1.0 + np.exp(-G))), dtype=np.float32).astype(np.float64))
    check_hidden(*Hq, X, W1q, W2q, "errors at the bound", max_flip_frac=1.0)


def test_down_bar_covers_errors_at_the_instruction_bound():
    rng, X, W1q, W2q, W3q = case(8)
    Hq = emulate_hidden(X, W1q, W2q, rng)
    Hd, W3d = deq(Hq), deq(W3q)
    Y = bf16(Hd @ W3d.T + 0.99 * rng.choice([-1.0, 1.0], (X.shape[0], W3d.shape[0])) * instr_bound(Hd, W3d))
    check_down(Y, Hq, W3q, "errors at the bound")


def test_exact_implementation_matches_codes():
    rng, X, W1q, W2q, _ = case(3)
    Hq = emulate_hidden(X, W1q, W2q, rng, err=0.0)
    assert check_hidden(*Hq, X, W1q, W2q, "exact") <= 2


@pytest.mark.parametrize("mistake", ["truncate", "exp+1", "scale_block", "no_silu", "shifted_row"])
def test_hidden_bar_rejects_planted_mistakes(mistake):
    rng, X, W1q, W2q, _ = case(11)
    Hq = emulate_hidden(X, W1q, W2q, rng, mistake=mistake)
    with pytest.raises(AssertionError):
        check_hidden(*Hq, X, W1q, W2q, mistake)


@pytest.mark.parametrize("mistake", ["scale_block", "bf16_truncate"])
def test_down_bar_rejects_planted_mistakes(mistake):
    rng, X, W1q, W2q, W3q = case(12)
    Hq = emulate_hidden(X, W1q, W2q, rng)
    Y = emulate_down(Hq, W3q, rng, mistake=mistake)
    with pytest.raises(AssertionError):
        check_down(Y, Hq, W3q, mistake)
