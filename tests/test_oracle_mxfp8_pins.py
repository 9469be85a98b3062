"""Pins of the MXFP8 oracle (oracle/mxfp8.py) to the format's definition and to properties that do
not come from the oracle itself.  CPU only."""
import numpy as np
import pytest

import oracle

mx = oracle.mxfp8


def _finite_codes():
    return np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


def test_e4m3_extreme_values_of_the_format():
    # the format's defining values: largest normal, smallest normal, largest and smallest subnormal
    assert mx.e4m3_decode([0x7E])[0] == 448.0
    assert mx.e4m3_decode([0x08])[0] == 2.0 ** -6
    assert mx.e4m3_decode([0x07])[0] == 0.875 * 2.0 ** -6
    assert mx.e4m3_decode([0x01])[0] == 2.0 ** -9
    assert mx.e4m3_decode([0x38])[0] == 1.0
    assert np.isnan(mx.e4m3_decode([0x7F, 0xFF])).all()
    neg_zero = mx.e4m3_decode([0x80])[0]
    assert neg_zero == 0 and np.signbit(neg_zero)
    assert mx.e4m3_decode([0xFE])[0] == -448.0


def test_e4m3_value_set_structure():
    """126 distinct positive finite values, increasing with the code; 7 subnormals k * 2^-9; 8 values
    per binade [2^e, 2^(e+1)) for e = -6 .. 7 (spaced 2^(e-3)), and 256 .. 448 in the top one."""
    pos = mx.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0) and pos.size == 126
    np.testing.assert_array_equal(pos[:7], np.arange(1, 8) * 2.0 ** -9)
    for e in range(-6, 8):
        vals = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        np.testing.assert_array_equal(vals, 2.0 ** e + np.arange(8) * 2.0 ** (e - 3))
    np.testing.assert_array_equal(pos[pos >= 256], 256 + np.arange(7) * 32.0)
    # negative codes mirror the positive ones
    np.testing.assert_array_equal(mx.e4m3_decode(np.arange(0x81, 0xFF, dtype=np.uint8)), -pos)


def test_e4m3_round_trip_every_finite_code():
    c = _finite_codes()
    np.testing.assert_array_equal(mx.e4m3_encode(mx.e4m3_decode(c)), c)


def test_e4m3_ties_to_even_and_saturation():
    pos = mx.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    lo_codes = np.arange(0, 0x7E)
    want = np.where(lo_codes % 2 == 0, lo_codes, lo_codes + 1)
    np.testing.assert_array_equal(mx.e4m3_encode(mids), want)
    np.testing.assert_array_equal(mx.e4m3_encode(-mids), want | 0x80)
    # just past a midpoint goes to the nearer (upper) value
    np.testing.assert_array_equal(mx.e4m3_encode(np.nextafter(mids, np.inf)), lo_codes + 1)
    for x in (448.0, 460.0, 464.0, 479.9, 480.0, 512.0, 1e6, 3.0e38):
        assert mx.e4m3_encode(x) == 0x7E and mx.e4m3_encode(-x) == 0xFE
    assert mx.e4m3_encode(-1e-30) == 0x80 and mx.e4m3_encode(1e-30) == 0x00


def test_e4m3_encode_is_the_nearest_value_bruteforce():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(-470, 470, 4000), rng.choice([-1, 1], 4000) * 2.0 ** rng.uniform(-12, 9.2, 4000)])
    got = mx.e4m3_encode(x)
    codes = _finite_codes()
    vals = mx.e4m3_decode(codes)
    for xi, g in zip(x, got):
        xc = float(np.clip(xi, -448, 448))
        d = np.abs(vals - xc)
        best = codes[d == d.min()]
        best = best[np.signbit(mx.e4m3_decode(best)) == np.signbit(xi)] if best.size > 1 else best
        if best.size > 1:  # a tie between two neighbours: the even code
            best = best[best % 2 == 0]
        assert g == best[0], (xi, hex(g), [hex(b) for b in best])


def test_mx_block_scale_rule():
    X = np.zeros((1, 6 * 32))
    X[0, 0] = 1.0            # block 0: amax 1 -> s = -8 (1 * 2^8 = 256 <= 448 < 512)
    X[0, 32] = 448.0         # block 1: amax 448 -> s = 0
    X[0, 64] = -0.75         # block 2: amax 0.75 -> s = -9 (384)
    X[0, 96] = 1.9           # block 3: 1.9 * 2^8 = 486.4 > 448 -> s = -7 (243.2 -> 240)
    X[0, 128] = 449.0        # block 4: s = 1 (224.5 -> 224)
    codes, scales = mx.mx_quantize(X)   # block 5: all zero -> s = 0
    np.testing.assert_array_equal(scales[0], [127 - 8, 127, 127 - 9, 127 - 7, 128, 127])
    deq = mx.mx_dequantize(codes, scales)
    assert deq[0, 0] == 1.0 and deq[0, 32] == 448.0 and deq[0, 64] == -0.75
    assert deq[0, 96] == 240.0 / 128 and deq[0, 128] == 448.0
    assert np.all(codes[0, 160:] == 0)


def test_mx_representable_blocks_quantize_exactly():
    rng = np.random.default_rng(3)
    R, nb = 7, 6
    codes = rng.choice(_finite_codes(), size=(R, nb * 32))
    blocks = codes.reshape(R, nb, 32)
    blocks[:, :, 5] = rng.choice(np.arange(0x78, 0x7F), size=(R, nb))   # block max in [256, 448]
    blocks[:, :, :5] &= 0xF7   # other entries at most 240 ... (exponent field <= 14)
    blocks[:, :, 6:] &= 0xF7
    blocks[:, :, 9] = 0   # zero entries stay zero
    scales = rng.integers(60, 190, size=(R, nb)).astype(np.uint8)
    X = mx.mx_dequantize(codes, scales)
    c2, s2 = mx.mx_quantize(X)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(mx.e4m3_decode(c2), mx.e4m3_decode(codes))


def test_mx_elementwise_error_bound_across_scales():
    """Blocks of very different magnitudes: every element keeps its block's precision (relative
    error <= 2^-4 above the subnormal range, absolute <= 2^(s-10) within it), nothing saturates and
    each block maximum lands in (224, 448] * 2^s, so the blocks are rows' runs of 32 consecutive
    elements."""
    rng = np.random.default_rng(11)
    R, nb = 16, 8
    X = rng.standard_normal((R, nb * 32)) * np.repeat(2.0 ** rng.integers(-30, 30, size=(R, nb)), 32, axis=1)
    codes, scales = mx.mx_quantize(X)
    D = mx.mx_dequantize(codes, scales)
    s = np.repeat(scales.astype(np.int64) - 127, 32, axis=1)
    y = np.abs(X) / 2.0 ** s
    normal = (y >= 2.0 ** -6) & (y <= 448)
    assert np.all(np.abs(D - X)[normal] <= 2.0 ** -4 * np.abs(X)[normal])
    sub = y < 2.0 ** -6
    assert np.all(np.abs(D - X)[sub] <= 2.0 ** (s[sub] - 10))
    assert np.all(y <= 448)
    ymax = y.reshape(R, nb, 32).max(axis=2)
    assert np.all((ymax > 224) & (ymax <= 448))


def test_mlp_mxfp8_equals_the_mlp_on_representable_operands():
    """With X, W1, W2, W3 MX-representable and G >= 64 (SiLU(G) = G in float64), H = U * G is a
    power-of-two multiple of representable values, so no quantisation changes anything and the
    MXFP8 MLP equals the plain MLP of the page on the same numbers."""
    rng = np.random.default_rng(5)
    d, c, n = 64, 64, 5
    X = np.zeros((n, d))
    X[np.arange(n), rng.integers(0, d, n)] = 1.0
    def rep(shape):
        v = mx.e4m3_decode(rng.choice(np.arange(0x30, 0x40), size=shape))   # 0.5 .. 1.875
        return v * rng.choice([-1, 1], size=shape)
    W1 = rep((c, d))
    W2 = np.full((c, d), 64.0)
    W3 = rep((d, c))
    q = lambda W: mx.mx_quantize(W)
    got = mx.mlp_mxfp8(X, q(W1), q(W2), q(W3))
    np.testing.assert_array_equal(got, oracle.mlp(X, W1, W2, W3))


def test_mlp_mxfp8_close_to_the_bf16_mlp():
    """Three quantisations of 3-bit mantissas (X, the weights, H): a few percent of the output scale,
    far below what a mistake in the block layout or the scale exponent gives."""
    rng = np.random.default_rng(9)
    d, c = 256, 128
    X = rng.standard_normal((40, d))
    W1, W2 = rng.standard_normal((c, d)) / 16, rng.standard_normal((c, d)) / 16
    W3 = rng.standard_normal((d, c)) / 11
    q = lambda W: mx.mx_quantize(W)
    ref = oracle.mlp(X, W1, W2, W3)
    got = mx.mlp_mxfp8(X, q(W1), q(W2), q(W3))
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 0.12


@pytest.mark.parametrize("sizes", [[3, 0, 5], [0, 0, 1], [8]])
def test_grouped_mlp_mxfp8_is_per_group(sizes):
    rng = np.random.default_rng(sum(sizes))
    d, c, G = 64, 32, len(sizes)
    N = sum(sizes)
    X = rng.standard_normal((N, d))
    Wq = [[mx.mx_quantize(rng.standard_normal(sh)) for _ in range(G)] for sh in ((c, d), (c, d), (d, c))]
    off = np.concatenate([[0], np.cumsum(sizes)])
    Y = mx.grouped_mlp_mxfp8(X, off, *Wq)
    for g in range(G):
        a, b = off[g], off[g + 1]
        if b > a:
            np.testing.assert_array_equal(Y[a:b], mx.mlp_mxfp8(X[a:b], Wq[0][g], Wq[1][g], Wq[2][g]))


def test_mlp_mxfp8_hand_example_quantises_the_hidden():
    """Worked by hand: X = [1, 1, 0 ...]; every row of W1 is [1, 1/16, 0 ...] (U = 1.0625), of W2
    [64, 64, 0 ...] (G = 128, SiLU(G) = 128 in float64), so every H entry is 136.  The H block has
    max 136: s = ceil(log2(136 / 448)) = -1 and 136 * 2 = 272 lies halfway between the E4M3 values
    256 and 288: ties to the even code give 256, i.e. H = 128.  W3 = I returns H itself."""
    d = c = 32
    X = np.zeros((1, d))
    X[0, :2] = 1.0
    W1 = np.zeros((c, d))
    W1[:, 0], W1[:, 1] = 1.0, 1.0 / 16
    W2 = np.zeros((c, d))
    W2[:, :2] = 64.0
    W3 = np.eye(d, c)
    q = lambda W: mx.mx_quantize(W)
    Y = mx.mlp_mxfp8(X, q(W1), q(W2), q(W3))
    np.testing.assert_array_equal(Y, np.full((1, d), 128.0))
