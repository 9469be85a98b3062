"""The element-wise bar against the store-mirrored oracle (tests/helpers.py: assert_mirror,
mirror_bound, combine_bound), checked on the CPU before any GPU comparison relies on it.

An emulation of the kernels' arithmetic (each output an fp32 running sum over 32-wide K steps of
exact bf16 products, the hidden H and the output Y stored as bf16, the combine summed in fp32) must
pass it; plausible mistakes must fail it: a 1% error confined to one 16 x 16 output tile, a tile
computed with another expert's weights, a combine that swaps two slots' gate weights, and a
combine that drops the shared-expert term.
"""
import numpy as np
import pytest

import oracle
from tests.helpers import assert_mirror, bf16_ulp, combine_bound, mirror_bound
from tests.kernel_emulation import bf, emulated_mlp

rnd = oracle.round_to_bf16


def weights(rng, d, c, std=0.02):
    return (bf(rng.standard_normal((c, d)) * std), bf(rng.standard_normal((c, d)) * std),
            bf(rng.standard_normal((d, c)) * std))


@pytest.mark.parametrize("seed,n,d,c", [(1, 32, 1024, 512), (2, 48, 2048, 256), (3, 16, 512, 1024)])
def test_emulated_kernel_arithmetic_passes(seed, n, d, c):
    rng = np.random.default_rng(seed)
    X = bf(rng.standard_normal((n, d)))
    W1, W2, W3 = weights(rng, d, c)
    Y = emulated_mlp(X, W1, W2, W3)
    ref = oracle.mlp(X, W1, W2, W3, store=rnd)
    assert np.any(Y != ref)          # the emulation really differs from the mirror somewhere
    assert assert_mirror(Y, ref, "emulated") <= 0.9


def test_one_percent_error_on_one_tile_fails():
    rng = np.random.default_rng(4)
    X = bf(rng.standard_normal((32, 1024)))
    W1, W2, W3 = weights(rng, 1024, 512)
    Y = emulated_mlp(X, W1, W2, W3)
    ref = oracle.mlp(X, W1, W2, W3, store=rnd)
    Y[16:32, 32:48] *= 1.01
    with pytest.raises(AssertionError):
        assert_mirror(Y, ref, "planted 1% tile error")


def test_tile_with_another_experts_weights_fails():
    rng = np.random.default_rng(5)
    X = bf(rng.standard_normal((32, 512)))
    Wa, Wb = weights(rng, 512, 256), weights(rng, 512, 256)
    Y = emulated_mlp(X, *Wa)
    Y[:16] = emulated_mlp(X[:16], *Wb)   # one 16-row tile given expert b's weights
    ref = oracle.mlp(X, *Wa, store=rnd)
    with pytest.raises(AssertionError):
        assert_mirror(Y, ref, "planted wrong expert")


def test_bf16_ulp_values():
    np.testing.assert_array_equal(bf16_ulp([1.0, 1.99, 2.0, 0.5, -3.0]),
                                  [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -8, 2.0 ** -6])
    # consecutive bf16 values differ by exactly one unit
    for v in (1.3, -0.07, 300.0):
        r = rnd(np.array([v], np.float32))
        nxt = (r.view(np.uint32) + np.uint32(1 << 16)).view(np.float32)
        assert abs(float(nxt[0]) - float(r[0])) == bf16_ulp(r[0])
    m = mirror_bound(np.array([1.0, 0.0]))
    assert m[1] > 0 and m[0] > bf16_ulp(1.0)


def _layer(rng, T=24, d=512, c=256, E=4, k=2, shared=True):
    A = bf(rng.standard_normal((T, d)))
    W = {"W_R": bf(rng.standard_normal((E, d)) * 0.05), "bias": None}
    Ws = [weights(rng, d, c) for _ in range(E)]
    W["W1"] = [w[0] for w in Ws]
    W["W2"] = [w[1] for w in Ws]
    W["W3"] = [w[2] for w in Ws]
    W["Ws1"], W["Ws2"], W["Ws3"] = weights(rng, d, c) if shared else (None, None, None)
    return A, W


def _emulated_layer(A, W, k, ref, swap_w=False, drop_shared=False):
    """The GPU's layer output from the oracle's own routing, with emulated expert products and an
    fp32 combine of the bf16 Y and S."""
    T = A.shape[0]
    off, src = ref["offsets"], ref["sorted_src"]
    Xp = oracle.permute_rows(A, src, k)
    Y = np.zeros_like(ref["Y"])
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            Y[a:b] = emulated_mlp(Xp[a:b], W["W1"][e], W["W2"][e], W["W3"][e])
    S = emulated_mlp(A, W["Ws1"], W["Ws2"], W["Ws3"])
    w = ref["topk_w"].astype(np.float32)
    if swap_w:
        w = w[:, ::-1].copy()
    dest = ref["dest_row"].reshape(T, k)
    out = (np.zeros_like(S) if drop_shared else S).astype(np.float32)
    for i in range(k):
        out = (out + w[:, i:i + 1] * Y[dest[:, i]].astype(np.float32)).astype(np.float32)
    return out.astype(np.float64)


@pytest.mark.parametrize("planted", [None, "swap_w", "drop_shared"])
def test_combine_bound(planted):
    rng = np.random.default_rng(6)
    k = 2
    A, W = _layer(rng, k=k)
    ref = oracle.moe_layer(A, W, k, "softmax", True, n_shared=1, c_shared=256, store=rnd)
    got = _emulated_layer(A, W, k, ref, swap_w=planted == "swap_w", drop_shared=planted == "drop_shared")
    bound = combine_bound(ref["S"], ref["Y"], ref["topk_w"], ref["dest_row"].reshape(A.shape[0], k))
    if planted is None:
        assert assert_mirror(got, ref["out"], "emulated layer", bound=bound) <= 0.9
    else:
        with pytest.raises(AssertionError):
            assert_mirror(got, ref["out"], f"planted {planted}", bound=bound)
