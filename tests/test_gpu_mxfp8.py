"""GPU parity of the MXFP8 expert products against the MXFP8 oracle (oracle/mxfp8.py).

Bars:
- quantisation (codes and scales): bit-exact.  Every decision is taken from the bf16 input scaled
  by a power of two, which is exact in fp32 and in fp64 alike, so both sides see the same numbers.
- the two grouped products, each through its own call, to the bars of tests/mx_bound.py: H's
  codes identical to the oracle's except where the scaled fp8 instruction's measured accumulation
  error can carry H across a rounding decision (at most 1% of them); Y of the second product,
  from MXFP8 operands made by the test, element by element within its bf16 rounding and the
  instruction's error; the fused call equal, bit for bit, to the two calls; the whole MLP's mean
  error at most 2^-8 of the mean |Y|.
The oracle takes the weights quantised by oracle.mxfp8 from the same bf16 values; the tests also
check that the library's quantisation of those weights is bit-identical to the oracle's.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.helpers import report, to_np
from tests.mx_bound import E_INSTR, check_down, check_end_to_end, check_hidden, instr_bound

pytestmark = pytest.mark.gpu

DEV = "cuda"
mx = oracle.mxfp8


@pytest.fixture(scope="module")
def ops():
    from mixture_experts_layer_sum_amd import ops as _ops
    return _ops


def _sync():
    torch.cuda.synchronize()


# =================================================================================================
# quantisation
# =================================================================================================
def run_quantize(ops, X):
    codes = torch.full(X.shape, 0x5A, dtype=torch.uint8, device=DEV)
    scales = torch.full(X.shape[:-1] + (X.shape[-1] // 32,), 0x5A, dtype=torch.uint8, device=DEV)
    ops.moe_mx_quantize(X, codes, scales)
    _sync()
    return codes.cpu().numpy(), scales.cpu().numpy()


def check_quantize(ops, X):
    codes, scales = run_quantize(ops, X)
    ref_codes, ref_scales = mx.mx_quantize(to_np(X).astype(np.float64))
    np.testing.assert_array_equal(scales, ref_scales)
    np.testing.assert_array_equal(codes, ref_codes)
    return codes, scales


@pytest.mark.parametrize("R,K,spread", [(1, 32, 0), (37, 96, 4), (1000, 512, 12), (64, 7168, 30)])
def test_mx_quantize_bitexact_random(ops, R, K, spread):
    X = mi.block_scaled_normal((R, K), 1.0, mi.seed_for(93, R, K, spread), DEV, torch.bfloat16, spread=spread)
    check_quantize(ops, X)


def _special_rows():
    """Hand-made 32-element blocks: zeros of both signs, every E4M3 value, midpoints (ties), the
    subnormal range, a block maximum exactly at and just past 448 * 2^s, and bf16 extremes."""
    pos = mx.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2                        # 4 significant bits: exact in bf16
    rows = []
    rows.append(np.zeros(32))
    rows.append(np.full(32, -0.0))
    vals = np.concatenate([pos, -pos[1:]])                 # 253 values, 31 to a block + the maximum 448
    vals = np.concatenate([vals, np.zeros(9 * 31 - vals.size)]).reshape(9, 31)
    rows.extend(np.concatenate([vals, np.full((9, 1), 448.0)], axis=1))   # every value, s = 0
    m = np.concatenate([mids, -mids[:2]])                   # 126 + 2 = 128 midpoints of both signs
    for blk in m.reshape(4, 32):
        b = blk.copy()
        b[0] = 448.0                                        # keeps s = 0 so the midpoints stay midpoints
        rows.append(b)
        rows.append(b * 2.0 ** 5)                           # the same decisions at s = 5
        rows.append(b * 2.0 ** -20)                         # ... and at s = -20
    sub = np.arange(32) / 1024.0                            # 0 .. 31/1024: subnormal codes and midpoints
    sub[31] = 448.0
    rows.append(sub)
    rows.append(-sub)
    for amax in (448.0, 452.0, 480.0, 512.0, 896.0, 1.0, 0.875, 0.9375, 2.0 ** -30, 3.0e38):
        b = np.linspace(-1, 1, 32) * amax
        b[7] = amax
        rows.append(b)
    tiny = np.zeros(32)
    tiny[3] = 2.0 ** -133                                   # the smallest bf16 subnormal: s clamps to -127
    tiny[5] = -(2.0 ** -130)
    rows.append(tiny)
    big = np.full(32, 2.0 ** -100)
    big[0] = 3.3895313892515355e38                          # the largest bf16 value: tiny neighbours vanish
    rows.append(big)
    return np.stack(rows)


def test_mx_quantize_special_values(ops):
    S = _special_rows()
    X = torch.from_numpy(S).to(torch.float32).to(torch.bfloat16)
    Xn = to_np(X).astype(np.float64)
    n_exact = 2 + 9 + 12 + 2                                # rows built from values exact in bf16
    assert np.array_equal(Xn[:n_exact], S[:n_exact]), "hand-made values must be exact in bf16"
    codes, scales = check_quantize(ops, X.to(DEV))
    # the format's fixed points: blocks of exact E4M3 values with maximum 448 keep their codes
    np.testing.assert_array_equal(scales[2:11], 127)
    np.testing.assert_array_equal(mx.e4m3_decode(codes[2:11]).ravel(), S[2:11].ravel())
    assert (codes[1] == 0x80).all() and (codes[0] == 0).all() and (scales[:2] == 127).all()


def test_mx_quantize_empty_and_3d(ops):
    codes, scales = run_quantize(ops, torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    assert codes.shape == (0, 64) and scales.shape == (0, 2)
    X = mi.block_scaled_normal((3, 5, 64), 1.0, 7, DEV, torch.bfloat16)
    codes, scales = run_quantize(ops, X)
    ref_codes, ref_scales = mx.mx_quantize(to_np(X).reshape(15, 64).astype(np.float64))
    np.testing.assert_array_equal(codes.reshape(15, 64), ref_codes)
    np.testing.assert_array_equal(scales.reshape(15, 2), ref_scales)


# =================================================================================================
# grouped MXFP8 SwiGLU products
# =================================================================================================
def oracle_stack(W, gq=None):
    """Per-group oracle quantisation of [G, r, K] bf16 device weights; with gq (the library's
    quantisation of W) it also checks the two are bit-identical."""
    out = []
    for g in range(W.shape[0]):
        q = mx.mx_quantize(to_np(W[g]).astype(np.float64))
        if gq is not None:
            np.testing.assert_array_equal(gq[0][g].cpu().numpy(), q[0])
            np.testing.assert_array_equal(gq[1][g].cpu().numpy(), q[1])
        out.append(q)
    return out


def offsets_of(sizes):
    off = np.zeros(len(sizes) + 1, dtype=np.int32)
    off[1:] = np.cumsum(np.asarray(sizes, dtype=np.int64))
    return off


def make_weights(G, d, c, seed):
    W1 = mi.block_scaled_normal((G, c, d), d ** -0.5, seed + 2, DEV, spread=2)
    W2 = mi.block_scaled_normal((G, c, d), d ** -0.5, seed + 3, DEV, spread=2)
    W3 = mi.block_scaled_normal((G, d, c), c ** -0.5, seed + 4, DEV, spread=2)
    return W1, W2, W3


def empty_h(N, c):
    return (torch.full((N, c), 0x5A, dtype=torch.uint8, device=DEV),
            torch.full((N, c // 32), 0x5A, dtype=torch.uint8, device=DEV))


def host(pair, a=None, b=None):
    return tuple(t[a:b].cpu().numpy() for t in pair)


def run_phases_and_fused(ops, Xq, offd, W1q, W2q, W3q, N, c, d, sorted_src=None, k=1):
    """(H from the gate/up call, Y from the down call on it, Y from the fused call)."""
    H = empty_h(N, c)
    ops.moe_grouped_mxfp8_gate_up(Xq, offd, W1q, W2q, H, sorted_src=sorted_src, k=k)
    Y2 = torch.full((N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ops.moe_grouped_mxfp8_down(H, offd, W3q, Y2)
    Yf = torch.full_like(Y2, float("nan"))
    ops.moe_grouped_swiglu_mxfp8(Xq, offd, W1q, W2q, W3q, Yf, sorted_src=sorted_src, k=k)
    _sync()
    return H, Y2, Yf


SHAPES = [
    (1000, 8, 256, 256, None),                  # ragged tails in every group
    (777, 5, 128, 128, [0, 700, 0, 77, 0]),     # empty groups
    (129, 1, 256, 128, None),                   # one group, one row past a tile
    (1, 3, 128, 128, [0, 1, 0]),                # a single row
    (0, 4, 128, 128, [0, 0, 0, 0]),             # empty input
    (600, 2, 384, 640, None),                   # partial output tiles in both products
    (3000, 16, 512, 384, "zipf"),               # skewed groups spanning many tiles
]


def sizes_for(N, G, seed, sizes):
    if sizes is None:
        return mi.group_sizes(N, G, seed).tolist()
    if sizes == "zipf":
        return mi.group_sizes(N, G, seed, zipf=1.5).tolist()
    return sizes


@pytest.mark.parametrize("N,G,d,c,sizes", SHAPES)
def test_grouped_mxfp8_products(ops, N, G, d, c, sizes):
    seed = mi.seed_for(92, N, G, d, c)
    sizes = sizes_for(N, G, seed, sizes)
    X = mi.block_scaled_normal((N, d), 1.0, seed + 1, DEV, spread=3)
    W1, W2, W3 = make_weights(G, d, c, seed)
    Xq = ops.mx_quantized(X)
    W1q, W2q, W3q = ops.mx_quantized(W1), ops.mx_quantized(W2), ops.mx_quantized(W3)
    off = offsets_of(sizes)
    H, Y2, Yf = run_phases_and_fused(ops, Xq, torch.from_numpy(off).to(DEV), W1q, W2q, W3q, N, c, d)
    assert torch.equal(Y2, Yf), "fused call differs from gate/up + down"
    if N == 0:
        return
    o1, o2, o3 = oracle_stack(W1, W1q), oracle_stack(W2, W2q), oracle_stack(W3, W3q)
    Xn = to_np(X).astype(np.float64)
    flips = 0
    for g in range(G):
        a, b = int(off[g]), int(off[g + 1])
        if b == a:
            continue
        flips += check_hidden(*host(H, a, b), Xn[a:b], o1[g], o2[g], f"H of group {g}")
        check_down(to_np(Y2[a:b]), host(H, a, b), o3[g], f"Y of group {g} from the call's own H")
        check_end_to_end(to_np(Yf[a:b]), Xn[a:b], o1[g], o2[g], o3[g], f"group {g}")
    print(f"H values differing from the oracle's: {flips} of {N * c}")


@pytest.mark.parametrize("N,G,d,c,sizes", SHAPES)
def test_grouped_mxfp8_down_given_operands(ops, N, G, d, c, sizes):
    """The second product alone on MXFP8 operands drawn by the test (random finite codes and
    scales, so every E4M3 value and a wide range of block scales occur)."""
    seed = mi.seed_for(90, N, G, d, c)
    sizes = sizes_for(N, G, seed, sizes)
    Hq = mi.mx_random_codes(N, c, seed + 1, DEV)
    W3q = mi.mx_random_codes(G * d, c, seed + 2, DEV)
    W3q = (W3q[0].view(G, d, c), W3q[1].view(G, d, c // 32))
    off = offsets_of(sizes)
    Y = torch.full((N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ops.moe_grouped_mxfp8_down(Hq, torch.from_numpy(off).to(DEV), W3q, Y)
    _sync()
    for g in range(G):
        a, b = int(off[g]), int(off[g + 1])
        if b > a:
            check_down(to_np(Y[a:b]), host(Hq, a, b), (W3q[0][g].cpu().numpy(), W3q[1][g].cpu().numpy()),
                       f"group {g}")


@pytest.mark.parametrize("T,E,k,d,c", [(333, 6, 2, 128, 256), (1000, 16, 4, 256, 128), (5, 8, 8, 128, 128)])
def test_grouped_mxfp8_gathered(ops, T, E, k, d, c):
    """Rows gathered through the permutation give the same bits as the permuted copy."""
    seed = mi.seed_for(91, T, E, k)
    idx = mi.topk_assignments(T, E, k, seed, DEV)
    A = mi.block_scaled_normal((T, d), 1.0, seed + 1, DEV, spread=3)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    src = torch.empty(T * k, dtype=torch.int32, device=DEV)
    dest = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ops.moe_permute(idx, E, off, src, dest)
    W1, W2, W3 = make_weights(E, d, c, seed)
    Aq = ops.mx_quantized(A)
    W1q, W2q, W3q = ops.mx_quantized(W1), ops.mx_quantized(W2), ops.mx_quantized(W3)
    N = T * k
    Hg, Yg2, Ygf = run_phases_and_fused(ops, Aq, off, W1q, W2q, W3q, N, c, d, sorted_src=src, k=k)
    tok = (src // k).long()
    Pq = (Aq[0][tok].contiguous(), Aq[1][tok].contiguous())
    Hp, Yp2, Ypf = run_phases_and_fused(ops, Pq, off, W1q, W2q, W3q, N, c, d)
    assert torch.equal(Hg[0], Hp[0]) and torch.equal(Hg[1], Hp[1])
    assert torch.equal(Ygf, Ypf) and torch.equal(Yg2, Ygf)
    off_np, src_np = off.cpu().numpy(), src.cpu().numpy()
    Xp = oracle.permute_rows(to_np(A).astype(np.float64), src_np, k)
    o1, o2, o3 = oracle_stack(W1), oracle_stack(W2), oracle_stack(W3)
    for g in range(E):
        a, b = int(off_np[g]), int(off_np[g + 1])
        if b > a:
            check_hidden(*host(Hg, a, b), Xp[a:b], o1[g], o2[g], f"H of group {g}")
            check_end_to_end(to_np(Ygf[a:b]), Xp[a:b], o1[g], o2[g], o3[g], f"group {g}")


def test_grouped_mxfp8_small_tiles_bitwise_equal_large(ops):
    """Groups averaging at most 96 rows (or grids too small to give every CU a workgroup) run on
    64-row tiles with three stages, the rest on 256-row tiles with two.  The same rows and weights
    with empty groups appended (which moves the average below the switch) must give bit-identical
    H and Y: both tilings sum every output over K in the same order.  Then the 64-row result
    against the oracle's bars."""
    d, c = 256, 2048
    sizes = [2500, 0, 3100, 2592]                   # 2048 rows per group, 640 big tiles: 256-row tiles
    extra = [0] * 100                               # 8192 rows over 104 groups: 64-row tiles
    N = sum(sizes)
    seed = mi.seed_for(89, N, d, c)
    A = mi.block_scaled_normal((N, d), 1.0, seed, DEV, spread=3)
    G = len(sizes) + len(extra)
    W1, W2, W3 = make_weights(G, d, c, seed)
    Aq = ops.mx_quantized(A)
    g = len(sizes)
    big = [ops.mx_quantized(W[:g].contiguous()) for W in (W1, W2, W3)]
    small = [ops.mx_quantized(W) for W in (W1, W2, W3)]
    off_big = torch.from_numpy(offsets_of(sizes)).to(DEV)
    off_small = torch.from_numpy(offsets_of(sizes + extra)).to(DEV)
    H_big, _, Y_big = run_phases_and_fused(ops, Aq, off_big, *big, N, c, d)
    H_small, _, Y_small = run_phases_and_fused(ops, Aq, off_small, *small, N, c, d)
    assert torch.equal(H_big[0], H_small[0]) and torch.equal(H_big[1], H_small[1])
    assert torch.equal(Y_big, Y_small)
    A_np = to_np(A).astype(np.float64)
    o1, o2, o3 = oracle_stack(W1[:g]), oracle_stack(W2[:g]), oracle_stack(W3[:g])
    off_np = offsets_of(sizes)
    for e in range(g):
        a, b = int(off_np[e]), int(off_np[e + 1])
        if b > a:
            rows = np.array(list(range(a, min(a + 40, b))) + list(range(max(a, b - 40), b)))
            check_hidden(H_small[0][rows].cpu().numpy(), H_small[1][rows].cpu().numpy(), A_np[rows], o1[e], o2[e],
                         f"H of group {e}")
            check_end_to_end(to_np(Y_small[rows]), A_np[rows], o1[e], o2[e], o3[e], f"group {e}")


DSV3 = {c.name: c for c in mi.CONFIGS}["dsv3-stack"]


def test_grouped_mxfp8_dsv3_full_size_sampled(ops):
    """The DeepSeek-V3-shaped layer at full size in the bench's launch configuration: 65536 tokens
    x 8 slots over 256 experts (d = 7168, c = 2048), activations quantised and gathered through the
    permutation.  Sampled token rows quantise bit-exactly; for the first and last rows of eight
    experts (the first and the last, the largest and the smallest group, four seeded others) H is
    checked against the oracle (weights quantised by the oracle from the same bf16 values) and the
    whole MLP's Y to its mean bar; the fused call equals the two calls bit for bit."""
    cfg = DSV3
    T, E, k, d, c = cfg.T, cfg.E, cfg.k, cfg.d, cfg.c
    W = mi.layer_weights(cfg, 0, DEV)
    A = mi.activations(cfg, DEV)
    idx = mi.topk_assignments(T, E, k, mi.seed_for(cfg.cfg_id, 0, mi.T_TOPK), DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    src = torch.empty(T * k, dtype=torch.int32, device=DEV)
    dest = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ops.moe_permute(idx, E, off, src, dest)
    Aq = ops.mx_quantized(A)
    W1q, W2q, W3q = ops.mx_quantized(W["W1"]), ops.mx_quantized(W["W2"]), ops.mx_quantized(W["W3"])
    H, Y2, Yf = run_phases_and_fused(ops, Aq, off, W1q, W2q, W3q, T * k, c, d, sorted_src=src, k=k)
    assert torch.equal(Y2, Yf), "fused call differs from gate/up + down"
    assert not torch.isnan(Yf.float()).any().item()
    off_np, src_np = off.cpu().numpy(), src.cpu().numpy()
    A_np = to_np(A).astype(np.float64)
    rows_t = mi.sample_rows(T, 64, mi.seed_for(cfg.cfg_id, 0, mi.T_SAMPLE)).numpy()
    ref = mx.mx_quantize(A_np[rows_t])
    np.testing.assert_array_equal(Aq[0][rows_t].cpu().numpy(), ref[0])
    np.testing.assert_array_equal(Aq[1][rows_t].cpu().numpy(), ref[1])
    sizes = np.diff(off_np)
    sel = {0, E - 1, int(np.argmax(sizes)), int(np.argmin(sizes))}
    for e in np.random.default_rng(mi.seed_for(cfg.cfg_id, 0, mi.T_SAMPLE, 2)).permutation(E):
        if len(sel) == 8:
            break
        sel.add(int(e))
    for e in sorted(sel):
        a, b = int(off_np[e]), int(off_np[e + 1])
        rows = np.array(list(range(a, min(a + 6, b))) + list(range(max(a, b - 6), b)))
        Wq = []
        for Wt, Wg in ((W["W1"], W1q), (W["W2"], W2q), (W["W3"], W3q)):
            q = mx.mx_quantize(to_np(Wt[e]).astype(np.float64))
            np.testing.assert_array_equal(Wg[0][e].cpu().numpy(), q[0])
            np.testing.assert_array_equal(Wg[1][e].cpu().numpy(), q[1])
            Wq.append(q)
        Xe = A_np[src_np[rows] // k]
        check_hidden(H[0][rows].cpu().numpy(), H[1][rows].cpu().numpy(), Xe, Wq[0], Wq[1], f"H of expert {e}")
        check_end_to_end(to_np(Yf[rows]), Xe, *Wq, f"expert {e}")


def test_grouped_mxfp8_down_dsv3_full_size_sampled(ops):
    """The second product at the DeepSeek-V3 layer's full size (524288 grouped rows over 256
    experts, c = 2048 -> d = 7168) on random MXFP8 operands: the first and the last row of every
    expert (its first and last M-tile) on 256 sampled output columns, one in each 28-column stripe
    (so every 256-column N-tile is reached)."""
    cfg = DSV3
    N, E, d, c = cfg.T * cfg.k, cfg.E, cfg.d, cfg.c
    seed = mi.seed_for(cfg.cfg_id, 0, mi.T_MISC, 0, 77)
    sizes = mi.group_sizes(N, E, mi.seed_for(cfg.cfg_id, 0, mi.T_GROUPS)).tolist()
    off = offsets_of(sizes)
    Hq = mi.mx_random_codes(N, c, seed, DEV)
    W3 = mi.mx_random_codes(E * d, c, seed + 1, DEV)
    W3q = (W3[0].view(E, d, c), W3[1].view(E, d, c // 32))
    Y = torch.empty((N, d), dtype=torch.bfloat16, device=DEV)
    ops.moe_grouped_mxfp8_down(Hq, torch.from_numpy(off).to(DEV), W3q, Y)
    _sync()
    stripe = d // 256
    cols = np.arange(0, d, stripe) + np.random.default_rng(seed).integers(0, stripe, size=256)
    cols_d = torch.from_numpy(cols).to(DEV)
    checked = 0
    for e in range(E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        rows = np.array(sorted({a, b - 1}))
        check_down(to_np(Y[rows][:, cols_d]), (Hq[0][rows].cpu().numpy(), Hq[1][rows].cpu().numpy()),
                   (W3q[0][e][cols_d].cpu().numpy(), W3q[1][e][cols_d].cpu().numpy()), f"expert {e}")
        checked += 1
    assert checked == int(np.count_nonzero(np.diff(off)))


# =================================================================================================
# the scaled fp8 instruction's accumulation error: the measurement behind E_INSTR (tests/mx_bound.py)
# =================================================================================================
@pytest.mark.parametrize("c", [128, 2048, 7168], ids=["one-instruction", "chain-16", "chain-56"])
@pytest.mark.parametrize("kind", ["random-codes", "cancelling-pairs"])
def test_mxfp8_instruction_error_measured(ops, c, kind):
    """The second product with one group on operands drawn by the test (c = 128: each output is one
    instruction's result; 2048 and 7168: chains of 16 and 56 into one fp32 accumulator).  Per
    output, the error beyond Y's own bf16 rounding (2^-8 |ref|), over the sum across its 128-wide K
    chunks of 2^floor(log2 max(largest |product|, |partial sum|)), is the instruction's error in the
    unit the MXFP8 bars use; its maximum is reported and must not exceed E_INSTR.  Random codes
    are what the bars meet in the products; the cancelling pairs leave small results beside large
    products, so that the output's rounding does not hide the instruction's error."""
    N, d = 256, 256
    seed = mi.seed_for(93, c, 0 if kind == "random-codes" else 1)
    if kind == "random-codes":
        Hq = mi.mx_random_codes(N, c, seed + 1, DEV)
        W3q = mi.mx_random_codes(d, c, seed + 2, DEV)
    else:
        Hq, W3q = mi.mx_cancelling_codes(N, c, d, seed, DEV)
    Y = torch.full((N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    off = torch.tensor([0, N], dtype=torch.int32, device=DEV)
    ops.moe_grouped_mxfp8_down(Hq, off, (W3q[0].view(1, d, c), W3q[1].view(1, d, c // 32)), Y)
    _sync()
    Hh = (Hq[0].cpu().numpy(), Hq[1].cpu().numpy())
    Wh = (W3q[0].cpu().numpy(), W3q[1].cpu().numpy())
    ref = mx.mx_matmul(Hh, Wh)
    unit = instr_bound(mx.mx_dequantize(*Hh), mx.mx_dequantize(*Wh)) / E_INSTR
    err = np.abs(to_np(Y).astype(np.float64) - ref)
    beyond = np.maximum(err - 2.0 ** -8 * np.abs(ref), 0.0)
    e_meas = float((beyond / unit).max())
    hidden = float((2.0 ** -8 * np.abs(ref) / unit).mean())
    report(f"fp8 instruction error, {kind}, K = {c}", e_instr_measured=e_meas, e_instr_bar=E_INSTR,
           bf16_rounding_over_unit_mean=hidden)
    if kind == "cancelling-pairs":   # the construction makes the instruction's error visible
        assert hidden < 0.25 * E_INSTR
    assert e_meas <= E_INSTR, f"measured {e_meas:.3e} = 2^{np.log2(max(e_meas, 1e-300)):.2f} > E_INSTR"
