"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Bars: integer and copy outputs (top-k indices given identical fp32 logits, permutation arrays,
permuted rows) bit-exact; float outputs max|err| <= 2e-2 * max|ref| (bf16 storage, fp32
accumulation) or <= 1e-4 * max|ref| (fp32).  Full-size workloads are checked on seeded samples of
rows: with dropless routing every output row depends only on its own input row, so the oracle
evaluates exactly those rows.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.helpers import (NEAR_TIE, ExpertSlices, assert_mirror, assert_parity, combine_bound, dkey, max_rel_err,
                           oracle_weights, report, to_np)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def ops():
    from mixture_experts_layer_sum_amd import ops as _ops
    return _ops


def _sync():
    torch.cuda.synchronize()


CFG = {c.name: c for c in mi.CONFIGS}
ALL = [c.name for c in mi.CONFIGS]


# =================================================================================================
# a2: top-k selection and gate weights, identical fp32 logits on both sides
# =================================================================================================
def run_topk(ops, L, k, gate, renorm):
    T, E = L.shape
    Ld = L.to(DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, k), dtype=torch.float32, device=DEV)
    ops.moe_route_from_logits(Ld, k, gate, renorm, idx, w)
    _sync()
    return idx.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name", ALL)
def test_topk_bitexact_config(ops, name):
    c = CFG[name]
    bias = mi.normal((c.E,), 1.0, mi.seed_for(c.cfg_id, 0, mi.T_BIAS)) if c.router_bias else None
    L = mi.logits(c.T, c.E, mi.seed_for(c.cfg_id, 0, mi.T_LOGITS), bias=bias)
    idx, w = run_topk(ops, L, c.k, c.gate, c.renormalize)
    Ln = L.numpy()
    ref_idx = oracle.select_topk(Ln, c.k)
    np.testing.assert_array_equal(idx, ref_idx)
    ref_w = oracle.gate_weights(Ln, ref_idx, c.gate, c.renormalize)
    np.testing.assert_allclose(w, ref_w, rtol=2e-6, atol=1e-7)


@pytest.mark.parametrize("E,k", [(1, 1), (3, 3), (8, 2), (16, 16), (64, 6), (65, 7), (128, 8), (200, 5), (256, 8),
                                 (256, 16), (257, 9), (64, 17), (512, 16), (1024, 32)])
@pytest.mark.parametrize("gate,renorm", [("softmax", False), ("softmax", True), ("sigmoid", True)])
def test_topk_ties_and_shapes(ops, E, k, gate, renorm):
    # logits snapped to multiples of 0.5 so that exact ties are everywhere; the shapes straddle the
    # two selection kernels (sixteen lanes per token up to E = 256 and k = 16, a wavefront beyond) and
    # T = 777 leaves a partial block of tokens
    L = mi.logits(777, E, mi.seed_for(99, E, mi.T_LOGITS, k), quantum=0.5)
    idx, w = run_topk(ops, L, k, gate, renorm)
    ref_idx = oracle.select_topk(L.numpy(), k)
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_allclose(w, oracle.gate_weights(L.numpy(), ref_idx, gate, renorm), rtol=2e-6, atol=1e-7)


def test_topk_all_equal_and_signed_zero(ops):
    L = torch.zeros((5, 16), dtype=torch.float32)
    L[1] = -0.0
    L[2, ::2] = -0.0
    L[3] = 1.0
    L[4] = torch.arange(16, dtype=torch.float32)
    idx, w = run_topk(ops, L, 4, "softmax", False)
    np.testing.assert_array_equal(idx, oracle.select_topk(L.numpy(), 4))
    assert idx[0].tolist() == [0, 1, 2, 3] and idx[4].tolist() == [15, 14, 13, 12]


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (256, 8), (1024, 32)])
def test_topk_nan_logits_rank_last(ops, E, k):
    """A NaN logit is read as -infinity: every returned id lies in [0, E), and the selection and
    weights equal the oracle's on the logits with NaN replaced by -inf (rows where all but k - 1
    logits are NaN included, so a NaN must be selected)."""
    T = 300
    L = mi.logits(T, E, mi.seed_for(99, E, mi.T_LOGITS, k, 7))
    g = np.random.default_rng(E + k)
    nan = g.random((T, E)) < 0.3
    nan[:20] = True
    nan[:20, : k - 1] = False   # the first rows keep only k - 1 numbers
    Ln = np.where(nan, np.float32(np.nan), L.numpy()).astype(np.float32)
    idx, w = run_topk(ops, torch.from_numpy(Ln), k, "softmax", True)
    assert idx.min() >= 0 and idx.max() < E
    ref_in = np.where(np.isnan(Ln), -np.inf, Ln)
    ref_idx = oracle.select_topk(ref_in, k)
    np.testing.assert_array_equal(idx, ref_idx)
    np.testing.assert_allclose(w[20:], oracle.gate_weights(ref_in, ref_idx, "softmax", True)[20:], rtol=2e-6,
                               atol=1e-7)


# =================================================================================================
# a1: router logits (bf16 MFMA / fp32), sampled rows at full size
# =================================================================================================
@pytest.mark.parametrize("name", ALL)
def test_router_logits(ops, name):
    c = CFG[name]
    A = mi.activations(c, DEV)
    W_R = mi.normal((c.E, c.d), c.w_std, mi.seed_for(c.cfg_id, 0, mi.T_WR), DEV, c.torch_dtype)
    bias = mi.normal((c.E,), 1.0, mi.seed_for(c.cfg_id, 0, mi.T_BIAS), DEV) if c.router_bias else None
    logits = torch.empty((c.T, c.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((c.T, c.k), dtype=torch.int32, device=DEV)
    w = torch.empty((c.T, c.k), dtype=torch.float32, device=DEV)
    ops.moe_route(A, W_R, c.k, c.gate, c.renormalize, logits, idx, w, bias=bias)
    _sync()
    rows = mi.sample_rows(c.T, 1024, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE))
    ref = oracle.router_logits(to_np(A[rows.to(DEV)]), to_np(W_R), None if bias is None else to_np(bias))
    got = to_np(logits[rows.to(DEV)])
    # the products are exact in fp32 and summed in fp32: far inside the bf16 bar
    assert_parity(got, ref, c.torch_dtype, "logits")
    assert max_rel_err(got, ref) < 1e-5   # exact products, fp32 sums of at most d = 7168 terms
    # the selection made on the GPU's own logits satisfies the top-k rule (property, all T)
    check_topk_property(to_np(logits), idx.cpu().numpy())


@pytest.mark.parametrize("T,E,k,gate,renorm,bias", [(65536 + 77, 256, 8, "sigmoid", True, False),
                                                    (66000, 128, 8, "softmax", True, True),
                                                    (65600, 64, 6, "softmax", False, False),
                                                    (65536, 200, 5, "softmax", True, True),
                                                    (65536, 16, 1, "sigmoid", False, False)])
def test_route_equals_topk_of_its_logits(ops, T, E, k, gate, renorm, bias):
    """moe_route at batch sizes that run the 256-row router tiles: its ids and weights equal, bit for
    bit, those of the logits-input call on the logits it wrote (so every bit-exact top-k test covers
    this path); the logits match the oracle on sampled rows; the selection follows the oracle's rule
    on them; a ragged last tile and E below the tile width are covered."""
    d = 256
    seed = mi.seed_for(92, T, E, k)
    A = mi.normal((T, d), 1.0, seed, DEV, torch.bfloat16)
    W_R = mi.normal((E, d), 0.1, seed + 1, DEV, torch.bfloat16)
    b = mi.normal((E,), 1.0, seed + 2, DEV) if bias else None
    logits = torch.full((T, E), float("nan"), dtype=torch.float32, device=DEV)
    idx = torch.full((T, k), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device=DEV)
    ops.moe_route(A, W_R, k, gate, renorm, logits, idx, w, bias=b)
    idx2 = torch.full_like(idx, -1)
    w2 = torch.full_like(w, float("nan"))
    ops.moe_route_from_logits(logits, k, gate, renorm, idx2, w2)
    _sync()
    assert torch.equal(idx, idx2)
    assert torch.equal(w.view(torch.int32), w2.view(torch.int32))
    rows = mi.sample_rows(T, 512, seed + 3)
    ref = oracle.router_logits(to_np(A[rows.to(DEV)]), to_np(W_R), None if b is None else to_np(b))
    assert max_rel_err(to_np(logits[rows.to(DEV)]), ref) < 1e-5
    np.testing.assert_array_equal(idx[rows.to(DEV)].cpu().numpy(), oracle.select_topk(to_np(logits[rows.to(DEV)]), k))


def check_topk_property(L, idx):
    T, E = L.shape
    k = idx.shape[1]
    sel = np.take_along_axis(L, idx.astype(np.int64), 1)
    # slot order: descending logit, ties by ascending index
    assert np.all((sel[:, :-1] > sel[:, 1:]) | ((sel[:, :-1] == sel[:, 1:]) & (idx[:, :-1] < idx[:, 1:])))
    mask = np.ones((T, E), bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, 1)
    rest = np.where(mask, L, -np.inf)
    worst_sel = sel[:, -1]
    best_rest = rest.max(1)
    assert np.all(worst_sel >= best_rest)
    # where the boundary ties, the unselected equal logits have larger indices
    tie_rows = np.nonzero(worst_sel == best_rest)[0]
    for t in tie_rows:
        tied = np.nonzero(mask[t] & (L[t] == worst_sel[t]))[0]
        assert tied.min() > idx[t][sel[t] == worst_sel[t]].max()


# =================================================================================================
# a3: dispatch permutation, bit-exact
# =================================================================================================
def run_permute(ops, idx_np, E, A=None):
    T, k = idx_np.shape
    idx = torch.from_numpy(np.ascontiguousarray(idx_np)).to(torch.int32).to(DEV)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    src = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    dest = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
    Ap = torch.empty((T * k, A.shape[1]), dtype=A.dtype, device=DEV) if A is not None else None
    ops.moe_permute(idx, E, off, src, dest, A=A, A_perm=Ap)
    _sync()
    return off.cpu().numpy(), src.cpu().numpy(), dest.cpu().numpy(), Ap


@pytest.mark.parametrize("name", ALL)
def test_permute_bitexact_config(ops, name):
    c = CFG[name]
    zipf = 1.1 if c.router_bias else 0.0
    idx = mi.topk_assignments(c.T, c.E, c.k, mi.seed_for(c.cfg_id, 0, mi.T_TOPK), zipf=zipf).numpy()
    A = mi.activations(c, DEV)
    off, src, dest, Ap = run_permute(ops, idx, c.E, A)
    r_off, r_src, r_dest = oracle.permute(idx, c.E)
    np.testing.assert_array_equal(off, r_off)
    np.testing.assert_array_equal(src, r_src)
    np.testing.assert_array_equal(dest, r_dest)
    rows = mi.sample_rows(c.T * c.k, 4096, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 1))
    got = Ap[rows.to(DEV)]
    ref_tok = torch.from_numpy(r_src[rows.numpy()].astype(np.int64) // c.k).to(DEV)
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                       A[ref_tok].view(torch.int16) if A.dtype == torch.bfloat16 else A[ref_tok].view(torch.int32))


@pytest.mark.parametrize("T,E,k,kind", [(1, 1, 1, "uniform"), (1, 8, 8, "uniform"), (3, 4, 2, "uniform"),
                                        (4097, 5, 3, "uniform"), (5000, 64, 6, "one-hot"),
                                        (2500, 1024, 4, "zipf"), (333, 7, 5, "repeats"), (1, 1024, 32, "uniform")])
def test_permute_edges(ops, T, E, k, kind):
    seed = mi.seed_for(98, T, E, k)
    if kind == "one-hot":
        idx = np.zeros((T, k), np.int32)
        idx[:] = np.arange(k, dtype=np.int32)  # every token picks experts 0..k-1: the rest stay empty
    elif kind == "repeats":
        g = np.random.default_rng(seed)
        idx = g.integers(0, E, size=(T, k)).astype(np.int32)  # ids may repeat inside a token
    else:
        idx = mi.topk_assignments(T, E, k, seed, zipf=1.5 if kind == "zipf" else 0.0).numpy()
    A = mi.normal((T, 64), 1.0, seed, DEV, torch.bfloat16)
    off, src, dest, Ap = run_permute(ops, idx, E, A)
    r_off, r_src, r_dest = oracle.permute(idx, E)
    np.testing.assert_array_equal(off, r_off)
    np.testing.assert_array_equal(src, r_src)
    np.testing.assert_array_equal(dest, r_dest)
    ref = A[torch.from_numpy(r_src.astype(np.int64) // k).to(DEV)]
    assert torch.equal(Ap.view(torch.int16), ref.view(torch.int16))


def test_permute_empty_batch_writes_zero_offsets(ops):
    idx = np.zeros((0, 2), np.int32)
    off, _, _, _ = run_permute(ops, idx, 6)
    np.testing.assert_array_equal(off, np.zeros(7, np.int32))


def test_permute_is_deterministic(ops):
    c = CFG["dsv3-stack"]
    idx = mi.topk_assignments(c.T, c.E, c.k, mi.seed_for(c.cfg_id, 0, mi.T_TOPK)).numpy()
    a = run_permute(ops, idx, c.E)
    b = run_permute(ops, idx, c.E)
    for x, y in zip(a[:3], b[:3]):
        np.testing.assert_array_equal(x, y)


# =================================================================================================
# a4: grouped SwiGLU GEMM
# =================================================================================================
def run_swiglu(ops, X, sizes, W1, W2, W3):
    off = torch.zeros(len(sizes) + 1, dtype=torch.int32)
    off[1:] = torch.cumsum(torch.as_tensor(sizes, dtype=torch.int64), 0).to(torch.int32)
    offd = off.to(DEV)
    Y = torch.full((X.shape[0], X.shape[1]), float("nan"), dtype=X.dtype, device=DEV)
    ops.moe_grouped_swiglu(X, offd, W1, W2, W3, Y)
    _sync()
    return off.numpy(), Y


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,G,d,c,sizes", [
    (1000, 8, 256, 192, None),          # ragged tails in every group
    (777, 5, 128, 128, [0, 700, 0, 77, 0]),   # empty groups
    (129, 1, 192, 64, None),            # one group, one row past a tile
    (1, 3, 64, 64, [0, 1, 0]),          # a single row
    (0, 4, 64, 64, [0, 0, 0, 0]),       # empty input
    (3000, 16, 512, 320, "zipf"),       # skewed groups spanning many tiles
])
def test_grouped_swiglu_small(ops, dtype, N, G, d, c, sizes):
    seed = mi.seed_for(97, N, G, d, c)
    if sizes is None:
        sizes = mi.group_sizes(N, G, seed).tolist()
    elif sizes == "zipf":
        sizes = mi.group_sizes(N, G, seed, zipf=1.5).tolist()
    std = 1.0 / d ** 0.5
    X = mi.normal((N, d), 1.0, seed + 1, DEV, dtype)
    W1 = mi.normal((G, c, d), std, seed + 2, DEV, dtype)
    W2 = mi.normal((G, c, d), std, seed + 3, DEV, dtype)
    W3 = mi.normal((G, d, c), 1.0 / c ** 0.5, seed + 4, DEV, dtype)
    off, Y = run_swiglu(ops, X, sizes, W1, W2, W3)
    if N == 0:
        return
    W1s, W2s, W3s = ExpertSlices(W1), ExpertSlices(W2), ExpertSlices(W3)
    ref = oracle.grouped_mlp(to_np(X), off, W1s, W2s, W3s)
    assert_parity(to_np(Y), ref, dtype, "grouped swiglu")
    if dtype == torch.bfloat16:
        mref = oracle.grouped_mlp(to_np(X), off, W1s, W2s, W3s, store=oracle.round_to_bf16)
        assert_mirror(to_np(Y), mref, "grouped swiglu")


@pytest.mark.parametrize("name", ["dsv2-lite", "qwen3-30b-a3b", "llama4-scout", "dsv3-stack"])
def test_grouped_swiglu_config_dims(ops, name):
    """The workloads' (d, c) with a few experts and ragged row counts."""
    c = CFG[name]
    G = 3
    sizes = [130, 0, 301] if c.d <= 5120 else [70, 0, 200]
    N = sum(sizes)
    seed = mi.seed_for(c.cfg_id, 5, mi.T_MISC)
    X = mi.normal((N, c.d), 1.0, seed, DEV, c.torch_dtype)
    W1 = mi.normal((G, c.c, c.d), c.w_std, seed + 1, DEV, c.torch_dtype)
    W2 = mi.normal((G, c.c, c.d), c.w_std, seed + 2, DEV, c.torch_dtype)
    W3 = mi.normal((G, c.d, c.c), c.w3_std, seed + 3, DEV, c.torch_dtype)
    off, Y = run_swiglu(ops, X, sizes, W1, W2, W3)
    W1s, W2s, W3s = ExpertSlices(W1), ExpertSlices(W2), ExpertSlices(W3)
    ref = oracle.grouped_mlp(to_np(X), off, W1s, W2s, W3s)
    assert_parity(to_np(Y), ref, c.torch_dtype, name)
    assert_mirror(to_np(Y), oracle.grouped_mlp(to_np(X), off, W1s, W2s, W3s, store=oracle.round_to_bf16), name)


def check_every_expert_edges(c, off, X, Y, W, n_edge):
    """Rows of every group checked against the oracle: the first and the last n_edge rows of each
    expert (its first and last M-tile, so a tile given another expert's weights or rows fails).
    Each expert's weights are copied once and not kept (22.5 GB per DeepSeek-V3 layer)."""
    W1, W2, W3 = (ExpertSlices(W[key], cache=False) for key in ("W1", "W2", "W3"))
    got_all, ref_all, mref_all = [], [], []
    for e in range(c.E):
        a, b = int(off[e]), int(off[e + 1])
        if b == a:
            continue
        rows = sorted(set(range(a, min(a + n_edge, b))) | set(range(max(a, b - n_edge), b)))
        x = to_np(X[rows])
        w1, w2, w3 = W1[e], W2[e], W3[e]
        ref_all.append(oracle.mlp(x, w1, w2, w3))
        mref_all.append(oracle.mlp(x, w1, w2, w3, store=oracle.round_to_bf16))
        got_all.append(to_np(Y[rows]))
    assert len(W1.fetched) == int(np.count_nonzero(np.diff(off)))
    got, ref, mref = (np.concatenate(v) for v in (got_all, ref_all, mref_all))
    assert_parity(got, ref, c.torch_dtype, f"{c.name}: edge rows of {len(W1.fetched)} experts")
    assert_mirror(got, mref, f"{c.name}: edge rows of {len(W1.fetched)} experts")


def test_grouped_swiglu_dsv3_full_size_sampled(ops):
    """All 524288 routed rows of the DeepSeek-V3-shaped layer in the bench launch configuration
    (256-row tiles over 256 experts); the first and last row of every expert against the oracle."""
    c = CFG["dsv3-stack"]
    N = c.T * c.k
    W = mi.layer_weights(c, 0, DEV)
    sizes = mi.group_sizes(N, c.E, mi.seed_for(c.cfg_id, 0, mi.T_GROUPS)).tolist()
    X = mi.normal((N, c.d), 1.0, mi.seed_for(c.cfg_id, 0, mi.T_ACT, 9), DEV, c.torch_dtype)
    off, Y = run_swiglu(ops, X, sizes, W["W1"], W["W2"], W["W3"])
    assert not torch.isnan(Y.float()).any().item()
    check_every_expert_edges(c, off, X, Y, W, 1)


def test_grouped_swiglu_small_tiles_bitwise_equal_large(ops):
    """Groups averaging at most 96 rows (or grids too small to give every CU a workgroup) run on
    64-row tiles, the rest on 256-row tiles.  The same rows and weights with empty groups appended
    (which moves the average below the switch) must give bit-identical outputs: both tilings sum
    every output over K in the same order."""
    d, c = 128, 2048
    sizes = [2500, 0, 3100, 2592]                   # 2048 rows per group, 576 big tiles: 256-row tiles
    extra = [0] * 100                               # 8192 rows over 104 groups: 64-row tiles
    N = sum(sizes)
    seed = mi.seed_for(95, N, d, c)
    X = mi.normal((N, d), 1.0, seed, DEV, torch.bfloat16)
    G = len(sizes) + len(extra)
    W1 = mi.normal((G, c, d), d ** -0.5, seed + 1, DEV, torch.bfloat16)
    W2 = mi.normal((G, c, d), d ** -0.5, seed + 2, DEV, torch.bfloat16)
    W3 = mi.normal((G, d, c), c ** -0.5, seed + 3, DEV, torch.bfloat16)
    g = len(sizes)
    _, Y_large = run_swiglu(ops, X, sizes, W1[:g].contiguous(), W2[:g].contiguous(), W3[:g].contiguous())
    off, Y_small = run_swiglu(ops, X, sizes + extra, W1, W2, W3)
    assert torch.equal(Y_large, Y_small)
    # 30 more empty groups take the average to at most 64 rows (one 64-row tile per group on
    # average), where the routed launches stream the weights with the nontemporal hint: the cache
    # policy changes no value
    more = [0] * 30
    Gm = G + len(more)
    W1m, W2m, W3m = (torch.cat([w, w[:len(more)]]) for w in (W1, W2, W3))
    _, Y_stream = run_swiglu(ops, X, sizes + extra + more, W1m, W2m, W3m)
    assert N <= 64 * Gm < 96 * Gm and torch.equal(Y_stream, Y_small)
    ref = oracle.grouped_mlp(to_np(X), off, ExpertSlices(W1), ExpertSlices(W2), ExpertSlices(W3))
    assert_parity(to_np(Y_small), ref, torch.bfloat16, "64-row tiles")


def test_grouped_swiglu_decode_shape_sampled(ops):
    """One decode step of the DeepSeek-V3-shaped layer: 1024 tokens x 8 slots over 256 experts
    (about 32 rows each, the 64-row tiling), real layer weights; the first and last two rows of
    every expert against the oracle."""
    c = CFG["dsv3-decode"]
    N = c.T * c.k
    W = mi.layer_weights(c, 0, DEV)
    sizes = mi.group_sizes(N, c.E, mi.seed_for(c.cfg_id, 0, mi.T_GROUPS)).tolist()
    X = mi.normal((N, c.d), 1.0, mi.seed_for(c.cfg_id, 0, mi.T_ACT, 9), DEV, c.torch_dtype)
    off, Y = run_swiglu(ops, X, sizes, W["W1"], W["W2"], W["W3"])
    assert not torch.isnan(Y.float()).any().item()
    check_every_expert_edges(c, off, X, Y, W, 2)


# =================================================================================================
# a3 + a4 fused: rows gathered through the permutation (the stack's launch configuration)
# =================================================================================================
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,E,k,d,c,kind", [(333, 6, 2, 128, 192, "uniform"), (1000, 16, 4, 256, 128, "zipf"),
                                            (5, 8, 8, 64, 64, "uniform"), (700, 4, 3, 192, 320, "repeats")])
def test_grouped_swiglu_gathered(ops, dtype, T, E, k, d, c, kind):
    seed = mi.seed_for(96, T, E, k)
    if kind == "repeats":
        idx = np.random.default_rng(seed).integers(0, E, size=(T, k)).astype(np.int32)
    else:
        idx = mi.topk_assignments(T, E, k, seed, zipf=1.5 if kind == "zipf" else 0.0).numpy()
    A = mi.normal((T, d), 1.0, seed + 1, DEV, dtype)
    off, src, dest, Ap = run_permute(ops, idx, E, A)
    std = 1.0 / d ** 0.5
    W1 = mi.normal((E, c, d), std, seed + 2, DEV, dtype)
    W2 = mi.normal((E, c, d), std, seed + 3, DEV, dtype)
    W3 = mi.normal((E, d, c), 1.0 / c ** 0.5, seed + 4, DEV, dtype)
    offd = torch.from_numpy(off).to(DEV)
    Yg = torch.full((T * k, d), float("nan"), dtype=dtype, device=DEV)
    ops.moe_grouped_swiglu_gathered(A, torch.from_numpy(src).to(DEV), k, offd, W1, W2, W3, Yg)
    Yp = torch.full_like(Yg, float("nan"))
    ops.moe_grouped_swiglu(Ap, offd, W1, W2, W3, Yp)
    _sync()
    assert torch.equal(Yg, Yp)  # same rows, same order: bit-identical
    Xp = oracle.permute_rows(to_np(A), src, k)
    W1s, W2s, W3s = ExpertSlices(W1), ExpertSlices(W2), ExpertSlices(W3)
    ref = oracle.grouped_mlp(Xp, off, W1s, W2s, W3s)
    assert_parity(to_np(Yg), ref, dtype, "gathered grouped swiglu")
    if dtype == torch.bfloat16:
        assert_mirror(to_np(Yg), oracle.grouped_mlp(Xp, off, W1s, W2s, W3s, store=oracle.round_to_bf16),
                      "gathered grouped swiglu")


# =================================================================================================
# a5: combine
# =================================================================================================
@pytest.mark.parametrize("name", ALL)
@pytest.mark.parametrize("with_add", [False, True])
def test_combine(ops, name, with_add):
    c = CFG[name]
    N = c.T * c.k
    seed = mi.seed_for(c.cfg_id, 0, mi.T_Y, int(with_add))
    Y = mi.normal((N, c.d), 1.0, seed, DEV, c.torch_dtype)
    w = mi.uniform((c.T, c.k), 0.0, 1.0, seed + 1, DEV)
    dest = mi.randperm(N, seed + 2, DEV)
    addend = mi.normal((c.T, c.d), 1.0, seed + 3, DEV, c.torch_dtype) if with_add else None
    resid = mi.normal((c.T, c.d), 2.0, seed + 4, DEV) if with_add else None
    out = torch.empty((c.T, c.d), dtype=torch.float32, device=DEV)
    out_x = torch.empty((c.T, c.d), dtype=c.torch_dtype, device=DEV)
    ops.moe_combine(Y, w, dest, out, addend=addend, residual=resid, out_x=out_x)
    _sync()
    rows = mi.sample_rows(c.T, 512, seed + 5)
    rd = rows.to(DEV)
    Yn = to_np(Y)
    ref = oracle.combine(Yn, to_np(w)[rows.numpy()], dest.cpu().numpy().reshape(c.T, c.k)[rows.numpy()].reshape(-1),
                         None if addend is None else to_np(addend[rd]), None if resid is None else to_np(resid[rd]))
    got = to_np(out[rd])
    # every product is exact in fp32: only fp32 summation rounding remains
    assert_parity(got, ref, torch.float32, "combine")
    # out_x is out rounded to the workload dtype (round to nearest even)
    if c.torch_dtype == torch.bfloat16:
        np.testing.assert_array_equal(to_np(out_x[rd]), oracle.round_to_bf16(got))
    else:
        np.testing.assert_array_equal(to_np(out_x[rd]), got)


def test_combine_in_place_residual(ops):
    T, k, d = 300, 3, 256
    Y = mi.normal((T * k, d), 1.0, 5, DEV, torch.bfloat16)
    w = mi.uniform((T, k), 0.0, 1.0, 6, DEV)
    dest = mi.randperm(T * k, 7, DEV)
    o = mi.normal((T, d), 1.0, 8, DEV)
    o_ref = to_np(o)
    ops.moe_combine(Y, w, dest, o, residual=o)
    _sync()
    ref = oracle.combine(to_np(Y), to_np(w), dest.cpu().numpy(), residual=o_ref)
    assert_parity(to_np(o), ref, torch.float32, "in-place combine")


# =================================================================================================
# One MoE sublayer end to end (a1..a5), full size, sampled tokens, near-tie tokens excluded
# =================================================================================================
def cover_experts(rows, topk_idx, E, seed):
    """rows plus, for every expert that none of them routes to, one seeded token that does (so
    that the sample reaches every expert that has rows at all)."""
    rows = [int(r) for r in rows]
    hit = np.zeros(E, bool)
    hit[np.unique(topk_idx[rows])] = True
    g = np.random.default_rng(seed)
    for e in np.nonzero(~hit)[0]:
        cand = np.nonzero((topk_idx == e).any(axis=1))[0]
        if cand.size:
            t = int(g.choice(cand))
            rows.append(t)
            hit[np.unique(topk_idx[t])] = True
    return np.array(sorted(set(rows)), dtype=np.int64)


def layer_check(ops, c, n_sample):
    from mixture_experts_layer_sum_amd.ops import LayerBuffers, moe_layer_forward
    W = mi.layer_weights(c, 0, DEV)
    A = mi.activations(c, DEV)
    buf = LayerBuffers(c.T, c.d, c.E, c.k, c.c, c.shared_width, c.torch_dtype, DEV)
    out = moe_layer_forward(A, W, c.k, c.gate, c.renormalize, buf)
    _sync()
    sample = mi.sample_rows(c.T, n_sample, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 2)).numpy()
    rows = cover_experts(sample, buf.topk_idx.cpu().numpy(), c.E, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 5))
    big = c.E * c.c * c.d > 2 ** 31   # do not keep the expert weights on the host (DeepSeek-V3: 22.5 GB)
    Wo = oracle_weights(W, cache=not big)
    rd = torch.from_numpy(rows).to(DEV)
    x = to_np(A[rd])
    bf = c.dtype == "bf16"
    res = oracle.moe_layer(x, Wo, c.k, c.gate, c.renormalize, c.n_shared, c.c_shared,
                           store=oracle.round_to_bf16 if bf else None)
    keep = oracle.topk_gap(res["logits"], c.k) >= NEAR_TIE
    assert keep.mean() > 0.9
    got = to_np(out[rd])
    # routing of the kept tokens matches exactly
    idx = buf.topk_idx[rd].cpu().numpy()
    np.testing.assert_array_equal(idx[keep], res["topk_idx"][keep])
    routed = np.unique(idx)
    if len(routed) < c.E:   # every expert that the whole batch routes to is reached
        assert set(routed.tolist()) == set(np.unique(buf.topk_idx.cpu().numpy()).tolist())
    r = assert_parity(got[keep], res["out"][keep], c.torch_dtype, f"{c.name}: {len(rows)} tokens, {len(routed)} experts")
    if bf:   # S + R formed in fp32 from bf16-stored S and Y
        dest = res["dest_row"].reshape(len(rows), c.k)
        bound = combine_bound(res["S"], res["Y"], res["topk_w"], dest)
        assert_mirror(got[keep], res["out"][keep], c.name, bound=bound[keep])
    return r


@pytest.mark.parametrize("name,n_sample", [("tiny-fp32", 64), ("dsv2-lite", 256), ("qwen3-30b-a3b", 256),
                                           ("llama4-scout", 128), ("dsv3-decode", 256)])
def test_layer_end_to_end(ops, name, n_sample):
    layer_check(ops, CFG[name], n_sample)


def test_layer_dsv3_full_size_sampled(ops):
    """One DeepSeek-V3-shaped layer at full size (T = 65536): 256 seeded tokens plus tokens added
    until every expert is reached, each expert's weights copied once."""
    layer_check(ops, CFG["dsv3-stack"].scaled(layers=1), 256)
