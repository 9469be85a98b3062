"""GPU parity of farskip_stack_forward (the FarSkip residual stack of MoE sublayers).

- fp32 (tiny dims plus a shared expert, 4 layers): free-running against the oracle, 1e-4 bar, for
  every mode and a mixed skip mask.
- bf16 (mid-size stacks): free-running against the oracle with the implementation's storage
  precision mirrored (expert hidden, expert/shared outputs and layer inputs rounded to bf16), so
  that the routing decisions of layers 2..L see inputs of the same precision.  Tokens whose
  k-th/(k+1)-th logit gap falls below the margin at any layer are excluded: 1e-4 at layer 1
  (identical inputs), 1e-2 at deeper layers, where the two sides' inputs may still differ by one
  bf16 unit in a few elements (estimated logit shift ~2e-3 at d = 7168, so the margin is about
  5 sigma).
- bf16 (DeepSeek-V3-shaped stacks): teacher-forced per layer.  Without normalisation between the
  sublayers the activations grow through depth (|x| ~ 500 and logits ~ 500 by layer 4 with these
  random weights), so a bf16-unit difference between the two sides compounds and a free-running
  comparison flips tokens whose logit gap is far above any fixed margin.  The stack's own layer
  inputs and residuals (from the same ABI calls composed on one stream, asserted bitwise equal to
  the stack) are fed to the oracle one layer at a time; routing, S, R and the FarSkip bookkeeping
  o_j = o_{j-1} + S_j + R_j and x_{j+1} = bf16(o_{j-1} + S_j) are checked at every layer, tokens
  within 1e-4 of a top-k tie excluded.
- properties: two streams == one stream (bitwise), the stack == the same ABI calls composed by
  hand on one stream (bitwise), runs are bitwise repeatable.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.helpers import (NEAR_TIE, ExpertSlices, assert_mirror, assert_parity, bf16_ulp, combine_bound,
                           mirror_bound, oracle_weights, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"
DEEP_MARGIN_BF16 = 1e-2

TINY_STACK = mi.BY_NAME["tiny-fp32"].scaled(cfg_id=10, name="tiny-fp32-stack", n_shared=1, c_shared=256, layers=4)
MID_STACK = mi.MoEConfig(11, "mid-bf16-stack", T=2048, d=512, E=16, k=4, c=256, n_shared=1, c_shared=256,
                         gate="sigmoid", renormalize=True, dtype="bf16", layers=4)
MID_SOFTMAX_2SH = mi.MoEConfig(12, "mid-bf16-softmax-2shared", T=1536, d=256, E=12, k=3, c=192, n_shared=2,
                               c_shared=128, gate="softmax", renormalize=False, dtype="bf16", layers=3,
                               router_bias=True)


@pytest.fixture(scope="module")
def ops():
    from mixture_experts_layer_sum_amd import ops as _ops
    return _ops


def make_stack(c):
    layers = [mi.layer_weights(c, j, DEV) for j in range(c.layers)]
    o0 = mi.activations(c, DEV).float()  # values representable in the workload dtype
    return layers, o0


def run_stack(ops, c, layers, o0, mode, mask=None, two_streams=True, mx_layers=None):
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    oL = torch.full_like(o0, float("nan"))
    sm = torch.cuda.current_stream()
    ss = torch.cuda.Stream() if two_streams else sm
    if mx_layers is not None:
        ws = ops.workspace(ops.stack_mxfp8_workspace_bytes(cfg), DEV)
        ops.farskip_stack_forward_mxfp8(layers, mx_layers, cfg, mode, o0, oL, ws, skip_mask=mask, s_main=sm, s_side=ss)
    else:
        ws = ops.workspace(ops.stack_workspace_bytes(cfg), DEV)
        ops.farskip_stack_forward(layers, cfg, mode, o0, oL, ws, skip_mask=mask, s_main=sm, s_side=ss)
    torch.cuda.synchronize()
    return oL


def oracle_stack(c, layers, o0_rows, mode, mask=None):
    bf = c.dtype == "bf16"
    rnd = oracle.round_to_bf16 if bf else None
    rec = []
    Wo = [oracle_weights(W) for W in layers]
    oL = oracle.moe_stack(o0_rows, Wo, c.k, c.gate, c.renormalize, mode, mask, c.n_shared, c.c_shared,
                          round_inputs=rnd, record=rec, store=rnd)
    keep = np.ones(o0_rows.shape[0], bool)
    for j, (x, _, _, _) in enumerate(rec):
        gap = oracle.topk_gap(oracle.router_logits(x, Wo[j]["W_R"], Wo[j]["bias"]), c.k)
        keep &= gap >= (NEAR_TIE if (j == 0 or not bf) else DEEP_MARGIN_BF16)
    return oL, keep


MODES = [("none", None), ("partial", None), ("outdated", None), ("partial", [1, 0, 1, 1]),
         ("outdated", [0, 1, 1, 0])]


@pytest.mark.parametrize("mode,mask", MODES)
def test_stack_fp32_free_running(ops, mode, mask):
    c = TINY_STACK
    layers, o0 = make_stack(c)
    oL = run_stack(ops, c, layers, o0, mode, mask)
    ref, keep = oracle_stack(c, layers, to_np(o0), mode, mask)
    assert keep.mean() > 0.8
    assert_parity(to_np(oL)[keep], ref[keep], torch.float32, f"fp32 stack {mode} {mask}")


@pytest.mark.parametrize("c", [MID_STACK, MID_SOFTMAX_2SH], ids=lambda c: c.name)
@pytest.mark.parametrize("mode,mask", MODES[:4])
def test_stack_bf16_vs_oracle(ops, c, mode, mask):
    if mask is not None:
        mask = mask[:c.layers]
    layers, o0 = make_stack(c)
    oL = run_stack(ops, c, layers, o0, mode, mask)
    rows = mi.sample_rows(c.T, 384, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE))
    ref, keep = oracle_stack(c, layers, to_np(o0[rows.to(DEV)]), mode, mask)
    assert keep.mean() > 0.5
    assert_parity(to_np(oL[rows.to(DEV)])[keep], ref[keep], torch.bfloat16, f"bf16 stack {mode}")


def test_stack_modes_differ(ops):
    """The three wirings are really different functions (guards against a mode being ignored)."""
    c = MID_STACK
    layers, o0 = make_stack(c)
    outs = [run_stack(ops, c, layers, o0, m) for m in ("none", "partial", "outdated")]
    for a in range(3):
        for b in range(a + 1, 3):
            assert not torch.equal(outs[a], outs[b])


@pytest.mark.parametrize("mode,mask", MODES)
def test_stack_two_streams_equals_one_stream(ops, mode, mask):
    c = MID_STACK
    layers, o0 = make_stack(c)
    a = run_stack(ops, c, layers, o0, mode, mask, two_streams=True)
    b = run_stack(ops, c, layers, o0, mode, mask, two_streams=False)
    assert torch.equal(a, b)
    c2 = run_stack(ops, c, layers, o0, mode, mask, two_streams=True)
    assert torch.equal(a, c2)  # bitwise repeatable


def composed(ops, c, layers, o0, mode, mask, rows=None, record=None, mx_layers=None, keep=None, mx_parts=None):
    """The stack recursion written with the single ABI calls on one stream.  With rows and a record
    list, each layer appends (x_j, o_{j-1}, o_j, topk_idx_j, x_{j+1} or None) for those rows.  With
    a keep list instead, each layer appends the same five tensors for all tokens, on the device.
    With mx_layers, the expert MLPs are moe_grouped_swiglu_mxfp8 on moe_mx_quantize of x_j (routed:
    rows gathered through the permutation; shared: all rows as one group).  With an mx_parts list
    as well, each MLP runs as its two calls (moe_grouped_mxfp8_gate_up, moe_grouped_mxfp8_down; the
    same Y bit for bit) and each layer appends, on the device, the routed H (codes, scales) and Y in
    grouped row order, dest_row, the gate weights, and the shared H and S."""
    from mixture_experts_layer_sum_amd.ops import LayerBuffers
    dt = c.torch_dtype
    buf = LayerBuffers(c.T, c.d, c.E, c.k, c.c, c.shared_width, dt, DEV)
    o_prev = o0.clone()
    x = o0.to(dt)
    L = len(layers)
    for j, W in enumerate(layers):
        ops.moe_route(x, W["W_R"], c.k, c.gate, c.renormalize, buf.logits, buf.topk_idx, buf.topk_w, bias=W["bias"])
        parts = None
        if mx_layers is not None and mx_parts is not None:
            q = mx_layers[j]
            ops.moe_permute(buf.topk_idx, c.E, buf.offsets, buf.sorted_src, buf.dest_row, ws=buf.perm_ws)
            xq = ops.mx_quantized(x)
            N = c.T * c.k
            H = (torch.empty((N, c.c), dtype=torch.uint8, device=DEV),
                 torch.empty((N, c.c // 32), dtype=torch.uint8, device=DEV))
            ops.moe_grouped_mxfp8_gate_up(xq, buf.offsets, q["W1"], q["W2"], H, sorted_src=buf.sorted_src, k=c.k)
            ops.moe_grouped_mxfp8_down(H, buf.offsets, q["W3"], buf.Y)
            parts = {"H": H, "Y": buf.Y.clone(), "dest_row": buf.dest_row.clone(), "w": buf.topk_w.clone()}
        elif mx_layers is not None:
            q = mx_layers[j]
            ops.moe_permute(buf.topk_idx, c.E, buf.offsets, buf.sorted_src, buf.dest_row, ws=buf.perm_ws)
            ops.moe_grouped_swiglu_mxfp8(ops.mx_quantized(x), buf.offsets, q["W1"], q["W2"], q["W3"], buf.Y,
                                         sorted_src=buf.sorted_src, k=c.k)
        else:
            ops.moe_permute(buf.topk_idx, c.E, buf.offsets, buf.sorted_src, buf.dest_row, A=x, A_perm=buf.A_perm,
                            ws=buf.perm_ws)
            ops.moe_grouped_swiglu(buf.A_perm, buf.offsets, W["W1"], W["W2"], W["W3"], buf.Y, ws=buf.gemm_ws)
        S = None
        if c.shared_width:
            if parts is not None:
                q = mx_layers[j]
                Hs = (torch.empty((c.T, c.shared_width), dtype=torch.uint8, device=DEV),
                      torch.empty((c.T, c.shared_width // 32), dtype=torch.uint8, device=DEV))
                ops.moe_grouped_mxfp8_gate_up(ops.mx_quantized(x), buf.shared_off, q["Ws1"], q["Ws2"], Hs)
                ops.moe_grouped_mxfp8_down(Hs, buf.shared_off, q["Ws3"], buf.S)
                parts.update(Hs=Hs, S=buf.S.clone())
            elif mx_layers is not None:
                q = mx_layers[j]
                ops.moe_grouped_swiglu_mxfp8(ops.mx_quantized(x), buf.shared_off, q["Ws1"], q["Ws2"], q["Ws3"], buf.S)
            else:
                ops.moe_grouped_swiglu(x, buf.shared_off, W["Ws1"], W["Ws2"], W["Ws3"], buf.S, ws=buf.shared_ws)
            S = buf.S
        skip = mode != "none" and (mask is None or mask[j])
        x_next = None
        if skip and j + 1 < L:
            x_next = ((o_prev + S.float()) if (mode == "partial" and S is not None) else o_prev).to(dt)
        o_new = torch.empty_like(o_prev)
        ops.moe_combine(buf.Y, buf.topk_w, buf.dest_row, o_new, addend=S, residual=o_prev)
        if not skip and j + 1 < L:
            x_next = o_new.to(dt)
        if record is not None:
            rd = rows.to(DEV)
            record.append((to_np(x[rd]), to_np(o_prev[rd]), to_np(o_new[rd]), buf.topk_idx[rd].cpu().numpy(),
                           None if x_next is None else to_np(x_next[rd])))
        if keep is not None:
            keep.append((x.clone(), o_prev, o_new, buf.topk_idx.clone(), x_next))
        if mx_parts is not None:
            mx_parts.append(parts)
        o_prev, x = o_new, x_next
    torch.cuda.synchronize()
    return o_prev


@pytest.mark.parametrize("c", [MID_STACK, MID_SOFTMAX_2SH, TINY_STACK], ids=lambda c: c.name)
@pytest.mark.parametrize("mode,mask", MODES[:4])
def test_stack_equals_composed_ops(ops, c, mode, mask):
    if mask is not None:
        mask = mask[:c.layers]
    layers, o0 = make_stack(c)
    a = run_stack(ops, c, layers, o0, mode, mask)
    b = composed(ops, c, layers, o0, mode, mask)
    assert torch.equal(a, b)


def cover_rows(n_sample, topk_all, E, seed):
    """A seeded sample of n_sample tokens plus, for every layer and every expert that the sample
    does not reach there, one seeded token routed to it (topk_all: each layer's [T, k] routing)."""
    T = topk_all[0].shape[0]
    rows = set(mi.sample_rows(T, n_sample, seed).numpy().tolist())
    g = np.random.default_rng(seed)
    for idx in topk_all:
        hit = np.zeros(E, bool)
        hit[np.unique(idx[sorted(rows)])] = True
        for e in np.nonzero(~hit)[0]:
            cand = np.nonzero((idx == e).any(axis=1))[0]
            if cand.size:
                t = int(g.choice(cand))
                rows.add(t)
                hit[np.unique(idx[t])] = True
    return torch.from_numpy(np.array(sorted(rows), dtype=np.int64))


@pytest.mark.parametrize("name", ["dsv3-stack", "dsv3-decode"])
def test_stack_dsv3_full_size_sampled(ops, name):
    """The DeepSeek-V3-shaped 4-layer partial stack in the bench launch configuration (two streams),
    for the prefill batch (T = 65536, 256-row tiles) and one decode step (T = 1024, 64-row tiles).
    The stack output equals the composed single calls bitwise.  Then, at every layer, 256 seeded
    tokens plus tokens added until every expert of that layer is reached are checked against the
    oracle on the GPU's own layer inputs (teacher-forced): routing, S + R and the next input, each
    against the max|err| <= 2e-2 max|ref| bar and against the store-mirrored oracle's element-wise bar."""
    c = mi.BY_NAME[name]
    layers, o0 = make_stack(c)
    oL = run_stack(ops, c, layers, o0, "partial")
    assert not torch.isnan(oL).any().item()
    kept = []
    assert torch.equal(oL, composed(ops, c, layers, o0, "partial", None, keep=kept))
    rows = cover_rows(256, [k_[3].cpu().numpy() for k_ in kept], c.E, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 3))
    rd = rows.to(DEV)
    rnd = oracle.round_to_bf16
    for j, W in enumerate(layers):
        x, o_prev, o_new, idx, x_next = (None if t is None else t[rd] for t in kept[j])
        x, o_prev, o_new, idx = to_np(x), to_np(o_prev), to_np(o_new), idx.cpu().numpy()
        x_next = None if x_next is None else to_np(x_next)
        # every expert is fetched once per layer and not kept (22.5 GB per layer)
        Wo = oracle_weights(W, cache=False)
        res = oracle.moe_layer(x, Wo, c.k, c.gate, c.renormalize, c.n_shared, c.c_shared, store=rnd)
        assert len(Wo["W1"].fetched) == c.E or set(np.unique(kept[j][3].cpu().numpy())) == Wo["W1"].fetched
        keep = oracle.topk_gap(res["logits"], c.k) >= NEAR_TIE
        assert keep.sum() >= 240
        np.testing.assert_array_equal(idx[keep], res["topk_idx"][keep])
        what = f"{name} layer {j} ({len(rows)} tokens, {len(Wo['W1'].fetched)} experts)"
        # o_j = o_{j-1} + S_j + R_j, summed in fp32 on the GPU
        got = (o_new.astype(np.float64) - o_prev)[keep]
        assert_parity(got, res["out"][keep], torch.bfloat16, what + " S + R")
        bound = combine_bound(res["S"], res["Y"], res["topk_w"], res["dest_row"].reshape(len(rows), c.k), o_prev)
        assert_mirror(got, res["out"][keep], what + " S + R", bound=bound[keep])
        if x_next is not None:  # partial: x_{j+1} = bf16(o_{j-1} + S_j)
            ref_x = rnd(o_prev + res["S"])
            assert_parity(x_next[keep], ref_x[keep], torch.bfloat16, what + " x_next")
            # one bf16 unit of x, plus S's own bar, plus two fp32 roundings of o_{j-1} + S
            bx = bf16_ulp(ref_x) + mirror_bound(res["S"]) + 2.0 ** -23 * (np.abs(o_prev) + np.abs(res["S"]))
            assert_mirror(x_next[keep], ref_x[keep], what + " x_next", bound=bx[keep])
    del kept


@pytest.mark.parametrize("name,n_sample", [("tiny-fp32", 64), ("dsv2-lite", 128), ("qwen3-30b-a3b", 128),
                                           ("llama4-scout", 64)])
def test_stack_one_layer_each_workload(ops, name, n_sample):
    """One FarSkip layer of each smaller workload at its full size, launched as bench.py times it
    (farskip_stack_forward, L = 1, partial, two streams): bitwise equal to the composed single calls,
    and o_1 - o_0 on seeded tokens against the oracle's layer output (S + R), with exact routing
    away from top-k near-ties."""
    c = mi.BY_NAME[name]
    layers, o0 = make_stack(c)
    oL = run_stack(ops, c, layers, o0, "partial")
    assert not torch.isnan(oL).any().item()
    rows = mi.sample_rows(c.T, n_sample, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 4))
    rec = []
    assert torch.equal(oL, composed(ops, c, layers, o0, "partial", None, rows=rows, record=rec))
    x, o_prev, o_new, idx, x_next = rec[0]
    assert x_next is None
    np.testing.assert_array_equal(x, to_np(o0[rows.to(DEV)]))   # x_1 = o_0 (bf16-valued inputs)
    rnd = oracle.round_to_bf16 if c.dtype == "bf16" else None
    res = oracle.moe_layer(x, oracle_weights(layers[0]), c.k, c.gate, c.renormalize, c.n_shared, c.c_shared,
                           store=rnd)
    keep = oracle.topk_gap(res["logits"], c.k) >= NEAR_TIE
    assert keep.mean() > 0.9
    np.testing.assert_array_equal(idx[keep], res["topk_idx"][keep])
    got = (o_new.astype(np.float64) - o_prev)[keep]
    assert_parity(got, res["out"][keep], c.torch_dtype, f"{name} one-layer stack S + R")
    if rnd is not None:
        bound = combine_bound(res["S"], res["Y"], res["topk_w"], res["dest_row"].reshape(len(x), c.k), o_prev)
        assert_mirror(got, res["out"][keep], f"{name} one-layer stack S + R", bound=bound[keep])


@pytest.mark.parametrize("c,mx", [(TINY_STACK, False), (MID_STACK, False), (MID_STACK, True)],
                         ids=["tiny-fp32-stack", "mid-bf16-stack", "mid-mxfp8-stack"])
def test_stack_graph_replay(ops, c, mx):
    """The two-stream stack (bf16 / fp32, or with MXFP8 expert MLPs) captured into one HIP graph (the
    side stream joins the capture through the call's first event wait and rejoins the main stream
    at its end) and replayed three times, with eager calls and new input values in place between
    the replays: every replay equals the eager call on the same input, bitwise."""
    layers, o0 = make_stack(c)
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    mxl = [ops.layer_mx(W) for W in layers] if mx else None
    nbytes = ops.stack_mxfp8_workspace_bytes(cfg) if mx else ops.stack_workspace_bytes(cfg)
    ws = ops.workspace(nbytes, DEV)
    o_in = o0.clone()
    o_graph = torch.full_like(o0, float("nan"))
    side = torch.cuda.Stream()

    def call(out):
        sm = torch.cuda.current_stream()
        if mx:
            ops.farskip_stack_forward_mxfp8(layers, mxl, cfg, "partial", o_in, out, ws, s_main=sm, s_side=side)
        else:
            ops.farskip_stack_forward(layers, cfg, "partial", o_in, out, ws, s_main=sm, s_side=side)

    call(o_graph)   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        call(o_graph)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(7)
    for r in range(3):
        # new input values (the workload dtype's grid), then the eager reference on a fresh buffer
        o_in.copy_((o0.cpu() * (1.0 + 0.25 * r) + torch.randn(o0.shape, generator=gen) * 0.01)
                   .to(c.torch_dtype).float())
        ref = torch.full_like(o0, float("nan"))
        call(ref)
        torch.cuda.synchronize()
        o_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert not torch.isnan(ref).any().item()
        assert torch.equal(o_graph, ref), f"replay {r}"


@pytest.mark.parametrize("two", [True, False], ids=["two-streams", "one-stream"])
def test_stack_stats_out_parameter(ops, two):
    """farskip_stack_forward's stats: the call blocks, fills per-stream busy times and the overlap of
    its own kernels, leaves the result bitwise unchanged, and records nothing for the process-wide
    profiler.  On one stream there is no side-stream work and no overlap."""
    c = MID_STACK
    layers, o0 = make_stack(c)
    ref = run_stack(ops, c, layers, o0, "partial", two_streams=two)
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.stack_workspace_bytes(cfg), DEV)
    out = torch.full_like(o0, float("nan"))
    sm = torch.cuda.current_stream()
    ss = torch.cuda.Stream() if two else sm
    ops.profile_collect()
    ops.profile_enable(True)
    try:
        st = ops.farskip_stack_forward(layers, cfg, "partial", o0, out, ws, s_main=sm, s_side=ss, stats=True)
    finally:
        ops.profile_enable(False)
    assert sum(n for n, _ in ops.profile_collect().values()) == 0
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    print(f"[stats] {'two' if two else 'one'} stream(s): {st}", flush=True)
    assert st["launches_main"] >= 2 * c.layers
    assert st["main_busy_ms"] > 0 and st["wall_ms"] >= max(st["main_busy_ms"], st["side_busy_ms"]) - 1e-6
    assert 0.0 <= st["overlap_of_side"] <= 1.0 and 0.0 <= st["overlap_of_main"] <= 1.0
    # |M u S| = |M| + |S| - |M n S| cannot exceed the span from the first start to the last end
    assert st["main_busy_ms"] + st["side_busy_ms"] - st["overlap_ms"] <= st["wall_ms"] + 1e-6
    if two:
        assert st["launches_side"] >= 2 * c.layers and st["side_busy_ms"] > 0
    else:
        assert st["launches_side"] == 0 and st["overlap_ms"] == 0.0 and st["side_busy_ms"] == 0.0


def test_profile_intervals_of_a_two_stream_stack(ops):
    """The per-launch intervals behind bench.py's overlap figure: one per recorded launch, on both
    streams, consistent with the per-kind totals of the same collection."""
    c = MID_STACK
    layers, o0 = make_stack(c)
    run_stack(ops, c, layers, o0, "partial")   # warm-up outside the recording
    ops.profile_collect()
    ops.profile_enable(True)
    try:
        run_stack(ops, c, layers, o0, "partial")
    finally:
        ops.profile_enable(False)
    totals, launches = ops.profile_collect_intervals()
    assert len(launches) == sum(n for n, _ in totals.values()) > 0
    assert all(b >= a for _, _, a, b in launches)
    streams = {s for _, s, _, _ in launches}
    assert len(streams) == 2
    main = torch.cuda.current_stream().cuda_stream
    routed = {s for k, s, _, _ in launches if k in ("gemm_gate_up", "gemm_down", "permute_index")}
    assert routed == {main}
    for kind, (n, ms) in totals.items():
        mine = [b - a for k, _, a, b in launches if k == kind]
        assert len(mine) == n
        # both are differences of float event times (about 1 us resolution)
        assert abs(sum(mine) - ms) <= 2e-3 * n + 1e-4 * ms
    # nothing left behind: the next collection is empty
    totals2, launches2 = ops.profile_collect_intervals()
    assert launches2 == [] and all(n == 0 for n, _ in totals2.values())


# ---- the stack with MXFP8 expert MLPs ------------------------------------------------------------


@pytest.mark.parametrize("mode,mask", MODES[:4])
def test_mxfp8_stack_equals_composed_ops_and_one_stream(ops, mode, mask):
    c = MID_STACK
    layers, o0 = make_stack(c)
    mxl = [ops.layer_mx(W) for W in layers]
    a = run_stack(ops, c, layers, o0, mode, mask, mx_layers=mxl)
    assert not torch.isnan(a).any().item()
    assert torch.equal(a, run_stack(ops, c, layers, o0, mode, mask, two_streams=False, mx_layers=mxl))
    assert torch.equal(a, composed(ops, c, layers, o0, mode, mask, mx_layers=mxl))
    assert torch.equal(a, run_stack(ops, c, layers, o0, mode, mask, mx_layers=mxl))  # repeatable


def test_mxfp8_stack_vs_oracle_teacher_forced(ops):
    """Each layer of the MXFP8 stack on 64 seeded tokens, element by element, every stage against the
    MXFP8 oracle on the GPU's own input to that stage (the stack equals the composed calls bitwise,
    and the composed calls run each MLP as its two products, which give the fused call's Y bit for
    bit): selection identical away from near-ties and gate weights to 2e-6; each routed slot's and
    the shared expert's H codes within the reach of the instruction's error (tests/mx_bound.py
    check_hidden); their Y within check_down's bar of the exact product of that H; o_j - o_{j-1}
    within fp32 rounding of S + sum_i w_i Y_i; x_{j+1} = bf16(o_{j-1} + S_j) exactly.  The whole
    MLP's mean error is also held to 2^-8 of the mean |Y| against the oracle's own H."""
    from tests.mx_bound import check_down, check_end_to_end, check_hidden
    c = MID_STACK
    layers, o0 = make_stack(c)
    mxl = [ops.layer_mx(W) for W in layers]
    oL = run_stack(ops, c, layers, o0, "partial", mx_layers=mxl)
    rows = mi.sample_rows(c.T, 64, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 5))
    rn = rows.numpy()
    rec, parts = [], []
    assert torch.equal(oL, composed(ops, c, layers, o0, "partial", None, rows=rows, record=rec, mx_layers=mxl,
                                    mx_parts=parts))
    host = lambda t: t.cpu().numpy()  # noqa: E731
    for j, W in enumerate(layers):
        x, o_prev, o_new, idx, x_next = rec[j]
        p = parts[j]
        W_R = to_np(W["W_R"]).astype(np.float64)
        logits = oracle.router_logits(x, W_R, None if W.get("bias") is None else to_np(W["bias"]).astype(np.float64))
        ref_idx = oracle.select_topk(logits, c.k)
        keep = oracle.topk_gap(logits, c.k) >= NEAR_TIE
        assert keep.sum() >= 48
        np.testing.assert_array_equal(idx[keep], ref_idx[keep])
        w_gpu = host(p["w"])[rn]
        np.testing.assert_allclose(w_gpu[keep], oracle.gate_weights(logits, ref_idx, c.gate, c.renormalize)[keep],
                                   rtol=2e-6, atol=1e-7)
        wq = {n: host_q(mxl[j][n]) for n in ("Ws1", "Ws2", "Ws3")}
        # shared expert: H (rows = tokens) and Y
        Hs = (host(p["Hs"][0])[rn], host(p["Hs"][1])[rn])
        check_hidden(*Hs, x, wq["Ws1"], wq["Ws2"], f"layer {j} shared H")
        S = to_np(p["S"])[rn]
        check_down(S, Hs, wq["Ws3"], f"layer {j} shared Y")
        check_end_to_end(S, x, wq["Ws1"], wq["Ws2"], wq["Ws3"], f"layer {j} shared MLP")
        # routed slots of the kept tokens, expert by expert
        dest = host(p["dest_row"]).reshape(c.T, c.k)[rn]
        Y = to_np(p["Y"])
        Hc, Hsc = host(p["H"][0]), host(p["H"][1])
        for e in np.unique(idx[keep]):
            t_i = np.argwhere((idx == e) & keep[:, None])
            r = dest[t_i[:, 0], t_i[:, 1]]
            q = {n: host_q_expert(mxl[j][n], e) for n in ("W1", "W2", "W3")}
            Hr = (Hc[r], Hsc[r])
            check_hidden(*Hr, x[t_i[:, 0]], q["W1"], q["W2"], f"layer {j} expert {e} H")
            check_down(Y[r], Hr, q["W3"], f"layer {j} expert {e} Y")
            check_end_to_end(Y[r], x[t_i[:, 0]], q["W1"], q["W2"], q["W3"], f"layer {j} expert {e} MLP")
        # the combine on the GPU's own S, Y and w: fp32 sums of k + 2 terms
        got = (o_new.astype(np.float64) - o_prev)[keep]
        ref = S.copy()
        mag = np.abs(S) + np.abs(o_prev)
        for i in range(c.k):
            ref += w_gpu[:, i:i + 1] * Y[dest[:, i]]
            mag += w_gpu[:, i:i + 1] * np.abs(Y[dest[:, i]])
        bound = (c.k + 2) * 2.0 ** -24 * mag
        assert_mirror(got, ref[keep], f"MXFP8 layer {j} o_j - o_(j-1) on the GPU's S, Y, w", bound=bound[keep])
        if x_next is not None:   # x_{j+1} = bf16(o_{j-1} + S_j), formed in fp32
            np.testing.assert_array_equal(x_next, oracle.round_to_bf16((o_prev + S).astype(np.float32)))


def host_q(q):
    return q[0].cpu().numpy(), q[1].cpu().numpy()


def host_q_expert(q, e):
    return q[0][int(e)].cpu().numpy(), q[1][int(e)].cpu().numpy()


@pytest.mark.parametrize("name", ["dsv3-stack", "dsv3-decode"])
def test_mxfp8_stack_dsv3_full_size(ops, name):
    """The DeepSeek-V3-shaped layers (d = 7168, 256 experts, top-8; prefill T = 65536 and a decode
    batch T = 1024) through the MXFP8 stack in the bench launch configuration (two streams, partial
    inputs; two layers here): equal bit for bit to the composed single calls, whose MXFP8 grouped
    product the full-size tests of that call check against the oracle; finite."""
    c = mi.BY_NAME[name].scaled(layers=2)
    layers, o0 = make_stack(c)
    mxl = [ops.layer_mx(W) for W in layers]
    oL = run_stack(ops, c, layers, o0, "partial", mx_layers=mxl)
    assert torch.isfinite(oL).all().item()
    assert torch.equal(oL, composed(ops, c, layers, o0, "partial", None, mx_layers=mxl))


MAX_EK = mi.MoEConfig(14, "max-experts-topk", T=256, d=256, E=1024, k=32, c=128, n_shared=1, c_shared=128,
                      gate="softmax", renormalize=True, dtype="bf16", layers=3)


@pytest.mark.parametrize("mx", [False, True], ids=["bf16", "mxfp8"])
def test_stack_at_the_expert_and_topk_limits(ops, mx):
    """E = 1024 experts and k = 32 (the library's limits) through a 3-layer partial stack: the
    general combine kernel (k outside its fixed-k forms) also forms the next layer's input; the
    stack equals the composed single calls and one stream, bit for bit, bf16 and MXFP8 experts;
    the bf16 layer 0 against the oracle on 32 sampled tokens."""
    c = MAX_EK
    layers, o0 = make_stack(c)
    mxl = [ops.layer_mx(W) for W in layers] if mx else None
    a = run_stack(ops, c, layers, o0, "partial", mx_layers=mxl)
    assert torch.isfinite(a).all().item()
    assert torch.equal(a, run_stack(ops, c, layers, o0, "partial", two_streams=False, mx_layers=mxl))
    rows = mi.sample_rows(c.T, 32, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 7))
    rec = []
    assert torch.equal(a, composed(ops, c, layers, o0, "partial", None, rows=rows, record=rec, mx_layers=mxl))
    if not mx:   # layer 0 against the oracle on the sampled tokens (the bf16 bar, near-ties excluded)
        x, o_prev, o_new, idx, _ = rec[0]
        res = oracle.moe_layer(x, oracle_weights(layers[0]), c.k, c.gate, c.renormalize, c.n_shared, c.c_shared,
                               store=oracle.round_to_bf16)
        keep = oracle.topk_gap(res["logits"], c.k) >= NEAR_TIE
        assert keep.sum() >= 16
        np.testing.assert_array_equal(idx[keep], res["topk_idx"][keep])
        assert_parity((o_new - o_prev)[keep], res["out"][keep], torch.bfloat16, "E=1024 k=32 layer 0")
