"""GPU parity of farskip_attn_moe_stack_forward: layers of an attention sub-block (a dense SwiGLU block
standing in for it) and an MoE sub-block, wired as FSC section 3 gives it (attention input partial,
eq. 8b; MoE input outdated, eq. 8a) or as the standard stream.

- fp32 (tiny dims, shared experts, 4 layers): free-running against the oracle at 1e-4, both modes.
- bf16 (mid-size): free-running against the oracle with the storage precision mirrored, tokens
  near a top-k tie at any layer excluded (as for the MoE-only stack), both modes.
- bitwise: two streams == one stream == the same ABI calls composed on one stream.
- DeepSeek-V3 shapes in the bench launch configuration: the decode batch (T = 1024) teacher-forced
  at every layer on tokens reaching every expert; the prefill batch (T = 65536) equal to the
  composed calls bitwise and teacher-forced at its second layer, the first whose two inputs differ.
"""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle
from tests.helpers import (NEAR_TIE, assert_mirror, assert_parity, bf16_ulp, combine_bound, mirror_bound,
                           oracle_weights, to_np)

pytestmark = pytest.mark.gpu
DEV = "cuda"
DEEP_MARGIN_BF16 = 1e-2

TINY = mi.BY_NAME["tiny-fp32"].scaled(cfg_id=30, name="tiny-fp32-attn", n_shared=1, c_shared=256, layers=4)
MID = mi.MoEConfig(31, "mid-bf16-attn", T=2048, d=512, E=16, k=4, c=256, n_shared=1, c_shared=256,
                   gate="sigmoid", renormalize=True, dtype="bf16", layers=4)
C_ATTN = {"tiny-fp32-attn": 128, "mid-bf16-attn": 256, "dsv3-stack": 2048, "dsv3-decode": 2048}


@pytest.fixture(scope="module")
def ops():
    from mixture_experts_layer_sum_amd import ops as _ops
    return _ops


def make(c):
    layers = [mi.layer_weights(c, j, DEV) for j in range(c.layers)]
    attn = [mi.attn_weights(c, j, C_ATTN[c.name], DEV) for j in range(c.layers)]
    o0 = mi.activations(c, DEV).float()
    return layers, attn, o0


def run(ops, c, layers, attn, o0, mode, two=True):
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.attn_stack_workspace_bytes(cfg, C_ATTN[c.name]), DEV)
    oL = torch.full_like(o0, float("nan"))
    sm = torch.cuda.current_stream()
    ss = torch.cuda.Stream() if two else sm
    ops.farskip_attn_moe_stack_forward(layers, attn, cfg, C_ATTN[c.name], mode, o0, oL, ws, s_main=sm, s_side=ss)
    torch.cuda.synchronize()
    return oL


def oracle_run(c, layers, attn, o0_rows, mode):
    bf = c.dtype == "bf16"
    rnd = oracle.round_to_bf16 if bf else None
    rec = []
    Wo = [oracle_weights(W) for W in layers]
    Wa = [tuple(to_np(a[n]).astype(np.float64) for n in ("Wa1", "Wa2", "Wa3")) for a in attn]
    oL = oracle.attn_moe_layer_stack(o0_rows, Wo, Wa, c.k, c.gate, c.renormalize, mode, c.n_shared, c.c_shared,
                                     round_inputs=rnd, record=rec, store=rnd)
    keep = np.ones(o0_rows.shape[0], bool)
    for j, (a_in, m_in, A, S, R, o) in enumerate(rec):
        gap = oracle.topk_gap(oracle.router_logits(m_in, Wo[j]["W_R"], Wo[j]["bias"]), c.k)
        keep &= gap >= (NEAR_TIE if (j == 0 or not bf) else DEEP_MARGIN_BF16)
    return oL, keep


@pytest.mark.parametrize("mode", ["farskip", "none"])
def test_attn_stack_fp32_free_running(ops, mode):
    c = TINY
    layers, attn, o0 = make(c)
    oL = run(ops, c, layers, attn, o0, mode)
    ref, keep = oracle_run(c, layers, attn, to_np(o0), mode)
    assert keep.mean() > 0.8
    assert_parity(to_np(oL)[keep], ref[keep], torch.float32, f"fp32 attention stack {mode}")


@pytest.mark.parametrize("mode", ["farskip", "none"])
def test_attn_stack_bf16_vs_oracle(ops, mode):
    c = MID
    layers, attn, o0 = make(c)
    oL = run(ops, c, layers, attn, o0, mode)
    rows = mi.sample_rows(c.T, 384, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE))
    ref, keep = oracle_run(c, layers, attn, to_np(o0[rows.to(DEV)]), mode)
    assert keep.mean() > 0.5
    assert_parity(to_np(oL[rows.to(DEV)])[keep], ref[keep], torch.bfloat16, f"bf16 attention stack {mode}")


def test_attn_stack_modes_differ_and_equal_without_attention(ops):
    """The two wirings are different functions; with every attention output zero (Wa3 = 0) the
    paper wiring's MoE input is the full residual, so it equals the standard MoE-only stack."""
    c = MID
    layers, attn, o0 = make(c)
    a = run(ops, c, layers, attn, o0, "farskip")
    b = run(ops, c, layers, attn, o0, "none")
    assert not torch.equal(a, b)
    zero = [dict(x, Wa3=torch.zeros_like(x["Wa3"])) for x in attn]
    z = run(ops, c, layers, zero, o0, "farskip")
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.stack_workspace_bytes(cfg), DEV)
    ref = torch.empty_like(o0)
    ops.farskip_stack_forward(layers, cfg, "none", o0, ref, ws)
    torch.cuda.synchronize()
    # same routing and experts; the combine adds S in one step here, in two steps there
    r = torch.max(torch.abs(z - ref)).item() / torch.max(torch.abs(ref)).item()
    assert r < 1e-5, r


def composed(ops, c, layers, attn, o0, mode, keep=None):
    """The attention + MoE recursion written with the single ABI calls on one stream, the partial
    residual formed with torch adds in the kernel's order ((o + A) + S).  keep: each layer appends
    (attn_in, mlp_in, o_{j-1}, o_j, topk_idx) for all tokens, on the device."""
    from mixture_experts_layer_sum_amd.ops import LayerBuffers
    dt = c.torch_dtype
    ca = C_ATTN[c.name]
    buf = LayerBuffers(c.T, c.d, c.E, c.k, c.c, c.shared_width, dt, DEV)
    aws = ops.workspace(ops.grouped_swiglu_workspace_bytes(c.T, 1, ca, dt), DEV)
    A = torch.empty((c.T, c.d), dtype=dt, device=DEV)
    o_prev = o0.clone()
    partial = o0.clone()
    for j, W in enumerate(layers):
        a_in = (partial if mode == "farskip" else o_prev).to(dt)
        ops.moe_grouped_swiglu(a_in, buf.shared_off, attn[j]["Wa1"], attn[j]["Wa2"], attn[j]["Wa3"], A, ws=aws)
        m32 = o_prev if mode == "farskip" else o_prev + A.float()
        m_in = m32.to(dt)
        ops.moe_route(m_in, W["W_R"], c.k, c.gate, c.renormalize, buf.logits, buf.topk_idx, buf.topk_w, bias=W["bias"])
        ops.moe_permute(buf.topk_idx, c.E, buf.offsets, buf.sorted_src, buf.dest_row, A=m_in, A_perm=buf.A_perm,
                        ws=buf.perm_ws)
        ops.moe_grouped_swiglu(buf.A_perm, buf.offsets, W["W1"], W["W2"], W["W3"], buf.Y, ws=buf.gemm_ws)
        ops.moe_grouped_swiglu(m_in, buf.shared_off, W["Ws1"], W["Ws2"], W["Ws3"], buf.S, ws=buf.shared_ws)
        o_new = torch.empty_like(o_prev)
        if mode == "farskip":
            partial = (o_prev + A.float()) + buf.S.float()
            ops.moe_combine(buf.Y, buf.topk_w, buf.dest_row, o_new, residual=partial)
        else:
            ops.moe_combine(buf.Y, buf.topk_w, buf.dest_row, o_new, addend=buf.S, residual=m32)
        if keep is not None:
            keep.append((a_in.clone(), m_in.clone(), o_prev, o_new, buf.topk_idx.clone()))
        o_prev = o_new
    torch.cuda.synchronize()
    return o_prev


@pytest.mark.parametrize("mode", ["farskip", "none"])
@pytest.mark.parametrize("c", [TINY, MID], ids=lambda c: c.name)
def test_attn_stack_equals_composed_and_one_stream(ops, c, mode):
    layers, attn, o0 = make(c)
    a = run(ops, c, layers, attn, o0, mode, two=True)
    b = run(ops, c, layers, attn, o0, mode, two=False)
    assert torch.equal(a, b)
    assert torch.equal(a, composed(ops, c, layers, attn, o0, mode))
    assert torch.equal(a, run(ops, c, layers, attn, o0, mode, two=True))   # repeatable


def test_attn_stack_stats(ops):
    c = MID
    layers, attn, o0 = make(c)
    ref = run(ops, c, layers, attn, o0, "farskip")
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.attn_stack_workspace_bytes(cfg, C_ATTN[c.name]), DEV)
    out = torch.empty_like(o0)
    st = ops.farskip_attn_moe_stack_forward(layers, attn, cfg, C_ATTN[c.name], "farskip", o0, out, ws,
                                            s_main=torch.cuda.current_stream(), s_side=torch.cuda.Stream(), stats=True)
    assert torch.equal(out, ref)
    assert st["launches_main"] >= 2 * c.layers and st["launches_side"] >= 4 * c.layers
    assert 0.0 <= st["overlap_of_side"] <= 1.0


def check_layers(c, layers, attn, kept, rows, which):
    """Teacher-forced per layer: the oracle's sub-blocks on the GPU's own inputs for `rows`."""
    rnd = oracle.round_to_bf16
    rd = rows.to(DEV)
    for j in which:
        a_in, m_in, o_prev, o_new, idx = kept[j]
        a_in, m_in, o_prev, o_new = to_np(a_in[rd]), to_np(m_in[rd]), to_np(o_prev[rd]), to_np(o_new[rd])
        idx = idx[rd].cpu().numpy()
        Wo = oracle_weights(layers[j], cache=False)
        Wa = tuple(to_np(attn[j][n]).astype(np.float64) for n in ("Wa1", "Wa2", "Wa3"))
        A = oracle.mlp(a_in, *Wa, store=rnd)
        res = oracle.moe_layer(m_in, Wo, c.k, c.gate, c.renormalize, c.n_shared, c.c_shared, store=rnd)
        keep = oracle.topk_gap(res["logits"], c.k) >= NEAR_TIE
        assert keep.mean() > 0.9
        np.testing.assert_array_equal(idx[keep], res["topk_idx"][keep])
        what = f"{c.name} attention stack layer {j} ({len(rows)} tokens, {len(Wo['W1'].fetched)} experts)"
        got = (o_new.astype(np.float64) - o_prev)[keep]
        ref = (A + res["out"])[keep]
        assert_parity(got, ref, torch.bfloat16, what + " attn + S + R")
        bound = combine_bound(res["S"], res["Y"], res["topk_w"], res["dest_row"].reshape(len(rows), c.k), o_prev)
        bound = bound + mirror_bound(A) + 2.0 ** -24 * np.abs(A)
        assert_mirror(got, ref, what + " attn + S + R", bound=bound[keep])
        if j + 1 < len(kept):   # the next layer's inputs follow the wiring
            a_next, m_next = to_np(kept[j + 1][0][rd]), to_np(kept[j + 1][1][rd])
            np.testing.assert_array_equal(m_next, rnd(o_new))                 # mlp-in = o_j
            ref_a = rnd(o_prev + A + res["S"])                                # attn-in = o_{j-1} + A_j + S_j
            bx = bf16_ulp(ref_a) + mirror_bound(A) + mirror_bound(res["S"]) + \
                2.0 ** -22 * (np.abs(o_prev) + np.abs(A) + np.abs(res["S"]))
            assert_mirror(a_next[keep], ref_a[keep], what + " next attention input", bound=bx[keep])


def test_attn_stack_dsv3_decode_teacher_forced(ops):
    """One decode step (T = 1024) of the DeepSeek-V3-shaped 4-layer attention + MoE stack, two
    streams: equal to the composed calls bitwise, then every layer against the oracle on 256 seeded
    tokens plus tokens added until every expert of that layer is reached."""
    from tests.test_gpu_stack import cover_rows
    c = mi.BY_NAME["dsv3-decode"]
    layers, attn, o0 = make(c)
    oL = run(ops, c, layers, attn, o0, "farskip")
    kept = []
    assert torch.equal(oL, composed(ops, c, layers, attn, o0, "farskip", keep=kept))
    rows = cover_rows(256, [k_[4].cpu().numpy() for k_ in kept], c.E, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 8))
    check_layers(c, layers, attn, kept, rows, range(c.layers))


def test_attn_stack_dsv3_prefill(ops):
    """The prefill batch (T = 65536) in the bench launch configuration: equal to the composed calls
    bitwise; the second layer (whose attention and MoE inputs differ) teacher-forced on 32 tokens."""
    c = mi.BY_NAME["dsv3-stack"]
    layers, attn, o0 = make(c)
    oL = run(ops, c, layers, attn, o0, "farskip")
    assert not torch.isnan(oL).any().item()
    kept = []
    assert torch.equal(oL, composed(ops, c, layers, attn, o0, "farskip", keep=kept))
    rows = mi.sample_rows(c.T, 32, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 9))
    check_layers(c, layers, attn, kept, rows, [1])
