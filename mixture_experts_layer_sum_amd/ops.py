"""Python binding of libfarskip_moe: argument marshalling from torch tensors to the C ABI.

Every function takes device tensors that the caller allocated (outputs included) and enqueues the
work on a HIP stream (default: torch's current stream).  Nothing here computes; each step runs in
the library's HIP kernels.  Names and argument order follow include/farskip_moe.h.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import torch

from ._lib import (FARSKIP_NONE, FARSKIP_OUTDATED, FARSKIP_PAPER, FARSKIP_PARTIAL, KERNEL_KINDS, AttnDesc, MOE_BF16, MOE_F32,
                   MOE_GATE_SIGMOID, MOE_GATE_SOFTMAX, MOE_OPS, KernelInterval, KernelTime, LayerDesc, LayerMx,
                   LayerGrads, StackCfg, StackStats, check, lib)

GATES = {"softmax": MOE_GATE_SOFTMAX, "sigmoid": MOE_GATE_SIGMOID}
MODES = {"none": FARSKIP_NONE, "partial": FARSKIP_PARTIAL, "outdated": FARSKIP_OUTDATED, "farskip": FARSKIP_PAPER}


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MOE_F32
    if dt == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _s(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _gate(g) -> int:
    return GATES[g] if isinstance(g, str) else int(g)


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------------------------
def moe_route(A, W_R, k: int, gate, renormalize: bool, logits, topk_idx, topk_w, bias=None, stream=None):
    """logits = A W_R^T (+ bias); topk_idx / topk_w = top-k selection and gate weights."""
    T, d = A.shape
    E = W_R.shape[0]
    check("moe_route", lib.moe_route(_p(A), _p(W_R), _p(bias), dtype_code(A.dtype), T, d, E, k, _gate(gate),
                                     int(bool(renormalize)), _p(logits), _p(topk_idx), _p(topk_w), _s(stream)))


def moe_route_from_logits(logits, k: int, gate, renormalize: bool, topk_idx, topk_w, stream=None):
    """Selection and weights only, from given fp32 logits [T, E]."""
    T, E = logits.shape
    check("moe_route", lib.moe_route(None, None, None, MOE_F32, T, 0, E, k, _gate(gate), int(bool(renormalize)),
                                     _p(logits), _p(topk_idx), _p(topk_w), _s(stream)))


def permute_workspace_bytes(T: int, E: int, k: int) -> int:
    return int(lib.moe_permute_workspace_bytes(T, E, k))


def moe_permute(topk_idx, E: int, expert_offsets, sorted_src, dest_row, A=None, A_perm=None, ws=None,
                stream=None):
    T, k = topk_idx.shape
    if ws is None:
        ws = workspace(permute_workspace_bytes(T, E, k), topk_idx.device)
    d = A.shape[1] if A is not None else 0
    dt = dtype_code(A.dtype) if A is not None else MOE_F32
    check("moe_permute", lib.moe_permute(_p(A), dt, T, d, E, k, _p(topk_idx), _p(expert_offsets), _p(sorted_src),
                                         _p(dest_row), _p(A_perm), _p(ws), ws.numel(), _s(stream)))


def moe_permute_noalloc(topk_idx, E: int, expert_offsets, sorted_src, dest_row, A=None, A_perm=None, stream=None):
    """moe_permute without a workspace: the library's fixed device scratch holds the counts (for
    callers that cannot allocate; calls that may overlap on one GPU race)."""
    T, k = topk_idx.shape
    d = A.shape[1] if A is not None else 0
    dt = dtype_code(A.dtype) if A is not None else MOE_BF16
    check("moe_permute_noalloc", lib.moe_permute_noalloc(_p(A), dt, T, d, E, k, _p(topk_idx), _p(expert_offsets),
                                                         _p(sorted_src), _p(dest_row), _p(A_perm), _s(stream)))


def grouped_swiglu_workspace_bytes(N: int, G: int, c: int, dtype) -> int:
    return int(lib.moe_grouped_swiglu_workspace_bytes(N, G, c, dtype_code(dtype)))


def moe_grouped_swiglu(X, group_offsets, W1, W2, W3, Y, ws=None, stream=None):
    """Y[rows of group g] = ((X W1[g]^T) . SiLU(X W2[g]^T)) W3[g]^T.  W1/W2: [G,c,d] (or [c,d] for
    one group), W3: [G,d,c] (or [d,c])."""
    N, d = X.shape
    G = group_offsets.numel() - 1
    c = W1.shape[-2]
    if ws is None:
        ws = workspace(grouped_swiglu_workspace_bytes(N, G, c, X.dtype), X.device)
    check("moe_grouped_swiglu",
          lib.moe_grouped_swiglu(_p(X), _p(group_offsets), G, _p(W1), _p(W2), _p(W3), dtype_code(X.dtype), N, d, c,
                                 _p(Y), _p(ws), ws.numel(), _s(stream)))


def moe_grouped_swiglu_gathered(X, sorted_src, k: int, group_offsets, W1, W2, W3, Y, ws=None, stream=None):
    """moe_grouped_swiglu on the rows X[sorted_src[r] // k] without materialising them."""
    T, d = X.shape
    N = sorted_src.numel()
    G = group_offsets.numel() - 1
    c = W1.shape[-2]
    if ws is None:
        ws = workspace(grouped_swiglu_workspace_bytes(N, G, c, X.dtype), X.device)
    check("moe_grouped_swiglu_gathered",
          lib.moe_grouped_swiglu_gathered(_p(X), T, _p(sorted_src), k, _p(group_offsets), G, _p(W1), _p(W2), _p(W3),
                                          dtype_code(X.dtype), N, d, c, _p(Y), _p(ws), ws.numel(), _s(stream)))


def moe_mx_quantize(X, codes, scales, stream=None):
    """MXFP8 of the rows of bf16 X [R, K]: codes [R, K] uint8 (E4M3), scales [R, K/32] uint8 (E8M0)."""
    if X.dtype != torch.bfloat16:
        raise TypeError("moe_mx_quantize takes bf16 input")
    K = X.shape[-1]
    R = X.numel() // K if K else 0
    check("moe_mx_quantize", lib.moe_mx_quantize(_p(X), R, K, _p(codes), _p(scales), _s(stream)))


def mx_quantized(X, stream=None):
    """(codes, scales) of bf16 X [..., K], allocated here (quantised along the last dimension)."""
    codes = torch.empty(X.shape, dtype=torch.uint8, device=X.device)
    scales = torch.empty(X.shape[:-1] + (X.shape[-1] // 32,), dtype=torch.uint8, device=X.device)
    moe_mx_quantize(X, codes, scales, stream)
    return codes, scales


def grouped_swiglu_mxfp8_workspace_bytes(N: int, G: int, c: int) -> int:
    return int(lib.moe_grouped_swiglu_mxfp8_workspace_bytes(N, G, c))


def moe_grouped_swiglu_mxfp8(Xq, group_offsets, W1q, W2q, W3q, Y, sorted_src=None, k: int = 1, ws=None,
                             stream=None):
    """moe_grouped_swiglu on MXFP8 operands.  Xq and W*q are (codes, scales) pairs; W1/W2 codes
    [G, c, d], W3 codes [G, d, c]; Y [N, d] bf16.  With sorted_src, grouped row r is Xq row
    sorted_src[r] // k."""
    x_rows, d = Xq[0].shape
    N = Y.shape[0]
    G = group_offsets.numel() - 1
    c = W1q[0].shape[-2]
    if ws is None:
        ws = workspace(grouped_swiglu_mxfp8_workspace_bytes(N, G, c), Y.device)
    check("moe_grouped_swiglu_mxfp8",
          lib.moe_grouped_swiglu_mxfp8(_p(Xq[0]), _p(Xq[1]), x_rows, _p(sorted_src), k, _p(group_offsets), G,
                                       _p(W1q[0]), _p(W1q[1]), _p(W2q[0]), _p(W2q[1]), _p(W3q[0]), _p(W3q[1]), N,
                                       d, c, _p(Y), _p(ws), ws.numel(), _s(stream)))


def grouped_mxfp8_phase_workspace_bytes(N: int, G: int) -> int:
    return int(lib.moe_grouped_mxfp8_phase_workspace_bytes(N, G))


def moe_grouped_mxfp8_gate_up(Xq, group_offsets, W1q, W2q, H, sorted_src=None, k: int = 1, ws=None, stream=None):
    """Phase 1 alone: H = (codes [N, c], scales [N, c/32]) of (X W1^T) . SiLU(X W2^T) per group."""
    x_rows, d = Xq[0].shape
    N, c = H[0].shape
    G = group_offsets.numel() - 1
    if ws is None:
        ws = workspace(grouped_mxfp8_phase_workspace_bytes(N, G), H[0].device)
    check("moe_grouped_mxfp8_gate_up",
          lib.moe_grouped_mxfp8_gate_up(_p(Xq[0]), _p(Xq[1]), x_rows, _p(sorted_src), k, _p(group_offsets), G,
                                        _p(W1q[0]), _p(W1q[1]), _p(W2q[0]), _p(W2q[1]), N, d, c, _p(H[0]), _p(H[1]),
                                        _p(ws), ws.numel(), _s(stream)))


def moe_grouped_mxfp8_down(H, group_offsets, W3q, Y, ws=None, stream=None):
    """Phase 2 alone: Y [N, d] bf16 = H W3[g]^T per group, H = (codes, scales)."""
    N, c = H[0].shape
    d = Y.shape[1]
    G = group_offsets.numel() - 1
    if ws is None:
        ws = workspace(grouped_mxfp8_phase_workspace_bytes(N, G), Y.device)
    check("moe_grouped_mxfp8_down",
          lib.moe_grouped_mxfp8_down(_p(H[0]), _p(H[1]), _p(group_offsets), G, _p(W3q[0]), _p(W3q[1]), N, c, d,
                                     _p(Y), _p(ws), ws.numel(), _s(stream)))


def moe_combine(Y, topk_w, dest_row, out, addend=None, residual=None, out_x=None, stream=None):
    """out = residual + addend + sum_i topk_w[:, i] * Y[dest_row[t*k+i]]  (fp32)."""
    T, k = topk_w.shape
    d = Y.shape[1]
    check("moe_combine", lib.moe_combine(_p(Y), dtype_code(Y.dtype), _p(topk_w), _p(dest_row), T, d, k, _p(addend),
                                         _p(residual), _p(out), _p(out_x), _s(stream)))


# ---------------------------------------------------------------------------------------------
def stack_cfg(T, d, c, c_shared, E, k, gate, renormalize, dtype) -> StackCfg:
    return StackCfg(T=T, d=d, c=c, c_shared=c_shared, E=E, k=k, gate=_gate(gate),
                    renormalize=int(bool(renormalize)), dtype=dtype_code(dtype) if isinstance(dtype, torch.dtype)
                    else int(dtype))


def stack_workspace_bytes(cfg: StackCfg) -> int:
    return int(lib.farskip_stack_workspace_bytes(ctypes.byref(cfg)))


def layer_desc(W: dict, experts: bool = True) -> LayerDesc:
    """Device-pointer descriptor of one layer; experts=False leaves the expert weights W1-W3 and
    Ws1-Ws3 out (the MXFP8 stack takes them quantised)."""
    rp = lambda name: W[name].data_ptr() if experts and W.get(name) is not None else None  # noqa: E731
    return LayerDesc(W_R=W["W_R"].data_ptr(), bias=W["bias"].data_ptr() if W.get("bias") is not None else None,
                     W1=rp("W1"), W2=rp("W2"), W3=rp("W3"), Ws1=rp("Ws1"), Ws2=rp("Ws2"), Ws3=rp("Ws3"))


def stack_mxfp8_workspace_bytes(cfg: StackCfg) -> int:
    return int(lib.farskip_stack_mxfp8_workspace_bytes(ctypes.byref(cfg)))


def layer_mx(W: dict) -> dict:
    """MXFP8 (codes, scales) of one layer's expert weights: routed W1, W2 [E, c, d], W3 [E, d, c] and,
    when present, shared Ws1, Ws2 [c_shared, d], Ws3 [d, c_shared] (each along its last dimension)."""
    return {name: mx_quantized(W[name]) for name in ("W1", "W2", "W3", "Ws1", "Ws2", "Ws3")
            if W.get(name) is not None}


def _stats_dict(st: StackStats) -> dict:
    return {name: getattr(st, name) for name, _ in StackStats._fields_}


def farskip_stack_forward_mxfp8(layers: Sequence[dict], mx_layers: Sequence[dict], cfg: StackCfg, mode, o0, oL, ws,
                                skip_mask=None, s_main=None, s_side=None, stats: bool = False):
    """farskip_stack_forward with the routed experts on MXFP8 operands; mx_layers[j] as layer_mx()."""
    L = len(layers)
    if len(mx_layers) != L:
        raise ValueError("one MXFP8 expert set per layer is required")
    descs = (LayerDesc * L)(*[layer_desc(W, experts=False) for W in layers])
    def mx_desc(q):
        f = {}
        for name in ("W1", "W2", "W3", "Ws1", "Ws2", "Ws3"):
            f[name + "q"], f[name + "s"] = (q[name][0].data_ptr(), q[name][1].data_ptr()) if name in q else (None, None)
        return LayerMx(**f)

    mxd = (LayerMx * L)(*[mx_desc(q) for q in mx_layers])
    mask = None
    if skip_mask is not None:
        mask = (ctypes.c_uint8 * L)(*[1 if m else 0 for m in skip_mask])
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    sm = _s(s_main)
    ss = _s(s_side) if s_side is not None else sm
    st = StackStats() if stats else None
    check("farskip_stack_forward_mxfp8",
          lib.farskip_stack_forward_mxfp8(descs, mxd, L, ctypes.byref(cfg), m, mask, _p(o0), _p(oL), _p(ws), ws.numel(),
                                          sm, ss, ctypes.byref(st) if stats else None))
    return _stats_dict(st) if stats else None


def farskip_stack_forward(layers: Sequence[dict], cfg: StackCfg, mode, o0, oL, ws, skip_mask=None,
                          s_main=None, s_side=None, stats: bool = False):
    """o_L of the FarSkip stack (mode "none" | "partial" | "outdated").  s_side defaults to s_main.
    stats=True: the call blocks until the stack is done and returns the library's per-stream kernel
    timing (moe_stack_stats_t as a dict); otherwise it is asynchronous and returns None."""
    L = len(layers)
    descs = (LayerDesc * L)(*[layer_desc(W) for W in layers])
    mask = None
    if skip_mask is not None:
        mask = (ctypes.c_uint8 * L)(*[1 if m else 0 for m in skip_mask])
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    sm = _s(s_main)
    ss = _s(s_side) if s_side is not None else sm
    st = StackStats() if stats else None
    check("farskip_stack_forward",
          lib.farskip_stack_forward(descs, L, ctypes.byref(cfg), m, mask, _p(o0), _p(oL), _p(ws), ws.numel(), sm, ss,
                                    ctypes.byref(st) if stats else None))
    return _stats_dict(st) if stats else None


def attn_stack_workspace_bytes(cfg: StackCfg, c_attn: int) -> int:
    return int(lib.farskip_attn_moe_stack_workspace_bytes(ctypes.byref(cfg), c_attn))


def farskip_attn_moe_stack_forward(layers: Sequence[dict], attn: Sequence[dict], cfg: StackCfg, c_attn: int, mode,
                                   o0, oL, ws, s_main=None, s_side=None, stats: bool = False):
    """o_L of the attention + MoE stack (mode "farskip": attention input partial, MoE input outdated;
    "none": the standard stream).  attn[j]: the layer's attention stand-in weights Wa1, Wa2, Wa3."""
    L = len(layers)
    if len(attn) != L:
        raise ValueError("one attention block per layer is required")
    descs = (LayerDesc * L)(*[layer_desc(W) for W in layers])
    ad = (AttnDesc * L)(*[AttnDesc(Wa1=a["Wa1"].data_ptr(), Wa2=a["Wa2"].data_ptr(), Wa3=a["Wa3"].data_ptr())
                          for a in attn])
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    sm = _s(s_main)
    ss = _s(s_side) if s_side is not None else sm
    st = StackStats() if stats else None
    check("farskip_attn_moe_stack_forward",
          lib.farskip_attn_moe_stack_forward(descs, ad, L, ctypes.byref(cfg), c_attn, m, _p(o0), _p(oL), _p(ws),
                                             ws.numel(), sm, ss, ctypes.byref(st) if stats else None))
    return _stats_dict(st) if stats else None


def workspace_bytes(op: str, T: int, d: int, E: int, k: int, c: int, L: int = 1, c_shared: int = 0,
                    dtype=torch.bfloat16) -> int:
    """moe_workspace_bytes: scratch bytes of the call named by op (a key of MOE_OPS)."""
    return int(lib.moe_workspace_bytes(MOE_OPS[op], T, d, E, k, c, L, c_shared,
                                       dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype)))


def layer_backward_workspace_bytes(cfg: StackCfg) -> int:
    return int(lib.moe_layer_backward_workspace_bytes(ctypes.byref(cfg)))


GRAD_NAMES = ("dA", "dW_R", "dbias", "dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3")


def _grads(grads: dict) -> LayerGrads:
    return LayerGrads(*[None if grads.get(n) is None else grads[n].data_ptr() for n in GRAD_NAMES])


def moe_layer_backward(W: dict, cfg: StackCfg, A, logits, topk_idx, topk_w, expert_offsets, sorted_src, dest_row, Y,
                       dOut, grads: dict, ws=None, stream=None, dOut_shared=None):
    """Gradients of one MoE sublayer's output for dOut (float32 [T, d]) into the float32 tensors of
    grads (keys as GRAD_NAMES; dbias and the shared ones may be absent).  dOut_shared: the shared
    experts' own output gradient (default dOut)."""
    if ws is None:
        ws = workspace(layer_backward_workspace_bytes(cfg), A.device)
    check("moe_layer_backward",
          lib.moe_layer_backward(ctypes.byref(layer_desc(W)), ctypes.byref(cfg), _p(A), _p(logits), _p(topk_idx),
                                 _p(topk_w), _p(expert_offsets), _p(sorted_src), _p(dest_row), _p(Y), _p(dOut),
                                 _p(dOut_shared), ctypes.byref(_grads(grads)), _p(ws), ws.numel(), _s(stream)))


def stack_backward_workspace_bytes(cfg: StackCfg, L: int) -> int:
    return int(lib.farskip_stack_backward_workspace_bytes(ctypes.byref(cfg), L))


def farskip_stack_backward(layers: Sequence[dict], cfg: StackCfg, mode, o0, dOL, dO0, grads: Sequence[dict], ws=None,
                           skip_mask=None, stream=None):
    """dO0 = dLoss/do_0 and each layer's gradients (grads[j] as for moe_layer_backward; its dA, if
    given, receives dLoss/dx_j) of the FarSkip stack for dOL = dLoss/do_L."""
    L = len(layers)
    descs = (LayerDesc * L)(*[layer_desc(W) for W in layers])
    gs = (LayerGrads * L)(*[_grads(g) for g in grads])
    mask = None
    if skip_mask is not None:
        mask = (ctypes.c_uint8 * L)(*[1 if m else 0 for m in skip_mask])
    if ws is None:
        ws = workspace(stack_backward_workspace_bytes(cfg, L), o0.device)
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    check("farskip_stack_backward",
          lib.farskip_stack_backward(descs, L, ctypes.byref(cfg), m, mask, _p(o0), _p(dOL), _p(dO0), gs, _p(ws),
                                     ws.numel(), _s(stream)))


def mfma_ceiling(shape: int, out, iters: int, stream=None) -> None:
    """Diagnostic: one register-only MFMA launch (shape 0 = 16x16x32, 1 = 32x32x16 bf16, 2 = scaled
    fp8 16x16x128) of out.numel() // 512 workgroups; FLOP = workgroups * 8 * iters * 262144 for the
    bf16 shapes, * 1048576 for the fp8 one."""
    check("moe_mfma_ceiling", lib.moe_mfma_ceiling(int(shape), int(iters), out.numel() // 512, _p(out), _s(stream)))


def delivery_probe(hot_pct: int, cold_bytes: int, iters: int, in_flight: int, buf, out, clocks=None,
                   stream=None) -> None:
    """Diagnostic: one operand-delivery launch of out.numel() // 512 workgroups, each moving `iters`
    64 KiB stages into LDS with hot_pct percent of its 1 KiB runs from an L2-resident window and
    the rest from its own cold region of cold_bytes in buf; bytes = workgroups * iters * 65536.
    clocks (2 int64 on the device, or None): workgroup 0's loop in shader cycles and in 100 MHz ticks."""
    check("moe_delivery_probe", lib.moe_delivery_probe(int(hot_pct), int(cold_bytes), int(iters), int(in_flight),
                                                       out.numel() // 512, _p(buf), buf.numel() * buf.element_size(),
                                                       _p(out), _p(clocks) if clocks is not None else None,
                                                       _s(stream)))


def profile_enable(on: bool = True) -> None:
    """Start/stop timing every library kernel launch with HIP events on its own stream."""
    check("moe_profile_enable", lib.moe_profile_enable(int(bool(on))))


def profile_collect() -> dict:
    """Wait for the recorded events; {kind: (launches, summed ms)} since the last collect."""
    out = (KernelTime * len(KERNEL_KINDS))()
    check("moe_profile_collect", lib.moe_profile_collect(out))
    return {name: (out[i].count, out[i].total_ms) for i, name in enumerate(KERNEL_KINDS)}


def profile_collect_intervals(cap: int = 16384):
    """profile_collect, plus every recorded launch as (kind, stream id, start ms, end ms) on one time
    axis (the first recorded launch's start event is 0)."""
    out = (KernelTime * len(KERNEL_KINDS))()
    iv = (KernelInterval * cap)()
    n = ctypes.c_int32(0)
    check("moe_profile_collect_intervals", lib.moe_profile_collect_intervals(out, iv, cap, ctypes.byref(n)))
    totals = {name: (out[i].count, out[i].total_ms) for i, name in enumerate(KERNEL_KINDS)}
    launches = [(KERNEL_KINDS[r.kind] if 0 <= r.kind < len(KERNEL_KINDS) else str(r.kind), int(r.stream),
                 r.start_ms, r.end_ms) for r in iv[:min(n.value, cap)]]
    return totals, launches


# ---------------------------------------------------------------------------------------------
class LayerBuffers:
    """Preallocated device buffers for one MoE sublayer forward (so a timed loop allocates nothing)."""

    def __init__(self, T, d, E, k, c, c_shared, dtype, device):
        N = T * k
        self.logits = torch.empty((T, E), dtype=torch.float32, device=device)
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=device)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=device)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=device)
        self.sorted_src = torch.empty((N,), dtype=torch.int32, device=device)
        self.dest_row = torch.empty((N,), dtype=torch.int32, device=device)
        self.A_perm = torch.empty((N, d), dtype=dtype, device=device)
        self.Y = torch.empty((N, d), dtype=dtype, device=device)
        self.perm_ws = workspace(permute_workspace_bytes(T, E, k), device)
        self.gemm_ws = workspace(grouped_swiglu_workspace_bytes(N, E, c, dtype), device)
        self.S = torch.empty((T, d), dtype=dtype, device=device) if c_shared else None
        self.shared_off = torch.tensor([0, T], dtype=torch.int32, device=device)
        self.shared_ws = workspace(grouped_swiglu_workspace_bytes(T, 1, c_shared, dtype), device) if c_shared else None
        self.out = torch.empty((T, d), dtype=torch.float32, device=device)


def moe_layer_forward(A, W: dict, k: int, gate, renormalize: bool, buf: LayerBuffers, residual=None,
                      stream=None):
    """One MoE sublayer: route, permute, routed grouped SwiGLU, shared expert, combine.
    Returns buf.out = residual + S(A) + sum_i w_i Y_i (fp32)."""
    E = W["W_R"].shape[0]
    moe_route(A, W["W_R"], k, gate, renormalize, buf.logits, buf.topk_idx, buf.topk_w, bias=W.get("bias"),
              stream=stream)
    moe_permute(buf.topk_idx, E, buf.offsets, buf.sorted_src, buf.dest_row, A=A, A_perm=buf.A_perm, ws=buf.perm_ws,
                stream=stream)
    moe_grouped_swiglu(buf.A_perm, buf.offsets, W["W1"], W["W2"], W["W3"], buf.Y, ws=buf.gemm_ws, stream=stream)
    if buf.S is not None:
        moe_grouped_swiglu(A, buf.shared_off, W["Ws1"], W["Ws2"], W["Ws3"], buf.S, ws=buf.shared_ws, stream=stream)
    moe_combine(buf.Y, buf.topk_w, buf.dest_row, buf.out, addend=buf.S, residual=residual, stream=stream)
    return buf.out
