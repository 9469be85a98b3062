"""ctypes loader for libfarskip_moe.so (the C ABI declared in include/farskip_moe.h).

There is no fallback: if the library is missing or cannot be loaded, importing raises.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfarskip_moe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16 = 0, 1
MOE_GATE_SOFTMAX, MOE_GATE_SIGMOID = 0, 1
FARSKIP_NONE, FARSKIP_PARTIAL, FARSKIP_OUTDATED, FARSKIP_PAPER = 0, 1, 2, 3
MOE_MAX_EXPERTS, MOE_MAX_TOPK = 1024, 32
MOE_PERMUTE_NOALLOC_SCRATCH_BYTES = 8 << 20

EXPORTS = ("moe_route", "moe_permute", "moe_permute_workspace_bytes", "moe_permute_noalloc", "moe_grouped_swiglu",
           "moe_grouped_swiglu_workspace_bytes", "moe_grouped_swiglu_gathered", "moe_mx_quantize",
           "moe_grouped_swiglu_mxfp8", "moe_grouped_swiglu_mxfp8_workspace_bytes", "moe_grouped_mxfp8_gate_up",
           "moe_grouped_mxfp8_down", "moe_grouped_mxfp8_phase_workspace_bytes", "moe_layer_backward",
           "moe_layer_backward_workspace_bytes", "farskip_stack_backward", "farskip_stack_backward_workspace_bytes",
           "moe_combine", "farskip_stack_forward", "farskip_attn_moe_stack_forward",
           "farskip_attn_moe_stack_workspace_bytes", "farskip_stack_forward_mxfp8", "farskip_stack_mxfp8_workspace_bytes",
           "farskip_stack_workspace_bytes", "moe_profile_enable", "moe_profile_collect",
           "moe_profile_collect_intervals", "moe_workspace_bytes", "moe_mfma_ceiling", "moe_delivery_probe", "moe_last_error",
           "moe_version")
# moe_op_t: the operations moe_workspace_bytes knows
MOE_OPS = {"permute": 0, "grouped_swiglu": 1, "grouped_swiglu_mxfp8": 2, "mxfp8_phase": 3, "stack": 4,
           "stack_mxfp8": 5, "layer_backward": 6, "stack_backward": 7}
KERNEL_KINDS = ("router_gemm", "topk", "permute_index", "permute_rows", "tile_table", "gemm_gate_up",
                "gemm_down", "combine", "layer_input", "dense_gate_up", "dense_down", "mx_quantize", "mx_gate_up",
                "mx_down", "bwd_recompute", "bwd_dgrad", "bwd_wgrad", "transpose", "bwd_pointwise",
                "mx_dense_gate_up", "mx_dense_down", "attn_gate_up", "attn_down")


class LayerDesc(ctypes.Structure):
    _fields_ = [("W_R", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("W1", ctypes.c_void_p),
                ("W2", ctypes.c_void_p), ("W3", ctypes.c_void_p), ("Ws1", ctypes.c_void_p),
                ("Ws2", ctypes.c_void_p), ("Ws3", ctypes.c_void_p)]


class LayerMx(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("W1q", "W1s", "W2q", "W2s", "W3q", "W3s",
                                                "Ws1q", "Ws1s", "Ws2q", "Ws2s", "Ws3q", "Ws3s")]


class AttnDesc(ctypes.Structure):
    _fields_ = [("Wa1", ctypes.c_void_p), ("Wa2", ctypes.c_void_p), ("Wa3", ctypes.c_void_p)]


class StackCfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("c", ctypes.c_int64),
                ("c_shared", ctypes.c_int64), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("gate", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dA", "dW_R", "dbias", "dW1", "dW2", "dW3", "dWs1", "dWs2", "dWs3")]


class KernelTime(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class KernelInterval(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("pad", ctypes.c_int32), ("stream", ctypes.c_uint64),
                ("start_ms", ctypes.c_double), ("end_ms", ctypes.c_double)]


class StackStats(ctypes.Structure):
    _fields_ = [("wall_ms", ctypes.c_double), ("main_busy_ms", ctypes.c_double), ("side_busy_ms", ctypes.c_double),
                ("overlap_ms", ctypes.c_double), ("overlap_of_side", ctypes.c_double),
                ("overlap_of_main", ctypes.c_double), ("launches_main", ctypes.c_int32),
                ("launches_side", ctypes.c_int32)]


class FarSkipMoEError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


def _declare(lib):
    vp, i64, i32, i, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_size_t
    lib.moe_route.argtypes = [vp, vp, vp, i, i64, i64, i32, i32, i, i, vp, vp, vp, vp]
    lib.moe_route.restype = i
    lib.moe_permute.argtypes = [vp, i, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.restype = i
    lib.moe_permute_noalloc.argtypes = [vp, i, i64, i64, i32, i32, vp, vp, vp, vp, vp, vp]
    lib.moe_permute_noalloc.restype = i
    lib.moe_permute_workspace_bytes.argtypes = [i64, i32, i32]
    lib.moe_permute_workspace_bytes.restype = sz
    lib.moe_grouped_swiglu.argtypes = [vp, vp, i32, vp, vp, vp, i, i64, i64, i64, vp, vp, sz, vp]
    lib.moe_grouped_swiglu.restype = i
    lib.moe_grouped_swiglu_workspace_bytes.argtypes = [i64, i32, i64, i]
    lib.moe_grouped_swiglu_workspace_bytes.restype = sz
    lib.moe_grouped_swiglu_gathered.argtypes = [vp, i64, vp, i32, vp, i32, vp, vp, vp, i, i64, i64, i64, vp, vp,
                                                 sz, vp]
    lib.moe_grouped_swiglu_gathered.restype = i
    lib.moe_mx_quantize.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.moe_mx_quantize.restype = i
    lib.moe_grouped_swiglu_mxfp8.argtypes = [vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp, i64, i64, i64,
                                             vp, vp, sz, vp]
    lib.moe_grouped_swiglu_mxfp8.restype = i
    lib.moe_grouped_swiglu_mxfp8_workspace_bytes.argtypes = [i64, i32, i64]
    lib.moe_grouped_swiglu_mxfp8_workspace_bytes.restype = sz
    lib.moe_grouped_mxfp8_gate_up.argtypes = [vp, vp, i64, vp, i32, vp, i32, vp, vp, vp, vp, i64, i64, i64, vp, vp,
                                              vp, sz, vp]
    lib.moe_grouped_mxfp8_gate_up.restype = i
    lib.moe_grouped_mxfp8_down.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, vp, vp, sz, vp]
    lib.moe_grouped_mxfp8_down.restype = i
    lib.moe_grouped_mxfp8_phase_workspace_bytes.argtypes = [i64, i32]
    lib.moe_grouped_mxfp8_phase_workspace_bytes.restype = sz
    lib.moe_layer_backward.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(StackCfg), vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, ctypes.POINTER(LayerGrads), vp, sz, vp]
    lib.moe_layer_backward.restype = i
    lib.moe_layer_backward_workspace_bytes.argtypes = [ctypes.POINTER(StackCfg)]
    lib.moe_layer_backward_workspace_bytes.restype = sz
    lib.farskip_stack_backward.argtypes = [ctypes.POINTER(LayerDesc), i32, ctypes.POINTER(StackCfg), i, vp, vp, vp, vp,
                                           ctypes.POINTER(LayerGrads), vp, sz, vp]
    lib.farskip_stack_backward.restype = i
    lib.farskip_stack_backward_workspace_bytes.argtypes = [ctypes.POINTER(StackCfg), i32]
    lib.farskip_stack_backward_workspace_bytes.restype = sz
    lib.moe_combine.argtypes = [vp, i, vp, vp, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.moe_combine.restype = i
    lib.farskip_stack_forward.argtypes = [ctypes.POINTER(LayerDesc), i32, ctypes.POINTER(StackCfg), i,
                                          ctypes.POINTER(ctypes.c_uint8), vp, vp, vp, sz, vp, vp,
                                          ctypes.POINTER(StackStats)]
    lib.farskip_stack_forward.restype = i
    lib.farskip_attn_moe_stack_forward.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(AttnDesc), i32,
                                                   ctypes.POINTER(StackCfg), i64, i, vp, vp, vp, sz, vp, vp,
                                                   ctypes.POINTER(StackStats)]
    lib.farskip_attn_moe_stack_forward.restype = i
    lib.farskip_attn_moe_stack_workspace_bytes.argtypes = [ctypes.POINTER(StackCfg), i64]
    lib.farskip_attn_moe_stack_workspace_bytes.restype = sz
    lib.farskip_stack_forward_mxfp8.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerMx), i32,
                                                ctypes.POINTER(StackCfg), i, ctypes.POINTER(ctypes.c_uint8), vp, vp,
                                                vp, sz, vp, vp, ctypes.POINTER(StackStats)]
    lib.farskip_stack_forward_mxfp8.restype = i
    lib.farskip_stack_mxfp8_workspace_bytes.argtypes = [ctypes.POINTER(StackCfg)]
    lib.farskip_stack_mxfp8_workspace_bytes.restype = sz
    lib.farskip_stack_workspace_bytes.argtypes = [ctypes.POINTER(StackCfg)]
    lib.farskip_stack_workspace_bytes.restype = sz
    lib.moe_profile_enable.argtypes = [i]
    lib.moe_profile_enable.restype = i
    lib.moe_profile_collect.argtypes = [ctypes.POINTER(KernelTime)]
    lib.moe_profile_collect.restype = i
    lib.moe_profile_collect_intervals.argtypes = [ctypes.POINTER(KernelTime), ctypes.POINTER(KernelInterval), i32,
                                                  ctypes.POINTER(i32)]
    lib.moe_profile_collect_intervals.restype = i
    lib.moe_workspace_bytes.argtypes = [i, i64, i64, i32, i32, i64, i32, i64, i]
    lib.moe_mfma_ceiling.argtypes = [i, i32, i32, vp, vp]
    lib.moe_mfma_ceiling.restype = i
    lib.moe_delivery_probe.argtypes = [i32, i64, i32, i32, i32, vp, i64, vp, vp, vp]
    lib.moe_delivery_probe.restype = i
    lib.moe_workspace_bytes.restype = sz
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    return lib


def load():
    # The library must run on the same HIP runtime as the framework that owns the device memory and
    # streams it is handed.  torch bundles its own libamdhip64; importing torch first makes the
    # library's libamdhip64.so.7 dependency resolve to that already-loaded copy instead of loading a
    # second runtime into the process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_sum_amd.build` "
                          "(the HIP library is required, there is no fallback)")
    return _declare(ctypes.CDLL(LIB_PATH))


lib = load()


def check(fn: str, rc: int) -> None:
    if rc != MOE_OK:
        raise FarSkipMoEError(fn, rc, lib.moe_last_error().decode(errors="replace"))
