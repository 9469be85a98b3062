"""The C-ABI library on the CPU: it loads, exports every symbol the header declares, and every
argument check returns its documented error code before anything is enqueued (no GPU needed:
these calls never reach a kernel launch)."""
import ctypes
import os
import subprocess
import sys

import pytest

import mixture_experts_layer_sum_amd as pkg
from mixture_experts_layer_sum_amd import _lib as L
from tests.helpers import header_exports

lib = pkg.lib
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BAD = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host-side checks


def test_header_declares_the_boundary():
    names = header_exports()
    for fn in ("moe_route", "moe_permute", "moe_grouped_swiglu", "moe_combine", "farskip_stack_forward"):
        assert fn in names
    assert set(names) == set(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for fn in header_exports():
        assert fn in exported, fn
        assert hasattr(lib, fn)


def test_one_hip_runtime_in_the_process():
    """Loading the library (whatever was imported first) leaves a single HIP runtime mapped: the
    framework's.  Run in a fresh interpreter so that the import order is the library's own."""
    code = ("import mixture_experts_layer_sum_amd as m; m.lib; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'amdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True,
                         cwd=ROOT).stdout.strip()
    libs = eval(out)
    assert len(libs) == 1, libs


def test_version_and_empty_last_error():
    assert b"gfx950" in lib.moe_version()
    lib.moe_permute_workspace_bytes(0, 1, 1)
    assert isinstance(lib.moe_last_error(), bytes)


def err(rc, code, needle=None):
    assert rc == code, (rc, lib.moe_last_error())
    if needle:
        assert needle in lib.moe_last_error().decode()


def test_route_argument_errors():
    f = lib.moe_route
    err(f(BAD, None, None, 0, 4, 64, 8, 2, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG, "both")
    err(f(None, None, None, 0, 4, 0, 8, 9, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG, "k <= E")
    err(f(None, None, None, 0, 4, 0, 8, 0, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, None, None, 0, 4, 0, 0, 1, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, None, None, 0, -1, 0, 8, 2, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, None, None, 0, 4, 0, 2048, 2, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_UNSUPPORTED)
    err(f(None, None, None, 0, 4, 0, 64, 33, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_UNSUPPORTED)
    err(f(None, None, None, 0, 4, 0, 8, 2, 7, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG, "gate")
    err(f(BAD, BAD, None, 5, 4, 64, 8, 2, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG, "dtype")
    err(f(BAD, BAD, None, 1, 4, 100, 8, 2, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_UNSUPPORTED, "% 64")
    err(f(BAD, BAD, None, 1, 4, 0, 8, 2, 0, 0, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, None, None, 0, 4, 0, 8, 2, 0, 0, None, BAD, BAD, None), L.MOE_ERR_INVALID_ARG, "required")
    # an empty batch is valid and enqueues nothing
    assert f(None, None, None, 0, 0, 0, 8, 2, 0, 0, None, None, None, None) == L.MOE_OK


def test_permute_argument_errors():
    f = lib.moe_permute
    ws_need = lib.moe_permute_workspace_bytes(100, 8, 2)
    assert ws_need > 0
    err(f(None, 0, 100, 0, 8, 2, BAD, BAD, BAD, BAD, None, BAD, ws_need - 1, None), L.MOE_ERR_WORKSPACE)
    err(f(None, 0, 100, 0, 8, 2, BAD, BAD, BAD, BAD, None, None, ws_need, None), L.MOE_ERR_WORKSPACE)
    err(f(None, 0, 100, 0, 0, 2, BAD, BAD, BAD, BAD, None, BAD, ws_need, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, 0, -1, 0, 8, 2, BAD, BAD, BAD, BAD, None, BAD, ws_need, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, 0, 100, 0, 8, 2, BAD, None, BAD, BAD, None, BAD, ws_need, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, 0, 100, 0, 8, 2, None, BAD, BAD, BAD, None, BAD, ws_need, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, 1, 100, 64, 8, 2, BAD, BAD, BAD, BAD, BAD, BAD, ws_need, None), L.MOE_ERR_INVALID_ARG, "without A")
    err(f(BAD, 1, 100, 12, 8, 2, BAD, BAD, BAD, BAD, BAD, BAD, ws_need, None), L.MOE_ERR_UNSUPPORTED, "16")
    err(f(BAD, 1, 1 << 30, 64, 8, 4, BAD, BAD, BAD, BAD, BAD, BAD, ws_need, None), L.MOE_ERR_UNSUPPORTED)
    err(f(None, 0, 100, 0, 2000, 2, BAD, BAD, BAD, BAD, None, BAD, ws_need, None), L.MOE_ERR_UNSUPPORTED)


def test_grouped_swiglu_argument_errors():
    f = lib.moe_grouped_swiglu
    need = lib.moe_grouped_swiglu_workspace_bytes(256, 4, 128, 1)
    assert need >= 256 * 128 * 2
    assert lib.moe_grouped_swiglu_workspace_bytes(256, 4, 128, 0) >= 256 * 128 * 4
    err(f(BAD, BAD, 4, BAD, BAD, BAD, 1, 256, 128, 128, BAD, BAD, need - 1, None), L.MOE_ERR_WORKSPACE)
    err(f(BAD, BAD, 0, BAD, BAD, BAD, 1, 256, 128, 128, BAD, BAD, need, None), L.MOE_ERR_INVALID_ARG)
    err(f(BAD, BAD, 4, BAD, BAD, BAD, 1, 256, 100, 128, BAD, BAD, need, None), L.MOE_ERR_UNSUPPORTED, "% 64")
    err(f(BAD, BAD, 4, BAD, BAD, BAD, 1, 256, 128, 96, BAD, BAD, need, None), L.MOE_ERR_UNSUPPORTED)
    err(f(BAD, None, 4, BAD, BAD, BAD, 1, 256, 128, 128, BAD, BAD, need, None), L.MOE_ERR_INVALID_ARG)
    err(f(BAD, BAD, 4, BAD, None, BAD, 1, 256, 128, 128, BAD, BAD, need, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, BAD, 4, BAD, BAD, BAD, 1, 256, 128, 128, BAD, BAD, need, None), L.MOE_ERR_INVALID_ARG)
    err(f(BAD, BAD, 4, BAD, BAD, BAD, 9, 256, 128, 128, BAD, BAD, need, None), L.MOE_ERR_INVALID_ARG, "dtype")
    err(f(BAD, BAD, 4096, BAD, BAD, BAD, 1, 256, 128, 128, BAD, BAD, need, None), L.MOE_ERR_UNSUPPORTED)


def test_grouped_swiglu_gathered_argument_errors():
    f = lib.moe_grouped_swiglu_gathered
    need = lib.moe_grouped_swiglu_workspace_bytes(256, 4, 128, 1)
    args = [BAD, 128, BAD, 2, BAD, 4, BAD, BAD, BAD, 1, 256, 128, 128, BAD, BAD, need, None]
    bad = list(args); bad[15] = need - 1
    err(f(*bad), L.MOE_ERR_WORKSPACE)
    bad = list(args); bad[2] = None
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "sorted_src")
    bad = list(args); bad[3] = 0
    err(f(*bad), L.MOE_ERR_INVALID_ARG)
    bad = list(args); bad[1] = 1 << 20; bad[11] = 1024
    bad[15] = lib.moe_grouped_swiglu_workspace_bytes(256, 4, 128, 1)
    err(f(*bad), L.MOE_ERR_UNSUPPORTED, "2^31")
    bad = list(args); bad[11] = 100
    err(f(*bad), L.MOE_ERR_UNSUPPORTED, "% 64")


def test_combine_argument_errors():
    f = lib.moe_combine
    err(f(BAD, 1, BAD, BAD, 10, 12, 2, None, None, BAD, None, None), L.MOE_ERR_UNSUPPORTED, "% 8")
    err(f(BAD, 1, BAD, BAD, 10, 16, 0, None, None, BAD, None, None), L.MOE_ERR_INVALID_ARG)
    err(f(BAD, 1, None, BAD, 10, 16, 2, None, None, BAD, None, None), L.MOE_ERR_INVALID_ARG, "required")
    err(f(BAD, 1, BAD, BAD, 10, 16, 2, None, None, None, None, None), L.MOE_ERR_INVALID_ARG)
    err(f(BAD, 3, BAD, BAD, 10, 16, 2, None, None, BAD, None, None), L.MOE_ERR_INVALID_ARG, "dtype")
    assert f(None, 1, None, None, 0, 16, 2, None, None, None, None, None) == L.MOE_OK


def _cfg(**kw):
    base = dict(T=64, d=128, c=256, c_shared=0, E=8, k=2, gate=0, renormalize=1, dtype=0)
    base.update(kw)
    return L.StackCfg(**base)


def test_stack_argument_errors():
    f = lib.farskip_stack_forward
    cfg = _cfg()
    need = lib.farskip_stack_workspace_bytes(ctypes.byref(cfg))
    assert need > 64 * 2 * 128 * 4 * 2
    desc = (L.LayerDesc * 2)(*[L.LayerDesc(W_R=0x1000, W1=0x1000, W2=0x1000, W3=0x1000) for _ in range(2)])
    ok_args = (desc, 2, ctypes.byref(cfg), 1, None, BAD, ctypes.c_void_p(0x2000), BAD, need, None, None, None)
    bad = list(ok_args)
    bad[8] = need - 1
    err(f(*bad), L.MOE_ERR_WORKSPACE)
    bad = list(ok_args)
    bad[3] = 7
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "mode")
    bad = list(ok_args)
    bad[1] = 0
    err(f(*bad), L.MOE_ERR_INVALID_ARG)
    bad = list(ok_args)
    bad[6] = BAD
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "alias")
    c2 = _cfg(k=9)
    bad = list(ok_args)
    bad[2] = ctypes.byref(c2)
    err(f(*bad), L.MOE_ERR_INVALID_ARG)
    c3 = _cfg(c_shared=256)
    bad = list(ok_args)
    bad[2] = ctypes.byref(c3)
    bad[8] = lib.farskip_stack_workspace_bytes(ctypes.byref(c3))
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "shared")
    desc_missing = (L.LayerDesc * 2)(L.LayerDesc(W_R=0x1000, W1=0x1000, W2=0x1000, W3=0x1000), L.LayerDesc())
    bad = list(ok_args)
    bad[0] = desc_missing
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "layer 1")
    c4 = _cfg(dtype=1, d=96)
    bad = list(ok_args)
    bad[2] = ctypes.byref(c4)
    err(f(*bad), L.MOE_ERR_UNSUPPORTED)


def test_workspace_queries_scale():
    small = lib.moe_grouped_swiglu_workspace_bytes(1000, 8, 256, 1)
    big = lib.moe_grouped_swiglu_workspace_bytes(2000, 8, 256, 1)
    assert big > small
    assert lib.moe_grouped_swiglu_workspace_bytes(-1, 8, 256, 1) == 0
    assert lib.moe_permute_workspace_bytes(65536, 256, 8) >= 2 * (65536 * 8 // 4096) * 256 * 4
    c5 = _cfg(T=65536, d=7168, c=2048, c_shared=2048, E=256, k=8, gate=1, dtype=1)
    # two Y [T*k, d] buffers (a layer's combine reads one while the next layer's GEMM writes the
    # other) are the largest part; the permuted copy of the activations is not kept
    ws5 = lib.farskip_stack_workspace_bytes(ctypes.byref(c5))
    assert 2 * 65536 * 8 * 7168 * 2 < ws5 < 3 * 65536 * 8 * 7168 * 2


def test_python_binding_refuses_unknown_dtype():
    import torch
    from mixture_experts_layer_sum_amd import ops
    with pytest.raises(TypeError):
        ops.dtype_code(torch.float16)


def test_mxfp8_argument_errors():
    q = lib.moe_mx_quantize
    err(q(BAD, 4, 48, BAD, BAD, None), L.MOE_ERR_UNSUPPORTED, "multiple of 32")
    err(q(None, 4, 64, BAD, BAD, None), L.MOE_ERR_INVALID_ARG)
    assert q(None, 0, 64, None, None, None) == L.MOE_OK   # nothing to do
    f = lib.moe_grouped_swiglu_mxfp8
    need = lib.moe_grouped_swiglu_mxfp8_workspace_bytes(100, 4, 256)
    assert need >= 100 * 256 + 100 * 8
    ok = [BAD, BAD, 100, None, 1, BAD, 4, BAD, BAD, BAD, BAD, BAD, BAD, 100, 256, 256, BAD, BAD, need, None]
    bad = list(ok)
    bad[14] = 192                                    # d % 128 != 0
    err(f(*bad), L.MOE_ERR_UNSUPPORTED, "128")
    bad = list(ok)
    bad[18] = need - 1
    err(f(*bad), L.MOE_ERR_WORKSPACE)
    bad = list(ok)
    bad[2] = 99                                      # without sorted_src x_rows must equal N
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "x_rows")
    bad = list(ok)
    bad[3], bad[4] = BAD, 0                          # gathered with k = 0
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "k=0")
    bad = list(ok)
    bad[11] = None                                   # W3 codes missing
    err(f(*bad), L.MOE_ERR_INVALID_ARG)
    g = lib.moe_grouped_mxfp8_gate_up
    pneed = lib.moe_grouped_mxfp8_phase_workspace_bytes(100, 4)
    assert 0 < pneed < need
    err(g(BAD, BAD, 100, None, 1, BAD, 4, BAD, BAD, BAD, BAD, 100, 256, 256, None, BAD, BAD, pneed, None),
        L.MOE_ERR_INVALID_ARG, "Hq")
    dn = lib.moe_grouped_mxfp8_down
    err(dn(BAD, BAD, BAD, 4, BAD, BAD, 100, 256, 256, BAD, BAD, pneed - 1, None), L.MOE_ERR_WORKSPACE)


def test_backward_argument_errors():
    f = lib.moe_layer_backward
    cfg = _cfg(dtype=1)
    need = lib.moe_layer_backward_workspace_bytes(ctypes.byref(cfg))
    assert need > 0
    desc = L.LayerDesc(W_R=0x1000, W1=0x1000, W2=0x1000, W3=0x1000)
    grads = L.LayerGrads(dA=0x1000, dW_R=0x1000, dW1=0x1000, dW2=0x1000, dW3=0x1000)
    ok = [ctypes.byref(desc), ctypes.byref(cfg)] + [BAD] * 9 + [None, ctypes.byref(grads), BAD, need, None]
    bad = list(ok)
    bad[14] = need - 1
    err(f(*bad), L.MOE_ERR_WORKSPACE)
    c32 = _cfg(dtype=0)
    bad = list(ok)
    bad[1] = ctypes.byref(c32)
    err(f(*bad), L.MOE_ERR_UNSUPPORTED, "bf16")
    c12 = _cfg(dtype=1, E=12)
    bad = list(ok)
    bad[1] = ctypes.byref(c12)
    err(f(*bad), L.MOE_ERR_UNSUPPORTED, "multiple of 8")
    no_dw = L.LayerGrads(dA=0x1000, dW_R=0x1000, dW1=0x1000, dW2=0x1000)
    bad = list(ok)
    bad[12] = ctypes.byref(no_dw)
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "dW3")
    bad = list(ok)
    bad[10] = None                                   # dOut missing
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "dOut")
    s = lib.farskip_stack_backward
    sneed = lib.farskip_stack_backward_workspace_bytes(ctypes.byref(cfg), 2)
    assert sneed > need
    descs = (L.LayerDesc * 2)(desc, desc)
    gs = (L.LayerGrads * 2)(grads, grads)
    sok = [descs, 2, ctypes.byref(cfg), 1, None, BAD, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), gs, BAD, sneed,
           None]
    bad = list(sok)
    bad[7] = bad[6]                                  # dO0 aliases dOL
    err(s(*bad), L.MOE_ERR_INVALID_ARG, "alias")
    bad = list(sok)
    bad[10] = sneed - 1
    err(s(*bad), L.MOE_ERR_WORKSPACE)
    bad = list(sok)
    bad[3] = 5
    err(s(*bad), L.MOE_ERR_INVALID_ARG, "mode")


def test_kernel_kinds_match_the_header():
    """The binding's kernel-kind names follow moe_kernel_kind_t, in order and in number."""
    import re

    from mixture_experts_layer_sum_amd._lib import KERNEL_KINDS
    text = open(os.path.join(ROOT, "include", "farskip_moe.h")).read()
    body = text[text.index("MOE_K_ROUTER_GEMM"):text.index("} moe_kernel_kind_t;")]
    kinds = {int(v): n.lower() for n, v in re.findall(r"MOE_K_(\w+)\s*=\s*(\d+)", body)}
    count = int(re.search(r"MOE_KERNEL_KINDS\s*=\s*(\d+)", body).group(1))
    assert sorted(kinds) == list(range(count))
    assert tuple(kinds[i] for i in range(count)) == KERNEL_KINDS


def test_mxfp8_stack_argument_errors():
    """farskip_stack_forward_mxfp8 rejects bad calls on the host, before any launch."""
    f = lib.farskip_stack_forward_mxfp8
    cfg = _cfg(d=128, c=256, c_shared=128, dtype=1)
    need = lib.farskip_stack_mxfp8_workspace_bytes(ctypes.byref(cfg))
    assert need > lib.farskip_stack_workspace_bytes(ctypes.byref(cfg)) - 64 * 8 * 128 * 2 * 4
    assert lib.farskip_stack_mxfp8_workspace_bytes(ctypes.byref(_cfg(dtype=0))) == 0   # fp32: no MXFP8 stack
    desc = (L.LayerDesc * 2)(*[L.LayerDesc(W_R=0x1000) for _ in range(2)])   # expert weights not read
    full = {n: 0x1000 for n in ("W1q", "W1s", "W2q", "W2s", "W3q", "W3s", "Ws1q", "Ws1s", "Ws2q", "Ws2s", "Ws3q", "Ws3s")}
    mx = (L.LayerMx * 2)(*[L.LayerMx(**full) for _ in range(2)])
    ok_args = [desc, mx, 2, ctypes.byref(cfg), 1, None, BAD, ctypes.c_void_p(0x2000), BAD, need, None, None, None]
    bad = list(ok_args)
    bad[1] = None
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "mx")
    bad = list(ok_args)
    bad[9] = need - 1
    err(f(*bad), L.MOE_ERR_WORKSPACE)
    no_shared = dict(full, Ws3s=None)
    bad = list(ok_args)
    bad[1] = (L.LayerMx * 2)(L.LayerMx(**full), L.LayerMx(**no_shared))
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "shared")
    no_routed = dict(full, W2q=None)
    bad = list(ok_args)
    bad[1] = (L.LayerMx * 2)(L.LayerMx(**no_routed), L.LayerMx(**full))
    err(f(*bad), L.MOE_ERR_INVALID_ARG, "layer 0")
    for c_bad in (_cfg(d=128, c=192, c_shared=128, dtype=1), _cfg(d=128, c=256, c_shared=192, dtype=1),
                  _cfg(d=128, c=256, c_shared=0, dtype=0)):
        bad = list(ok_args)
        bad[3] = ctypes.byref(c_bad)
        err(f(*bad), L.MOE_ERR_UNSUPPORTED)


def test_workspace_bytes_dispatch():
    """moe_workspace_bytes(op, T, d, E, k, c, L, c_shared, dtype) returns what each per-call query
    returns for the same layer sizes (routed rows N = T * k in E groups), and 0 for an unknown op
    or sizes the op rejects."""
    T, d, E, k, c, cs = 4096, 2048, 64, 6, 1408, 2816
    for dt in (L.MOE_BF16, L.MOE_F32):
        cfg = _cfg(T=T, d=d, E=E, k=k, c=c, c_shared=cs, dtype=dt)
        ws = lambda op, Ls=1: lib.moe_workspace_bytes(L.MOE_OPS[op], T, d, E, k, c, Ls, cs, dt)  # noqa: E731
        assert ws("permute") == lib.moe_permute_workspace_bytes(T, E, k) > 0
        assert ws("grouped_swiglu") == lib.moe_grouped_swiglu_workspace_bytes(T * k, E, c, dt) > 0
        assert ws("grouped_swiglu_mxfp8") == lib.moe_grouped_swiglu_mxfp8_workspace_bytes(T * k, E, c) > 0
        assert ws("mxfp8_phase") == lib.moe_grouped_mxfp8_phase_workspace_bytes(T * k, E) > 0
        assert ws("stack") == lib.farskip_stack_workspace_bytes(ctypes.byref(cfg)) > 0
        assert ws("stack_mxfp8") == lib.farskip_stack_mxfp8_workspace_bytes(ctypes.byref(cfg))
        assert ws("layer_backward") == lib.moe_layer_backward_workspace_bytes(ctypes.byref(cfg)) > 0
        assert ws("stack_backward", 3) == lib.farskip_stack_backward_workspace_bytes(ctypes.byref(cfg), 3) > 0
    assert lib.moe_workspace_bytes(L.MOE_OPS["stack_mxfp8"], T, d, E, k, c, 1, cs, L.MOE_BF16) > 0
    assert lib.moe_workspace_bytes(L.MOE_OPS["stack_mxfp8"], T, d, E, k, c, 1, cs, L.MOE_F32) == 0
    assert lib.moe_workspace_bytes(99, T, d, E, k, c, 1, cs, L.MOE_BF16) == 0
    assert lib.moe_workspace_bytes(L.MOE_OPS["permute"], -1, d, E, k, c, 1, cs, L.MOE_BF16) == 0
    assert lib.moe_workspace_bytes(L.MOE_OPS["stack"], T, d, 0, k, c, 1, cs, L.MOE_BF16) == 0
    assert lib.moe_workspace_bytes(L.MOE_OPS["stack_backward"], T, d, E, k, c, 0, cs, L.MOE_BF16) == 0
    # the binding's wrapper passes the same arguments
    from mixture_experts_layer_sum_amd import ops
    assert ops.workspace_bytes("grouped_swiglu", T, d, E, k, c) == \
        lib.moe_grouped_swiglu_workspace_bytes(T * k, E, c, L.MOE_BF16)


def test_stack_stats_struct_layout():
    """moe_stack_stats_t: six doubles then two int32 (56 bytes), as the header declares it."""
    assert ctypes.sizeof(L.StackStats) == 56
    assert L.StackStats.launches_main.offset == 48 and L.StackStats.launches_side.offset == 52


def test_permute_noalloc_rejects_oversize_before_any_launch():
    """moe_permute_noalloc checks its arguments, and that the fixed scratch is large enough, on the
    host before touching the device."""
    f = lib.moe_permute_noalloc
    cap = L.MOE_PERMUTE_NOALLOC_SCRATCH_BYTES
    # 2^22 slots over 1024 experts need 2 x 1024 chunks x 1024 experts x 4 bytes = 8 MiB + 256 > cap
    T, k, E = 1 << 17, 32, 1024
    assert lib.moe_permute_workspace_bytes(T, E, k) > cap
    err(f(None, 1, T, 0, E, k, BAD, BAD, BAD, BAD, None, None), L.MOE_ERR_UNSUPPORTED, "scratch")
    err(f(None, 1, 10, 0, 8, 2, None, BAD, BAD, BAD, None, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, 1, 10, 0, 0, 2, BAD, BAD, BAD, BAD, None, None), L.MOE_ERR_INVALID_ARG)
    err(f(None, 1, 10, 64, 8, 2, BAD, BAD, BAD, BAD, BAD, None), L.MOE_ERR_INVALID_ARG, "A_perm")
    assert lib.moe_permute_workspace_bytes(1 << 16, 256, 8) < cap   # the DSV3 batch fits


def test_attn_stack_argument_errors():
    """farskip_attn_moe_stack_forward rejects bad calls on the host, before any launch."""
    f = lib.farskip_attn_moe_stack_forward
    cfg = _cfg(c_shared=256)
    need = lib.farskip_attn_moe_stack_workspace_bytes(ctypes.byref(cfg), 128)
    assert need > lib.farskip_stack_workspace_bytes(ctypes.byref(cfg))
    assert lib.farskip_attn_moe_stack_workspace_bytes(ctypes.byref(cfg), 0) == 0
    full = dict(W_R=0x1000, W1=0x1000, W2=0x1000, W3=0x1000, Ws1=0x1000, Ws2=0x1000, Ws3=0x1000)
    desc = (L.LayerDesc * 2)(*[L.LayerDesc(**full) for _ in range(2)])
    attn = (L.AttnDesc * 2)(*[L.AttnDesc(Wa1=0x1000, Wa2=0x1000, Wa3=0x1000) for _ in range(2)])
    ok = [desc, attn, 2, ctypes.byref(cfg), 128, L.FARSKIP_PAPER, BAD, ctypes.c_void_p(0x2000), BAD, need, None, None,
          None]
    for i, v, code, needle in ((5, L.FARSKIP_PARTIAL, L.MOE_ERR_INVALID_ARG, "mode"),
                               (1, None, L.MOE_ERR_INVALID_ARG, "attn"),
                               (4, 0, L.MOE_ERR_INVALID_ARG, "c_attn"),
                               (9, need - 1, L.MOE_ERR_WORKSPACE, None),
                               (7, BAD, L.MOE_ERR_INVALID_ARG, "alias"),
                               (1, (L.AttnDesc * 2)(L.AttnDesc(Wa1=0x1000, Wa2=0x1000, Wa3=0x1000), L.AttnDesc()),
                                L.MOE_ERR_INVALID_ARG, "layer 1")):
        bad = list(ok)
        bad[i] = v
        err(f(*bad), code, needle)
    c_bf = _cfg(c_shared=256, dtype=1)
    bad = list(ok)
    bad[3] = ctypes.byref(c_bf)
    bad[4] = 96
    bad[9] = lib.farskip_attn_moe_stack_workspace_bytes(ctypes.byref(c_bf), 96)
    err(f(*bad), L.MOE_ERR_UNSUPPORTED, "c_attn")


def test_mfma_ceiling_argument_errors():
    """The register-only MFMA diagnostic checks its arguments on the host before any launch."""
    f = lib.moe_mfma_ceiling
    err(f(3, 10, 4, BAD, None), L.MOE_ERR_INVALID_ARG, "shape")
    err(f(-1, 10, 4, BAD, None), L.MOE_ERR_INVALID_ARG, "shape")
    err(f(0, 0, 4, BAD, None), L.MOE_ERR_INVALID_ARG)
    err(f(1, 10, 0, BAD, None), L.MOE_ERR_INVALID_ARG)
    err(f(0, 10, 4, None, None), L.MOE_ERR_INVALID_ARG, "out")


def test_delivery_probe_argument_errors():
    """The operand-delivery diagnostic checks its arguments on the host before any launch."""
    f = lib.moe_delivery_probe
    MB = 1 << 20
    ok = dict(hot=50, cold=512 * 1024, iters=10, infl=1, blocks=4, buf=BAD, nbytes=16 * MB + 4 * 512 * 1024, out=BAD)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["hot"], a["cold"], a["iters"], a["infl"], a["blocks"], a["buf"], a["nbytes"], a["out"], None, None)

    err(call(hot=-1), L.MOE_ERR_INVALID_ARG, "hot_pct")
    err(call(hot=101), L.MOE_ERR_INVALID_ARG, "hot_pct")
    err(call(cold=0), L.MOE_ERR_INVALID_ARG, "cold_bytes")
    err(call(cold=1000), L.MOE_ERR_INVALID_ARG, "cold_bytes")
    err(call(iters=0), L.MOE_ERR_INVALID_ARG)
    err(call(blocks=0), L.MOE_ERR_INVALID_ARG)
    err(call(infl=3), L.MOE_ERR_INVALID_ARG, "in_flight")
    err(call(buf=None), L.MOE_ERR_INVALID_ARG, "null")
    err(call(out=None), L.MOE_ERR_INVALID_ARG, "null")
    err(call(nbytes=16 * MB), L.MOE_ERR_INVALID_ARG, "buf_bytes")
    err(call(cold=8 * MB, blocks=256, nbytes=1 << 31), L.MOE_ERR_UNSUPPORTED, "2 GiB")

