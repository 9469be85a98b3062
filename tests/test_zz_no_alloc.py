"""moe_permute_noalloc (the permutation with its scratch in the library's fixed device array, for
callers that cannot allocate) against moe_permute with a workspace, through the C ABI: bit-exact
offsets, sorted_src, dest_row and permuted rows, on two calls in a row, the second smaller (the
array keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import moe_inputs as mi
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bufs(T, E, k):
    return (torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
            torch.full((T * k,), -7, dtype=torch.int32, device=DEV),
            torch.full((T * k,), -7, dtype=torch.int32, device=DEV))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@pytest.mark.parametrize("shapes", [((65536, 256, 8, 7168), (1000, 256, 8, 7168)),
                                    ((20000, 1024, 32, 64), (3, 5, 2, 64))],
                         ids=["dsv3-then-small", "limits-then-tiny"])
def test_permute_noalloc_equals_workspace_call(shapes):
    from mixture_experts_layer_sum_amd import _lib as L
    from mixture_experts_layer_sum_amd import ops
    lib = L.lib
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for call, (T, E, k, d) in enumerate(shapes):
        seed = mi.seed_for(94, T, E, k, call)
        idx = mi.topk_assignments(T, E, k, seed, zipf=1.2 if call == 0 else 0.0).to(torch.int32).to(DEV)
        A = mi.normal((T, d), 1.0, seed + 1, DEV, torch.bfloat16)
        off_a, src_a, dest_a = _bufs(T, E, k)
        off_b, src_b, dest_b = _bufs(T, E, k)
        Ap_a = torch.empty((T * k, d), dtype=torch.bfloat16, device=DEV)
        Ap_b = torch.full_like(Ap_a, float("nan"))
        ws = ops.workspace(ops.permute_workspace_bytes(T, E, k), DEV)
        rc = lib.moe_permute(_p(A), L.MOE_BF16, T, d, E, k, _p(idx), _p(off_a), _p(src_a), _p(dest_a), _p(Ap_a),
                             _p(ws), ws.numel(), stream)
        assert rc == 0, lib.moe_last_error()
        rc = lib.moe_permute_noalloc(_p(A), L.MOE_BF16, T, d, E, k, _p(idx), _p(off_b), _p(src_b), _p(dest_b),
                                     _p(Ap_b), stream)
        assert rc == 0, lib.moe_last_error()
        torch.cuda.synchronize()
        for a, b in ((off_a, off_b), (src_a, src_b), (dest_a, dest_b)):
            assert torch.equal(a, b)
        assert torch.equal(Ap_a.view(torch.int16), Ap_b.view(torch.int16))
        # and both equal the oracle's counting sort
        r_off, r_src, r_dest = oracle.permute(idx.cpu().numpy(), E) if T * k <= 70000 else (None, None, None)
        if r_off is not None:
            np.testing.assert_array_equal(off_b.cpu().numpy(), r_off)
            np.testing.assert_array_equal(src_b.cpu().numpy(), r_src)
            np.testing.assert_array_equal(dest_b.cpu().numpy(), r_dest)
        print(f"[no-alloc] call {call}: T={T} E={E} k={k} bit-exact", flush=True)


def test_permute_noalloc_rejects_oversize():
    from mixture_experts_layer_sum_amd import _lib as L
    lib = L.lib
    idx = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    rc = lib.moe_permute_noalloc(None, L.MOE_BF16, 1 << 17, 0, 1024, 32, _p(idx), _p(idx), _p(idx), _p(idx), None,
                                 None)
    assert rc == L.MOE_ERR_UNSUPPORTED and b"scratch" in lib.moe_last_error()
