"""The register-only MFMA diagnostic (moe_mfma_ceiling) on the GPU: both shapes run, every thread
writes its value, and the throughput is within the chip's dense bf16 figure."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_ceiling_runs(shape):
    from mixture_experts_layer_sum_amd import ops
    blocks, iters = 512, 2000
    out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device="cuda")
    ops.mfma_ceiling(shape, out, iters)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all().item()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    ops.mfma_ceiling(shape, out, iters)
    e1.record()
    torch.cuda.synchronize()
    tflops = blocks * 8 * iters * 262144 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"shape {shape}: {tflops:.0f} TFLOP/s")
    assert 100.0 < tflops < 2600.0
