"""The diagnostics on the GPU: the register-only MFMA launch (moe_mfma_ceiling) runs every shape,
every thread writes its value, and the throughput is within the chip's dense bf16 or fp8 figure; the
operand-delivery launch (moe_delivery_probe) lands every stage in LDS, and more L2 hits deliver
faster."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [0, 1, 2])
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
    per_round = 1048576 if shape == 2 else 262144
    tflops = blocks * 8 * iters * per_round / (e0.elapsed_time(e1) * 1e-3) / 1e12
    print(f"shape {shape}: {tflops:.0f} TFLOP/s")
    assert 100.0 < tflops < (5100.0 if shape == 2 else 2600.0)   # the dense bf16 / fp8 figures


def test_delivery_probe_lands_stages():
    """Every workgroup's two LDS stages hold bytes of the buffer (all 0x01, so each thread's sum of
    one byte per stage is exactly 2), for both ring depths; workgroup 0's clock readout is a shader
    clock; an all-hot stream is faster than one whose runs all come from cold regions beyond the
    memory-side cache."""
    from mixture_experts_layer_sum_amd import ops
    MB = 1 << 20
    blocks, cold = 256, 4 * MB
    buf = torch.ones(16 * MB + blocks * cold, dtype=torch.uint8, device="cuda")
    out = torch.full((blocks * 512,), float("nan"), dtype=torch.float32, device="cuda")
    rate = {}
    for infl in (1, 2):
        for hot, iters in ((100, 400), (0, 64)):
            out.fill_(float("nan"))
            clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
            ops.delivery_probe(hot, cold, iters, infl, buf, out, clocks)
            torch.cuda.synchronize()
            assert torch.equal(out, torch.full_like(out, 2.0)), (hot, infl)
            cyc, ticks = clocks.tolist()
            ghz = cyc / ticks * 0.1
            print(f"hot {hot}% in flight {infl}: shader clock {ghz:.2f} GHz")
            assert 0.3 < ghz < 3.5   # a shader clock, read against the 100 MHz counter
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            ops.delivery_probe(hot, cold, iters, infl, buf, out)
            e1.record()
            torch.cuda.synchronize()
            rate[(hot, infl)] = blocks * iters * 65536 / (e0.elapsed_time(e1) * 1e-3) / 1e12
            print(f"hot {hot}% in flight {infl}: {rate[(hot, infl)]:.2f} TB/s")
    for infl in (1, 2):
        assert rate[(100, infl)] > rate[(0, infl)]
        assert rate[(0, infl)] < 9.0   # cold runs come from HBM: below its 8 TB/s figure, with margin

