"""Benchmark: the DeepSeek-V3-shaped 4-layer FarSkip MoE stack on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload dsv3-stack]

One step = one farskip_stack_forward over the whole hot path (router, top-k, permutation, routed
grouped SwiGLU GEMM, shared expert, combine, FarSkip wiring) for T tokens through L layers, with
the inputs and weights already resident in HBM.  Layer k's routed work runs on the main HIP stream
while layer k+1's router and shared expert run on a second stream.

Prints one JSON line.  value = T * L / step time: tokens through one MoE sublayer per second
(routed tokens/s of the metric).  The roofline object reports the dominant kernel (the grouped
gate/up GEMM, 2/3 of the routed FLOPs) from HIP-event timings recorded live on its own stream
during the timed steps.  cpu_baseline times the CPU oracle on a bounded sample of tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed tokens/s + MFMA util, bf16 MoE layer (DeepSeek-V3 shape), 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="dsv3-stack")
    p.add_argument("--mode", default="partial", choices=["none", "partial", "outdated"])
    p.add_argument("--cpu-sample", type=int, default=1024, help="tokens in the CPU-oracle sample; 0 = skip")
    p.add_argument("--cpu-configs", type=int, default=1,
                   help="with --configs: also time the CPU oracle on one layer of each smaller workload at full T")
    p.add_argument("--compare-steps", type=int, default=3,
                   help="interleaved two-stream / one-stream steps, profiling off for both; 0 = skip")
    p.add_argument("--decode", type=int, default=1,
                   help="after the steps, time a 1024-token decode step through the same layers; 0 = skip")
    p.add_argument("--standalone", type=int, default=1,
                   help="after the steps, time the layer-0 calls one at a time and the box's ceilings; 0 = skip")
    p.add_argument("--mxfp8", type=int, default=1,
                   help="after the steps, time the layer-0 routed experts with MXFP8 operands; 0 = skip")
    p.add_argument("--mxfp8-stack", type=int, default=1,
                   help="with --mxfp8: also time the prefill and decode stacks with MXFP8 expert MLPs")
    p.add_argument("--configs", type=int, default=1,
                   help="1 = also time one FarSkip layer of each smaller workload (tiny fp32, DSV2-Lite, "
                        "Qwen3-30B-A3B, Llama-4-Scout)")
    p.add_argument("--attn", type=int, default=1,
                   help="after the steps, time the attention + MoE stack over the same layers; 0 = skip")
    p.add_argument("--backward", type=int, default=1,
                   help="after the steps, time the backward pass of layer 0 (one MoE sublayer); 0 = skip")
    p.add_argument("--calibrate-copy-gib", type=float, default=0.0,
                   help="before the steps, one plain device copy of this many GiB (a known-size kernel whose "
                        "FETCH_SIZE / WRITE_SIZE calibrate the HBM counters); 0 = skip")
    return p.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemm_gate_up_dsv3_stack_hbm_traffic.txt")


def measured_traffic():
    """Calibrated HBM bytes per launch of the routed gate/up GEMM from the committed rocprofv3
    counter summary, or None when that summary was taken with other library sources."""
    from mixture_experts_layer_sum_amd.profiling import is_routed_gate_up, source_digest
    if not os.path.exists(TRAFFIC_PROFILE):
        return None
    lines = open(TRAFFIC_PROFILE).read().splitlines()
    digest = next((l.split()[5] for l in lines if l.startswith("# grouped GEMM source digest")), None)
    if digest != source_digest():
        return None
    for l in lines:
        f = l.split("|")
        if l.startswith("traffic|") and is_routed_gate_up(f[1]):
            return {"fetch_GB": float(f[3]), "write_GB": float(f[4]), "total_GB": float(f[5])}
    return None


COUNTER_PROFILE = os.path.join(ROOT, "profiles", "dsv3_stack_memory_pipeline_counters.txt")


def measured_l2_hit():
    """L2 hit rate (TCC_HIT / (TCC_HIT + TCC_MISS)) of the routed gate/up and down products from the
    committed counter summary of the stack, or {} when it was taken with other library sources."""
    from mixture_experts_layer_sum_amd.profiling import gemm_args, is_routed_gate_up, source_digest
    if not os.path.exists(COUNTER_PROFILE):
        return {}
    lines = open(COUNTER_PROFILE).read().splitlines()
    digest = next((l.split()[5] for l in lines if l.startswith("# grouped GEMM source digest")), None)
    if digest != source_digest():
        return {}
    out = {}
    for l in lines:
        if l.startswith("#") or "TCC_HIT_sum=" not in l or "TCC_MISS_sum=" not in l:
            continue
        name = l.split("  n=")[0]
        a = gemm_args(name)
        kind = ("gemm_gate_up" if is_routed_gate_up(name)
                else "gemm_down" if a is not None and len(a) >= 6 and a[4] == 0 and a[5] == 0 else None)
        if kind is None:
            continue
        hit = float(l.split("TCC_HIT_sum=")[1].split()[0])
        miss = float(l.split("TCC_MISS_sum=")[1].split()[0])
        out[kind] = hit / (hit + miss)
    return out


def delivery_ceilings(dev, hits: dict, tiles: dict) -> dict:
    """The library's operand-delivery launch (256 workgroups, 64 KiB stages loaded into LDS as a
    product's K step loads them, no arithmetic): all runs L2 hits; all from cold regions beyond the
    memory-side cache (HBM); and, for each routed product, its measured L2 hit rate with the misses
    from HBM, with one stage in flight (the products' two-stage ring) and with two, and with the
    misses served by the memory-side cache (one stage in flight).  `tiles` gives
    each product's 64 KiB operand stages per launch, so its K loop's operand rate can be read
    against the probe's at its own hit rate."""
    import torch

    from mixture_experts_layer_sum_amd import ops
    MB, blocks, cold = 1 << 20, 256, 7 << 20
    buf = torch.ones(16 * MB + blocks * cold, dtype=torch.uint8, device=dev)
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)

    def tbps(hot, infl, iters, cold_bytes=cold):
        ops.delivery_probe(hot, cold_bytes, iters, infl, buf, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        ops.delivery_probe(hot, cold_bytes, iters, infl, buf, out, clocks)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        cyc, ticks = clocks.tolist()
        return {"TBps": round(blocks * iters * 65536 / (ms * 1e-3) / 1e12, 2), "us_per_stage": round(ms * 1e3 / iters, 3),
                "clock_GHz": round(cyc / ticks * 0.1, 2) if ticks else None}

    res = {"what": "TB/s into LDS over 256 CUs and us per 64 KiB stage per CU; misses from HBM unless "
                   "named memside; the shader clock workgroup 0 ran at"}
    for infl in (1, 2):
        res[f"all_hit_in_flight_{infl}"] = tbps(100, infl, 2000)
        res[f"all_hbm_in_flight_{infl}"] = tbps(0, infl, 100)
    for kind, hit in hits.items():
        hot = int(round(100 * hit))
        row = {"l2_hit_pct": hot}
        for infl in (1, 2):
            row[f"in_flight_{infl}"] = tbps(hot, infl, 400)
        # the same hit rate with every miss served by the memory-side cache (512 KiB cold regions)
        row["memside_in_flight_1"] = tbps(hot, 1, 400, 512 << 10)
        if kind in tiles:
            row["operand_stages_per_launch"] = tiles[kind]
        res[kind] = row
    del buf, out, clocks
    return res


def stream_overlap(launches, main_stream) -> dict:
    """Cross-stream overlap of the timed stack steps from the per-launch HIP-event intervals: M = the
    main stream's busy time (permutations, routed GEMMs), S = the side stream's (routers, top-k,
    shared experts, combines, next-layer inputs)."""
    from mixture_experts_layer_sum_amd.profiling import overlap
    main = [(a, b) for _, s, a, b in launches if s == main_stream]
    side = [(a, b) for _, s, a, b in launches if s != main_stream]
    ov = overlap(main, side)
    r = lambda v: None if v is None else round(v, 4)  # noqa: E731
    return {"side_hidden_frac": r(ov["side_hidden"]), "main_covered_frac": r(ov["main_covered"]),
            "main_busy_ms": round(ov["main"], 2), "side_busy_ms": round(ov["side"], 2),
            "both_busy_ms": round(ov["both"], 2), "launches": len(launches),
            "what": "|M n S| / |S| and |M n S| / |M| over the timed steps (HIP events around each launch)"}


def fused_input_bytes(c, mode: str = "partial") -> float:
    """Bytes per stack step that the combine moves beyond its own formula: with the skip on at
    consecutive layers, combine_{j-1} also forms x_{j+1} = cast(o_{j-1} (+ S_j)) (L - 2 of the L
    combines of a step): one bf16 write of x, plus one read of S for partial inputs."""
    if mode == "none" or c.layers < 3:
        return 0.0
    per = c.T * c.d * 2.0 * (2 if (mode == "partial" and c.shared_width) else 1)
    return (c.layers - 2) * per


def kernel_report(prof: dict, c, steps: int, extra_bytes: dict = None) -> dict:
    """Per-kind averages and the algorithmic throughput of each kernel kind; extra_bytes adds
    bytes per step to a kind's per-launch formula (work that some of its launches also do)."""
    T, d, E, k, c_, cs = c.T, c.d, c.E, c.k, c.c, c.shared_width
    N = T * k
    per_launch = {  # (algorithmic work per launch, unit)
        "router_gemm": (2.0 * T * d * E, "flop"),
        "topk": (T * E * 4.0 + T * k * 8.0, "byte"),
        "permute_index": (N * 4.0 * 4 + (E + 1) * 4.0, "byte"),   # read idx twice, write 2 arrays
        "permute_rows": (T * d * 2.0 + N * d * 2.0 + N * 4.0, "byte"),  # not launched by the stack
        "gemm_gate_up": (4.0 * N * d * c_, "flop"),
        "gemm_down": (2.0 * N * d * c_, "flop"),
        "dense_gate_up": (4.0 * T * d * cs, "flop"),
        "dense_down": (2.0 * T * d * cs, "flop"),
        "attn_gate_up": (4.0 * T * d * (cs or c_), "flop"),   # the attention stand-in: width of the shared expert
        "attn_down": (2.0 * T * d * (cs or c_), "flop"),
        "combine": (N * d * 2.0 + N * 8.0 + T * d * (2.0 + 4.0 + 4.0), "byte"),
        "layer_input": (T * d * (4.0 + 2.0 + 2.0), "byte"),
        "mx_quantize": (T * d * (2.0 + 1.0 + 1.0 / 32), "byte"),   # the token rows, once per layer
        "mx_gate_up": (4.0 * N * d * c_, "flop_fp8"),
        "mx_down": (2.0 * N * d * c_, "flop_fp8"),
        "mx_dense_gate_up": (4.0 * T * d * cs, "flop_fp8"),
        "mx_dense_down": (2.0 * T * d * cs, "flop_fp8"),
    }
    out = {}
    for kind, (n, ms) in prof.items():
        if n == 0:
            continue
        avg = ms / n
        row = {"launches": n, "avg_ms": round(avg, 4), "ms_per_step": round(ms / steps, 3)}
        if kind in per_launch:
            work, unit = per_launch[kind]
            if unit in ("flop", "flop_fp8"):
                row["tflops"] = round(work / (avg * 1e-3) / 1e12, 1)
                peak = PEAK_FP8_TFLOPS if unit == "flop_fp8" else PEAK_BF16_TFLOPS
                row["frac_mfma_peak"] = round(row["tflops"] / peak, 4)
            else:
                total = work * n + (extra_bytes or {}).get(kind, 0.0) * steps
                row["gbs"] = round(total / (ms * 1e-3) / 1e9, 1)
                row["frac_hbm_peak"] = round(row["gbs"] / PEAK_HBM_GBS, 4)
        out[kind] = row
    return out


def route_report(kernels: dict, c) -> dict:
    """The route step per layer (router logits + top-k gating, one launch or two): its time, and its algorithmic bytes
    (read the layer input and W_R once, write the logits the call returns, write the top-k ids and
    weights) and FLOP over that time, against the HBM and bf16 MFMA peaks."""
    if "router_gemm" not in kernels:
        return None
    # where one router tile holds a token's logits the top-k runs in the router GEMM's epilogue
    ms = (kernels["router_gemm"]["ms_per_step"] + kernels.get("topk", {}).get("ms_per_step", 0.0)) / c.layers
    nbytes = c.T * c.d * 2.0 + c.E * c.d * 2.0 + c.T * c.E * 4.0 + c.T * c.k * 8.0
    flop = 2.0 * c.T * c.d * c.E
    gbs = nbytes / (ms * 1e-3) / 1e9
    tf = flop / (ms * 1e-3) / 1e12
    return {"ms_per_layer": round(ms, 4), "bytes_per_layer": nbytes, "gbs": round(gbs, 1),
            "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "tflops": round(tf, 1),
            "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def ep_share(c, W, A_perm, off, Y, gws, reps: int, ep: int = 8) -> dict:
    """One GPU's share of the routed experts under expert parallelism over `ep` GPUs: the grouped
    SwiGLU product over experts [0, E/ep) and the rows routed to them, which arrive from the
    dispatch exchange already grouped by expert (a slice of the permuted rows)."""
    import torch

    from mixture_experts_layer_sum_amd import ops
    E_loc = c.E // ep
    n_loc = int(off[E_loc].item())
    X = A_perm[:n_loc]
    o = off[:E_loc + 1]
    W1, W2, W3 = W["W1"][:E_loc], W["W2"][:E_loc], W["W3"][:E_loc]
    Yl = Y[:n_loc]
    ops.moe_grouped_swiglu(X, o, W1, W2, W3, Yl, ws=gws)
    torch.cuda.synchronize()
    ops.profile_collect()
    ops.profile_enable(True)
    for _ in range(reps):
        ops.moe_grouped_swiglu(X, o, W1, W2, W3, Yl, ws=gws)
    torch.cuda.synchronize()
    ops.profile_enable(False)
    prof = ops.profile_collect()
    row = {"experts": E_loc, "rows": n_loc}
    for kind, flop in (("gemm_gate_up", 4.0 * n_loc * c.d * c.c), ("gemm_down", 2.0 * n_loc * c.d * c.c)):
        n, ms = prof.get(kind, (0, 0.0))
        if n:
            avg = ms / n
            row[kind] = {"avg_ms": round(avg, 4), "tflops": round(flop / (avg * 1e-3) / 1e12, 1)}
    if "gemm_gate_up" in row and "gemm_down" in row:
        tot = row["gemm_gate_up"]["avg_ms"] + row["gemm_down"]["avg_ms"]
        row["tflops"] = round(6.0 * n_loc * c.d * c.c / (tot * 1e-3) / 1e12, 1)
    return row


def standalone(c, layers, o0, reps: int = 20) -> dict:
    """After the timed steps: the layer-0 calls one at a time on the whole GPU (the stack shares it
    between two streams), `reps` times each, including the explicit dispatch row copy that the stack
    folds into the gate/up GEMM; then the measured ceilings of the box (a device copy, a fill, a
    large hipBLASLt product through torch, and the library's register-only MFMA launch)."""
    import torch

    from mixture_experts_layer_sum_amd import ops
    dev = o0.device
    T, d, E, k, cc = c.T, c.d, c.E, c.k, c.c
    N = T * k
    W = layers[0]
    x = o0.to(c.torch_dtype)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    src = torch.empty((N,), dtype=torch.int32, device=dev)
    dest = torch.empty((N,), dtype=torch.int32, device=dev)
    A_perm = torch.empty((N, d), dtype=c.torch_dtype, device=dev)
    Y = torch.empty((N, d), dtype=c.torch_dtype, device=dev)
    pws = ops.workspace(ops.permute_workspace_bytes(T, E, k), dev)
    gws = ops.workspace(ops.grouped_swiglu_workspace_bytes(N, E, cc, c.torch_dtype), dev)
    ops.moe_route(x, W["W_R"], k, c.gate, c.renormalize, logits, idx, w, bias=W.get("bias"))
    ops.moe_permute(idx, E, off, src, dest, A=x, A_perm=A_perm, ws=pws)
    ops.moe_grouped_swiglu_gathered(x, src, k, off, W["W1"], W["W2"], W["W3"], Y, ws=gws)
    torch.cuda.synchronize()
    ops.profile_collect()
    ops.profile_enable(True)
    for _ in range(reps):
        ops.moe_permute(idx, E, off, src, dest, A=x, A_perm=A_perm, ws=pws)
        ops.moe_grouped_swiglu_gathered(x, src, k, off, W["W1"], W["W2"], W["W3"], Y, ws=gws)
        o = o0.clone()
        ops.moe_combine(Y, w, dest, o, addend=x, residual=o)   # in place on o, as in the stack
    torch.cuda.synchronize()
    ops.profile_enable(False)
    prof = ops.profile_collect()
    rep_ = kernel_report(prof, c, reps)
    out = {k_: rep_[k_] for k_ in ("permute_rows", "gemm_gate_up", "gemm_down", "combine") if k_ in rep_}
    out["ep8_share"] = ep_share(c, W, A_perm, off, Y, gws, reps)
    # 64 KiB operand stages per launch of each routed product: its live 256 x 256 tiles times its K steps
    rows_e = (off[1:] - off[:-1]).cpu()
    mt = int(((rows_e + 255) // 256).sum().item())
    stages = {"gemm_gate_up": mt * (2 * cc // 256) * (d // 64), "gemm_down": mt * (d // 256) * (cc // 64)}
    del A_perm, Y, gws, pws, logits
    # ceilings: plain device-to-device copy and a large bf16 product (hipBLASLt through torch)
    a = torch.empty(2**30 // 4 * 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    m = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)
    n = torch.randn((8192, 8192), device=dev).to(torch.bfloat16)

    def timed(fn, it):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(it):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / it

    ms_copy = timed(lambda: b.copy_(a), 5)
    ms_fill = timed(lambda: b.fill_(1.0), 5)
    ms_mm = timed(lambda: torch.matmul(m, n), 5)
    # the library's register-only MFMA launch (1024 workgroups of 8 waves, no memory traffic)
    probe, iters = torch.empty(1024 * 512, dtype=torch.float32, device=dev), 10000
    mfma = {}
    for shape, name in ((0, "16x16x32"), (1, "32x32x16")):
        ms = timed(lambda: ops.mfma_ceiling(shape, probe, iters), 3)
        mfma[name] = round(1024 * 8 * iters * 262144 / (ms * 1e-3) / 1e12, 1)
    ms = timed(lambda: ops.mfma_ceiling(2, probe, iters // 4), 3)   # scaled fp8, 4x the FLOP per MFMA
    mfma_fp8 = round(1024 * 8 * (iters // 4) * 1048576 / (ms * 1e-3) / 1e12, 1)
    nbytes = a.numel() * 4
    del a, b, m, n
    # the committed counter summary holds the DSV3 stack's products; other workloads get the bounds only
    delivery = delivery_ceilings(dev, measured_l2_hit() if c.name == "dsv3-stack" else {}, stages)
    out["ceilings"] = {
        "device_copy_GBps": round(2 * nbytes / (ms_copy * 1e-3) / 1e9, 1),
        "device_fill_GBps": round(nbytes / (ms_fill * 1e-3) / 1e9, 1),
        "hipblaslt_bf16_8192cubed_TFLOPs": round(2 * 8192**3 / (ms_mm * 1e-3) / 1e12, 1),
        "mfma_register_only_bf16_TFLOPs": mfma,
        "mfma_register_only_fp8_scaled_16x16x128_TFLOPs": mfma_fp8,
        "operand_delivery": delivery,
    }
    # each kernel against the box's measured ceiling of its kind, beside its fraction of the peak
    for kind, v in out.items():
        if not isinstance(v, dict):
            continue
        if "tflops" in v and kind != "ep8_share":
            v["frac_of_hipblaslt"] = round(v["tflops"] / out["ceilings"]["hipblaslt_bf16_8192cubed_TFLOPs"], 4)
            v["frac_of_mfma_ceiling"] = round(v["tflops"] / mfma["16x16x32"], 4)
        if "gbs" in v:
            v["frac_of_device_copy"] = round(v["gbs"] / out["ceilings"]["device_copy_GBps"], 4)
    # each routed product's operand rate (its 64 KiB stages over the launch) against the probe's at
    # the product's own L2 hit rate, one stage in flight as in its ring
    for kind in ("gemm_gate_up", "gemm_down"):
        if kind in out and kind in delivery and "avg_ms" in out[kind]:
            rate = stages[kind] * 65536 / (out[kind]["avg_ms"] * 1e-3) / 1e12
            out[kind]["operand_TBps"] = round(rate, 2)
            out[kind]["frac_of_delivery_ceiling"] = round(rate / delivery[kind]["in_flight_1"]["TBps"], 4)
    return out


def mxfp8(c, layers, o0, reps: int = 20) -> dict:
    """The layer-0 routed experts with MXFP8 operands: the weights quantised once (as at load
    time, untimed), then per repetition the token rows quantised and the gathered grouped product
    on them (fp8 MFMA against the 5 PFLOP/s dense fp8 peak)."""
    import torch

    from mixture_experts_layer_sum_amd import ops
    dev = o0.device
    T, d, E, k, cc = c.T, c.d, c.E, c.k, c.c
    N = T * k
    W = layers[0]
    x = o0.to(torch.bfloat16)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    src = torch.empty((N,), dtype=torch.int32, device=dev)
    dest = torch.empty((N,), dtype=torch.int32, device=dev)
    ops.moe_route(x, W["W_R"], k, c.gate, c.renormalize, logits, idx, w, bias=W.get("bias"))
    ops.moe_permute(idx, E, off, src, dest)
    W1q, W2q, W3q = ops.mx_quantized(W["W1"]), ops.mx_quantized(W["W2"]), ops.mx_quantized(W["W3"])
    xq = (torch.empty((T, d), dtype=torch.uint8, device=dev), torch.empty((T, d // 32), dtype=torch.uint8, device=dev))
    Y = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    ws = ops.workspace(ops.grouped_swiglu_mxfp8_workspace_bytes(N, E, cc), dev)

    def rep():
        ops.moe_mx_quantize(x, xq[0], xq[1])
        ops.moe_grouped_swiglu_mxfp8(xq, off, W1q, W2q, W3q, Y, sorted_src=src, k=k, ws=ws)

    rep()
    torch.cuda.synchronize()
    ops.profile_collect()
    ops.profile_enable(True)
    for _ in range(reps):
        rep()
    torch.cuda.synchronize()
    ops.profile_enable(False)
    rep_ = kernel_report(ops.profile_collect(), c, reps)
    assert torch.isfinite(Y.float()).all().item(), "non-finite MXFP8 output"
    out = {k_: rep_[k_] for k_ in ("mx_quantize", "tile_table", "mx_gate_up", "mx_down") if k_ in rep_}
    ms = sum(v["avg_ms"] for k_, v in out.items())
    out["routed_experts_ms"] = round(ms, 3)
    out["routed_experts_tflops"] = round(6.0 * N * d * cc / (ms * 1e-3) / 1e12, 1)
    del W1q, W2q, W3q, ws, Y
    return out


def mxfp8_stack(c, layers, mxl, o0=None, steps: int = 5, graph: bool = False) -> dict:
    """The same 4-layer FarSkip stack with the expert MLPs on MXFP8 operands
    (farskip_stack_forward_mxfp8) for workload c: the experts' weights quantised once beforehand (as
    at load time, untimed: mxl), then one warm-up and `steps` timed steps on the same two streams;
    per-kernel times and the cross-stream overlap from HIP events, and the weight stream per step
    against the HBM peak (the bound of a decode-sized batch)."""
    import torch

    import moe_inputs as mi
    from mixture_experts_layer_sum_amd import ops
    dev = layers[0]["W_R"].device
    if o0 is None:
        o0 = mi.activations(c, dev).float()
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.stack_mxfp8_workspace_bytes(cfg), dev)
    oL = torch.empty_like(o0)
    main_s, side_s = torch.cuda.current_stream(), torch.cuda.Stream()

    def step():
        ops.farskip_stack_forward_mxfp8(layers, mxl, cfg, "partial", o0, oL, ws, s_main=main_s, s_side=side_s)

    step()
    torch.cuda.synchronize()
    ops.profile_collect()
    ops.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ops.profile_enable(False)
    prof, launches = ops.profile_collect_intervals()
    gms = None
    if graph:   # the same two-stream step captured once into a HIP graph and replayed
        gms = graph_replay_ms(lambda sm: ops.farskip_stack_forward_mxfp8(layers, mxl, cfg, "partial", o0, oL, ws,
                                                                         s_main=sm, s_side=side_s))
    assert torch.isfinite(oL).all().item(), "non-finite MXFP8 stack output"
    ms = (t1 - t0) * 1e3 / steps
    weight_bytes = c.layers * ((3 * c.E * c.c * c.d + 3 * c.shared_width * c.d) * (1 + 1 / 32) + 2 * c.E * c.d)
    gbs = weight_bytes / (ms * 1e-3) / 1e9
    out = {"workload": c.name, "tokens": c.T, "layers": c.layers, "steps": steps, "ms_per_step": round(ms, 3),
           "tokens_per_s": round(c.T * c.layers / (ms * 1e-3), 1),
           "weight_stream": {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_step": round(weight_bytes)},
           "kernels": kernel_report(prof, c, steps, {"combine": fused_input_bytes(c)}),
           "overlap": stream_overlap(launches, main_s.cuda_stream),
           "graph_replay": None if gms is None else {
               "ms_per_step": round(gms, 3), "tokens_per_s": round(c.T * c.layers / (gms * 1e-3), 1)},
           # a batch with fewer than one 256-row tile of rows per expert streams its weights; a
           # prefill batch is bound by the fp8 products (kernels.mx_gate_up.frac_mfma_peak)
           "bound": "hbm (weight_stream)" if c.T * c.k < 256 * c.E else "mfma fp8 (kernels.mx_gate_up)",
           "what": "routed and shared experts MXFP8 (E4M3, E8M0 per 32); router and combine bf16 / fp32"}
    del ws, oL
    torch.cuda.empty_cache()
    return out


def backward(c, layers, o0, reps: int = 2) -> dict:
    """Layer 0's backward pass (moe_layer_backward) for a random output gradient, after its forward
    (router, permutation, gathered grouped product) on the same input.  Per kind of kernel: the
    summed time per call and, for the products, the algorithmic FLOP of that kind per call over it
    (bf16 MFMA peak).  Kinds: U and G recomputed; the activation-gradient products (dH = dY W3,
    dX = [dU | dG] [W1; W2], the router's dlogits W_R); the weight-gradient products (reductions
    over each expert's rows); transposes; pointwise kernels."""
    import torch

    from mixture_experts_layer_sum_amd import ops
    dev = o0.device
    T, d, E, k, cc, cs = c.T, c.d, c.E, c.k, c.c, c.shared_width
    N = T * k
    W = layers[0]
    x = o0.to(torch.bfloat16)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    src = torch.empty((N,), dtype=torch.int32, device=dev)
    dest = torch.empty((N,), dtype=torch.int32, device=dev)
    Y = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    ops.moe_route(x, W["W_R"], k, c.gate, c.renormalize, logits, idx, w, bias=W.get("bias"))
    ops.moe_permute(idx, E, off, src, dest)
    ops.moe_grouped_swiglu_gathered(x, src, k, off, W["W1"], W["W2"], W["W3"], Y)
    dOut = torch.randn((T, d), device=dev) * 0.01
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    grads = {"dA": f32(T, d), "dW_R": f32(E, d), "dW1": f32(E, cc, d), "dW2": f32(E, cc, d), "dW3": f32(E, d, cc)}
    if cs:
        grads.update(dWs1=f32(cs, d), dWs2=f32(cs, d), dWs3=f32(d, cs))
    cfg = ops.stack_cfg(T, d, cc, cs, E, k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.layer_backward_workspace_bytes(cfg), dev)
    log(f"backward workspace {ws.numel() / 2**30:.1f} GiB, HBM in use {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    def call():
        ops.moe_layer_backward(W, cfg, x, logits, idx, w, off, src, dest, Y, dOut, grads, ws=ws)

    call()
    torch.cuda.synchronize()
    ops.profile_collect()
    ops.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    ops.profile_enable(False)
    prof = ops.profile_collect()
    assert all(torch.isfinite(g).all().item() for g in grads.values()), "non-finite gradients"
    Ep = -(-E // 64) * 64
    flop = {"bwd_recompute": 4.0 * N * d * cc + 4.0 * T * d * cs,
            "bwd_dgrad": 6.0 * N * d * cc + 2.0 * T * Ep * d + 6.0 * T * d * cs,
            "bwd_wgrad": 6.0 * N * d * cc + 2.0 * E * d * T + 6.0 * T * d * cs}
    out = {"ms_per_layer": round(ms, 3), "tokens_per_s": round(T / (ms * 1e-3), 1)}
    total_flop = sum(flop.values())
    out["tflops_overall"] = round(total_flop / (ms * 1e-3) / 1e12, 1)
    kinds = {}
    for kind in ("bwd_recompute", "bwd_dgrad", "bwd_wgrad", "transpose", "bwd_pointwise", "tile_table", "combine"):
        n, t = prof.get(kind, (0, 0.0))
        if n == 0:
            continue
        row = {"launches_per_call": n // reps, "ms_per_call": round(t / reps, 3)}
        if kind in flop:
            row["tflops"] = round(flop[kind] / (t / reps * 1e-3) / 1e12, 1)
            row["frac_mfma_peak"] = round(row["tflops"] / PEAK_BF16_TFLOPS, 4)
        kinds[kind] = row
    out["kernels"] = kinds
    del grads, ws, Y
    torch.cuda.empty_cache()
    return out


def stack_backward(c, layers, o0, L: int = 2, reps: int = 1) -> dict:
    """farskip_stack_backward over the first L layers (partial inputs): the forward replay plus the
    L layers' backward passes.  All layers write their weight gradients into one set of buffers
    (the work is the same; 4 layers' fp32 gradients would not fit beside the weights)."""
    import torch

    from mixture_experts_layer_sum_amd import ops
    dev = o0.device
    T, d, E, cc, cs = c.T, c.d, c.E, c.c, c.shared_width
    f32 = lambda *shape: torch.empty(shape, dtype=torch.float32, device=dev)
    g = {"dW_R": f32(E, d), "dW1": f32(E, cc, d), "dW2": f32(E, cc, d), "dW3": f32(E, d, cc)}
    if cs:
        g.update(dWs1=f32(cs, d), dWs2=f32(cs, d), dWs3=f32(d, cs))
    cfg = ops.stack_cfg(T, d, cc, cs, E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.stack_backward_workspace_bytes(cfg, L), dev)
    dOL = torch.randn((T, d), device=dev) * 0.01
    dO0 = torch.empty_like(dOL)
    log(f"stack backward workspace {ws.numel() / 2**30:.1f} GiB, HBM in use "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    def call():
        ops.farskip_stack_backward(layers[:L], cfg, "partial", o0, dOL, dO0, [g] * L, ws=ws)

    call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    assert torch.isfinite(dO0).all().item(), "non-finite stack gradient"
    del g, ws
    torch.cuda.empty_cache()
    return {"layers": L, "mode": "partial", "ms": round(ms, 3), "ms_per_layer": round(ms / L, 3),
            "tokens_per_s": round(T * L / (ms * 1e-3), 1),
            "what": "forward replay (keeping inputs, routing, expert outputs) + backward of every layer"}


def interleaved(fns: dict, n: int) -> dict:
    """Median wall time (ms) of each callable in fns, alternated call by call n times (the device is
    synchronised before and after every call), so that both see the same clocks and temperature."""
    import torch
    times = {k: [] for k in fns}
    for _ in range(n):
        for k, fn in fns.items():
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            times[k].append((time.perf_counter() - t0) * 1e3)
    return {k: statistics.median(v) for k, v in times.items()}


def decode(layers, steps: int = 10) -> dict:
    """One decode step of a 1024-sequence batch through the same 4 layers and weights (the
    dsv3-decode workload): the FarSkip stack with T = 1024.  About 32 rows per expert, so a layer
    streams all of its weights for few tokens and the step is bound by HBM.  The roofline reports
    the weight stream: every routed, shared and router weight byte read once per layer."""
    import torch

    import moe_inputs as mi
    from mixture_experts_layer_sum_amd import ops
    c = mi.BY_NAME["dsv3-decode"]
    dev = layers[0]["W1"].device
    o0 = mi.activations(c, dev).float()
    oL = torch.empty_like(o0)
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.stack_workspace_bytes(cfg), dev)
    main_s, side_s = torch.cuda.current_stream(), torch.cuda.Stream()
    out = {"workload": c.name, "tokens": c.T, "layers": c.layers}

    def step(ss):
        ops.farskip_stack_forward(layers, cfg, "partial", o0, oL, ws, s_main=main_s, s_side=ss)

    for ss in (side_s, main_s, side_s):
        step(ss)
    # step times with profiling off, two streams and one stream alternated step by step
    med = interleaved({"two_streams": lambda: step(side_s), "one_stream": lambda: step(main_s)}, steps)
    for label, ms in med.items():
        out[label] = {"ms_per_step": round(ms, 3), "tokens_per_s": round(c.T * c.layers / (ms * 1e-3), 1)}
    out["two_stream_speedup"] = round(med["one_stream"] / med["two_streams"], 4)
    # per-kernel times from a separate pass with HIP events around every launch
    torch.cuda.synchronize()
    ops.profile_collect()
    ops.profile_enable(True)
    for _ in range(steps):
        step(side_s)
    torch.cuda.synchronize()
    ops.profile_enable(False)
    out["kernels"] = kernel_report(ops.profile_collect(), c, steps, {"combine": fused_input_bytes(c)})
    # the same two-stream step captured once into a HIP graph and replayed
    gms = graph_replay_ms(lambda sm: ops.farskip_stack_forward(layers, cfg, "partial", o0, oL, ws, s_main=sm,
                                                               s_side=side_s))
    out["graph_replay"] = {"ms_per_step": round(gms, 3), "tokens_per_s": round(c.T * c.layers / (gms * 1e-3), 1)}
    assert torch.isfinite(oL).all().item(), "non-finite decode output"
    esz = 2
    weight_bytes = c.layers * esz * (3 * c.E * c.c * c.d + 3 * c.shared_width * c.d + c.E * c.d)
    ms = out["two_streams"]["ms_per_step"]
    gbs = weight_bytes / (ms * 1e-3) / 1e9
    out["roofline"] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_step": weight_bytes,
                       "what": "expert, shared and router weights read once per layer / step time"}
    return out


def attn_stack(c, layers, o0, steps: int = 3) -> dict:
    """The attention + MoE stack (farskip_attn_moe_stack_forward) over the same layers, with a dense
    SwiGLU block of the shared expert's width standing in for each attention sub-block.  The
    section-3 wiring (attention input partial, MoE input outdated: layer j+1's attention runs beside
    layer j's routed experts) and the standard stream, each on two streams and on one, alternated
    step by step with profiling off; then the wiring's cross-stream overlap from one profiled pass."""
    import torch

    import moe_inputs as mi
    from mixture_experts_layer_sum_amd import ops
    dev = o0.device
    ca = c.shared_width or c.c
    attn = [mi.attn_weights(c, j, ca, dev) for j in range(c.layers)]
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.attn_stack_workspace_bytes(cfg, ca), dev)
    oL = torch.empty_like(o0)
    main_s, side_s = torch.cuda.current_stream(), torch.cuda.Stream()

    def step(mode, ss):
        ops.farskip_attn_moe_stack_forward(layers, attn, cfg, ca, mode, o0, oL, ws, s_main=main_s, s_side=ss)

    runs = {"farskip_two_streams": lambda: step("farskip", side_s), "farskip_one_stream": lambda: step("farskip", main_s),
            "none_two_streams": lambda: step("none", side_s), "none_one_stream": lambda: step("none", main_s)}
    for fn in runs.values():
        fn()
    med = interleaved(runs, steps)
    flop = c.layers * c.T * (c.flops_per_token()["total"] + 6 * c.d * ca)
    out = {"workload": c.name, "attn_stand_in_hidden": ca, "layers": c.layers, "steps_each": steps}
    for k_, ms in med.items():
        out[k_] = {"ms_per_step": round(ms, 3), "tokens_per_s": round(c.T * c.layers / (ms * 1e-3), 1),
                   "tflops": round(flop / (ms * 1e-3) / 1e12, 1)}
    out["two_stream_speedup_farskip"] = round(med["farskip_one_stream"] / med["farskip_two_streams"], 4)
    out["two_stream_speedup_none"] = round(med["none_one_stream"] / med["none_two_streams"], 4)
    out["farskip_vs_none_two_streams"] = round(med["none_two_streams"] / med["farskip_two_streams"], 4)
    torch.cuda.synchronize()
    ops.profile_collect()
    ops.profile_enable(True)
    step("farskip", side_s)
    torch.cuda.synchronize()
    ops.profile_enable(False)
    prof, launches = ops.profile_collect_intervals()
    out["overlap"] = stream_overlap(launches, main_s.cuda_stream)
    out["kernels"] = {k_: v for k_, v in kernel_report(prof, c, 1).items()
                      if k_ in ("attn_gate_up", "attn_down", "gemm_gate_up", "gemm_down", "combine", "layer_input")}
    assert torch.isfinite(oL).all().item(), "non-finite attention stack output"
    out["what"] = ("a dense SwiGLU block stands in for attention; farskip = attention input partial (eq. 8b), MoE "
                   "input outdated (eq. 8a); none = the standard stream")
    del attn, ws, oL
    torch.cuda.empty_cache()
    return out


def graph_replay_ms(enqueue, reps: int = 20) -> float:
    """Capture one call into a HIP graph (enqueue(s_main) puts the call on s_main, the capture
    stream; its side stream joins the capture through the call's own events) and return the median
    of `reps` replays between HIP events."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, capture_error_mode="relaxed"):
        enqueue(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record(s)
        g.replay()
        b.record(s)
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in ev)
    del g
    return ms


SMALL_WORKLOADS = ("tiny-fp32", "dsv2-lite", "qwen3-30b-a3b", "llama4-scout")


def per_config(names=SMALL_WORKLOADS, reps: int = 20, warmup: int = 3, cpu: bool = True) -> dict:
    """One FarSkip layer (router, top-k, permutation, routed and shared experts, combine; two
    streams) of each smaller workload: the median of `reps` calls bracketed by HIP events on the
    main stream (the call ends on that stream), then `reps` more calls with per-launch events for
    the kernel report, then `reps` replays of the call captured into a HIP graph.  Each
    workload's weights are released before the next one's are drawn."""
    import torch

    import moe_inputs as mi
    from mixture_experts_layer_sum_amd import ops

    dev = "cuda:0"
    out = {}
    for name in names:
        c = mi.BY_NAME[name]
        layers = [mi.layer_weights(c, j, dev) for j in range(c.layers)]
        o0 = mi.activations(c, dev).float()
        cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
        ws = ops.workspace(ops.stack_workspace_bytes(cfg), dev)
        oL = torch.empty_like(o0)
        main_s, side_s = torch.cuda.current_stream(), torch.cuda.Stream()

        def call():
            ops.farskip_stack_forward(layers, cfg, "partial", o0, oL, ws, s_main=main_s, s_side=side_s)

        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(main_s)
            call()
            b.record(main_s)
        torch.cuda.synchronize()
        ms = statistics.median(a.elapsed_time(b) for a, b in ev)
        ops.profile_enable(True)
        for _ in range(reps):
            call()
        torch.cuda.synchronize()
        ops.profile_enable(False)
        prof, _ = ops.profile_collect_intervals()
        # the same call captured once into a HIP graph: what the launches themselves cost
        gms = graph_replay_ms(lambda sm: ops.farskip_stack_forward(layers, cfg, "partial", o0, oL, ws, s_main=sm,
                                                                   s_side=side_s), reps)
        assert torch.isfinite(oL).all().item(), f"non-finite output ({name})"
        kernels = kernel_report(prof, c, reps)
        peak = PEAK_F32_TFLOPS if c.dtype == "f32" else PEAK_BF16_TFLOPS
        if c.dtype == "f32":   # fp32 products: fractions against the fp32 MFMA peak
            for row in kernels.values():
                if "tflops" in row:
                    row["frac_mfma_peak"] = round(row["tflops"] / peak, 4)
        flop = c.layers * c.T * c.flops_per_token()["total"]
        out[name] = {
            "shape": {"T": c.T, "d": c.d, "E": c.E, "k": c.k, "c": c.c, "shared": c.shared_width,
                      "gate": c.gate, "renormalize": c.renormalize, "dtype": c.dtype},
            "ms_per_layer": round(ms / c.layers, 4), "reps": reps,
            "graph_replay_ms_per_layer": round(gms / c.layers, 4),
            "tokens_per_s": round(c.T * c.layers / (ms * 1e-3), 1),
            "routed_assignments_per_s": round(c.T * c.k * c.layers / (ms * 1e-3), 1),
            "tflops": round(flop / (ms * 1e-3) / 1e12, 2),
            "frac_mfma_peak": round(flop / (ms * 1e-3) / 1e12 / peak, 4),
            "kernels": kernels,
        }
        log(f"{name}: {ms:.3f} ms per layer ({gms:.3f} ms as a graph replay), {out[name]['tflops']} TFLOP/s")
        if cpu:   # the CPU oracle on the same layer at full T
            try:
                out[name]["cpu_baseline"] = cpu_baseline_full(c, layers, o0)
                log(f"{name}: CPU oracle {out[name]['cpu_baseline']['oracle_s']} s per layer")
            except Exception as e:  # noqa: BLE001
                out[name]["cpu_baseline"] = {"error": f"{type(e).__name__}: {e}"}
        del layers, o0, ws, oL
        torch.cuda.empty_cache()
    return out


def host_cpu() -> dict:
    """The host's CPU model and the threads the oracle's BLAS uses."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=None)
    except Exception:  # noqa: BLE001
        pass
    return {"cores": threads or len(os.sched_getaffinity(0)), "cpu_model": model,
            "affinity_cpus": len(os.sched_getaffinity(0))}


class _TimedSlices:
    """W[e] -> expert e's weights as float64, copied from the device when first asked for (bf16
    moved as is, widened on the host) and kept while `keep`; the copy time is accumulated in
    self.clock[0] so that it can be excluded from the oracle's time."""

    def __init__(self, t, clock, keep: bool):
        self.t, self.clock, self.cache = t, clock, ({} if keep else None)

    def __getitem__(self, e):
        import torch
        e = int(e)
        if self.cache is not None and e in self.cache:
            return self.cache[e]
        t0 = time.perf_counter()
        host = self.t[e].detach().cpu().to(torch.float64).numpy()
        self.clock[0] += time.perf_counter() - t0
        if self.cache is not None:
            self.cache[e] = host
        return host


def _oracle_weights(W, clock, keep: bool):
    import torch

    def small(t):
        if t is None:
            return None
        t0 = time.perf_counter()
        a = t.detach().cpu().to(torch.float64).numpy()
        clock[0] += time.perf_counter() - t0
        return a
    return {"W_R": small(W["W_R"]), "bias": small(W.get("bias")), "W1": _TimedSlices(W["W1"], clock, keep),
            "W2": _TimedSlices(W["W2"], clock, keep), "W3": _TimedSlices(W["W3"], clock, keep),
            "Ws1": small(W.get("Ws1")), "Ws2": small(W.get("Ws2")), "Ws3": small(W.get("Ws3"))}


def cpu_baseline(c, layers, o0, n_tokens: int) -> dict:
    """The CPU oracle as it stands, on n_tokens seeded tokens through all layers of the stack.
    Each expert's weights are copied from the device once per layer (when the oracle first asks
    for them) and not kept; the copy time is measured and excluded."""
    import moe_inputs as mi
    import oracle

    fetch = [0.0]
    Wo = [_oracle_weights(W, fetch, keep=False) for W in layers]
    rows = mi.sample_rows(c.T, n_tokens, mi.seed_for(c.cfg_id, 0, mi.T_SAMPLE, 7))
    x0 = o0[rows.to(o0.device)].cpu().numpy()
    t0 = time.perf_counter()
    oracle.moe_stack(x0, Wo, c.k, c.gate, c.renormalize, "partial", None, c.n_shared, c.c_shared)
    wall = time.perf_counter() - t0
    compute = max(wall - fetch[0], 1e-9)
    host = host_cpu()
    return {"value": round(n_tokens * c.layers / compute, 3), "unit": "tokens/s", "cores": host["cores"],
            "kind": "oracle", "cpu_model": host["cpu_model"], "oracle_s": round(compute, 2),
            "weight_copy_s": round(fetch[0], 2),
            "sample": f"{n_tokens} seeded tokens of the {c.name} workload through all {c.layers} layers, "
                      f"every expert's weights copied once per layer (float64 NumPy oracle; {compute:.1f} s of "
                      f"oracle work; {fetch[0]:.1f} s of device-to-host weight copies excluded)"}


def cpu_baseline_full(c, layers, o0, long_run_s: float = 10.0) -> dict:
    """The CPU oracle on one layer of workload c at its full T: the median of 3 runs (1 run when the
    first takes longer than long_run_s).  Weights are copied to the host once, before the timing."""
    import statistics as st

    import oracle
    fetch = [0.0]
    Wo = _oracle_weights(layers[0], fetch, keep=True)
    for e in range(c.E):      # copy and widen every expert before the clock starts
        Wo["W1"][e], Wo["W2"][e], Wo["W3"][e]
    x = o0.cpu().numpy()
    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.moe_layer(x, Wo, c.k, c.gate, c.renormalize, c.n_shared, c.c_shared)
        times.append(time.perf_counter() - t0)
        if times[0] > long_run_s:
            break
    med = st.median(times)
    host = host_cpu()
    return {"value": round(c.T / med, 1), "unit": "tokens/s", "cores": host["cores"], "kind": "oracle",
            "cpu_model": host["cpu_model"], "runs": len(times), "oracle_s": round(med, 3),
            "sample": f"one layer of {c.name} at its full T = {c.T} (float64 NumPy oracle; median of "
                      f"{len(times)} run(s); weight copies excluded)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU expert-parallel "
              "path (collectives across GPUs) is not implemented in this library.", file=sys.stderr)
        sys.exit(2)

    import torch

    import moe_inputs as mi
    from mixture_experts_layer_sum_amd import ops

    c = mi.BY_NAME[args.workload]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    log(f"workload {c.name}: T={c.T} d={c.d} E={c.E} k={c.k} c={c.c} shared={c.shared_width} L={c.layers}")
    t0 = time.perf_counter()
    layers = []
    for j in range(c.layers):
        layers.append(mi.layer_weights(c, j, dev))
        torch.cuda.synchronize()
        log(f"layer {j} weights generated ({time.perf_counter() - t0:.1f} s)")
    o0 = mi.activations(c, dev).float()
    cfg = ops.stack_cfg(c.T, c.d, c.c, c.shared_width, c.E, c.k, c.gate, c.renormalize, c.torch_dtype)
    ws = ops.workspace(ops.stack_workspace_bytes(cfg), dev)
    oL = torch.empty_like(o0)
    main_s = torch.cuda.current_stream()
    side_s = torch.cuda.Stream()
    log(f"workspace {ws.numel() / 2**30:.1f} GiB, HBM in use {torch.cuda.memory_allocated() / 2**30:.1f} GiB")

    if args.calibrate_copy_gib > 0:
        n = int(args.calibrate_copy_gib * 2**30) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"calibration copy of {n * 4 / 2**30:.2f} GiB done")
        del src, dst

    def step(ss):
        ops.farskip_stack_forward(layers, cfg, args.mode, o0, oL, ws, s_main=main_s, s_side=ss)

    for _ in range(args.warmup):
        step(side_s)
    torch.cuda.synchronize()
    log("warmup done")

    ops.profile_enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step(side_s)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ops.profile_enable(False)
    prof, launches = ops.profile_collect_intervals()
    ms_per_step = (t_end - t_start) * 1e3 / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step")
    assert torch.isfinite(oL).all().item(), "non-finite stack output"

    compare = None
    if args.compare_steps > 0:
        # the two schedules with profiling off for both, alternated step by step
        med = interleaved({"two_streams": lambda: step(side_s), "one_stream": lambda: step(main_s)},
                          args.compare_steps)
        compare = {"steps_each": args.compare_steps, "two_streams_ms": round(med["two_streams"], 3),
                   "one_stream_ms": round(med["one_stream"], 3),
                   "two_stream_speedup": round(med["one_stream"] / med["two_streams"], 4),
                   "timing_events_cost_frac": round(ms_per_step / med["two_streams"] - 1.0, 4),
                   "what": "median step times, profiling off, two-stream and one-stream steps alternated; "
                           "timing_events_cost_frac compares the timed (event-bracketed) steps with them"}
        log(f"interleaved: two streams {med['two_streams']:.2f} ms, one stream {med['one_stream']:.2f} ms")
        # one profiled one-stream step: the share of its wall time in which a kernel runs (what is
        # left idle is all a second stream could fill without sharing a CU with the first)
        ops.profile_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step(main_s)
        torch.cuda.synchronize()
        wall_ms = (time.perf_counter() - t0) * 1e3
        ops.profile_enable(False)
        _, one = ops.profile_collect_intervals()
        busy_ms = stream_overlap(one, main_s.cuda_stream)["main_busy_ms"]
        compare["one_stream_kernel_busy_frac"] = round(busy_ms / wall_ms, 4)
        compare["one_stream_idle_ms"] = round(wall_ms - busy_ms, 3)

    kernels = kernel_report(prof, c, args.steps, {"combine": fused_input_bytes(c, args.mode)})
    g = kernels.get("gemm_gate_up", {})
    flops_launch = 4.0 * c.T * c.k * c.d * c.c
    traffic = measured_traffic()
    roofline = {"kernel": "k_gemm_bf16 (grouped gate/up + SwiGLU, rows gathered)", "bound": "mfma",
                "achieved": g.get("tflops"), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": g.get("frac_mfma_peak"), "traffic": None,
                "algorithmic_flop_per_launch": flops_launch, "avg_launch_ms": g.get("avg_ms")}
    if traffic is not None:
        # HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE); the algorithmic minimum is one
        # read of the permuted rows and of W1/W2 plus one write of H
        roofline["traffic"] = round(traffic["total_GB"] * 1e9)
        roofline["traffic_detail"] = traffic
        # rows are gathered from x (read once: T*d), W1/W2 read once, H written once
        roofline["algorithmic_bytes_per_launch"] = 2 * (c.T * c.d + 2 * c.E * c.c * c.d + c.T * c.k * c.c)

    route = route_report(kernels, c)
    total_flop = c.layers * c.T * c.flops_per_token()["total"]
    value = c.T * c.layers / (ms_per_step * 1e-3)
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": c.name, "tokens": c.T, "d_model": c.d, "experts": c.E, "top_k": c.k,
                   "expert_hidden": c.c, "shared_hidden": c.shared_width, "layers": c.layers,
                   "gate": c.gate, "renormalize": c.renormalize, "farskip": args.mode, "streams": 2,
                   "value_is": "tokens x layers / s"},
        "routed_assignments_per_s": round(c.T * c.k * c.layers / (ms_per_step * 1e-3), 1),
        "stack_tflops": round(total_flop / (ms_per_step * 1e-3) / 1e12, 1),
        "stack_frac_mfma_peak": round(total_flop / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "one_stream_ms_per_step": None if compare is None else compare["one_stream_ms"],
        "two_stream_speedup": None if compare is None else compare["two_stream_speedup"],
        "stream_comparison": compare,
        "roofline": roofline,
        "route": route,
        "kernels": kernels,
        "overlap": stream_overlap(launches, main_s.cuda_stream),
    }
    def leg(name, fn):
        """An optional measurement after the timed steps; a failure is reported in its field (and
        on stderr) instead of costing the whole result line."""
        try:
            return fn()
        except Exception as e:  # noqa: BLE001
            log(f"{name} failed: {type(e).__name__}: {e}")
            try:
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
            except Exception:  # noqa: BLE001
                pass
            return {"error": f"{type(e).__name__}: {e}"}

    if args.decode and c.name == "dsv3-stack":
        log("timing the decode-shaped stack")
        result["decode"] = leg("decode", lambda: decode(layers))
    if args.mxfp8 and c.name == "dsv3-stack":
        log("timing the MXFP8 routed experts")
        result["mxfp8"] = leg("mxfp8", lambda: mxfp8(c, layers, o0))
    if args.mxfp8 and args.mxfp8_stack and c.name == "dsv3-stack":
        log("quantising every layer's expert weights to MXFP8")
        mxl = leg("mxfp8 weights", lambda: [ops.layer_mx(W) for W in layers])
        if isinstance(mxl, dict):   # the quantisation failed: report it in place of both stack legs
            result["mxfp8"]["stack"] = result["mxfp8"]["decode_stack"] = mxl
        else:
            log("timing the stack with MXFP8 expert MLPs")
            result["mxfp8"]["stack"] = leg("mxfp8 stack", lambda: mxfp8_stack(c, layers, mxl, o0))
            log("timing the decode-shaped stack with MXFP8 expert MLPs")
            result["mxfp8"]["decode_stack"] = leg(
                "mxfp8 decode stack", lambda: mxfp8_stack(mi.BY_NAME["dsv3-decode"], layers, mxl, steps=10, graph=True))
        del mxl
        torch.cuda.empty_cache()
    if args.attn and c.name == "dsv3-stack":
        log("timing the attention + MoE stack")
        result["attn_stack"] = leg("attn_stack", lambda: attn_stack(c, layers, o0))
    if args.standalone:
        log("timing the single calls alone and the ceilings")
        result["standalone"] = leg("standalone", lambda: standalone(c, layers, o0))
        # the dominant kernel against its operand-delivery ceiling (both timed alone on the GPU)
        sa = result["standalone"] if isinstance(result.get("standalone"), dict) else {}
        gu = sa.get("gemm_gate_up", {})
        dl = sa.get("ceilings", {}).get("operand_delivery", {}).get("gemm_gate_up", {})
        if "frac_of_delivery_ceiling" in gu and dl:
            result["roofline"]["operand_delivery"] = {
                "l2_hit_pct": dl["l2_hit_pct"], "ceiling_TBps": dl["in_flight_1"]["TBps"],
                "probe_clock_GHz": dl["in_flight_1"].get("clock_GHz"),
                "achieved_TBps": gu["operand_TBps"], "frac": gu["frac_of_delivery_ceiling"],
                "what": "the kernel run alone: its 64 KiB operand stages per launch over its time, against the "
                        "delivery probe at its L2 hit rate with one stage in flight (standalone.ceilings)"}
        # the MXFP8 products against the chip's register-only scaled fp8 MFMA rate
        fp8 = (result["standalone"] or {}).get("ceilings", {}).get("mfma_register_only_fp8_scaled_16x16x128_TFLOPs")
        if fp8 and isinstance(result.get("mxfp8"), dict):
            for kind in ("mx_gate_up", "mx_down"):
                v = result["mxfp8"].get(kind)
                if isinstance(v, dict) and "tflops" in v:
                    v["frac_of_mfma_ceiling"] = round(v["tflops"] / fp8, 4)
    if args.configs and c.name == "dsv3-stack":
        log("timing one layer of each smaller workload")
        result["configs"] = leg("configs", lambda: per_config(cpu=bool(args.cpu_configs and args.cpu_sample)))
    if args.cpu_sample > 0:
        log("timing the CPU oracle on a token sample")
        result["cpu_baseline"] = leg("cpu_baseline", lambda: cpu_baseline(c, layers, o0, args.cpu_sample))
    else:
        result["cpu_baseline"] = None
    if args.backward and c.name == "dsv3-stack":
        # last: the backward legs hold the most memory; the stack workspace and the weights of the
        # layers they do not use are released first
        del ws
        del layers[2:]
        torch.cuda.empty_cache()
        log("timing the backward pass of one layer")
        result["backward"] = leg("backward", lambda: backward(c, layers, o0))
        log("timing the backward pass of the stack's first two layers")
        result["backward"]["stack"] = leg("stack backward", lambda: stack_backward(c, layers, o0, L=2))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
