"""Summaries of rocprofv3 CSV output for this library's kernels (text, a few KB).

    python -m mixture_experts_layer_sum_amd.profiling stats    <run_kernel_stats.csv>
    python -m mixture_experts_layer_sum_amd.profiling trace    <run_kernel_trace.csv> [--skip-first N]
    python -m mixture_experts_layer_sum_amd.profiling counters <run_counter_collection.csv> [--copy-gib G]
    python -m mixture_experts_layer_sum_amd.profiling traffic  --fetch <csv> --write <csv> --copy-gib G

stats    - rocprofv3's own per-kernel statistics, restricted to the library's kernels.
trace    - per-kernel launch counts / mean durations from the dispatch trace, per queue, and the
           cross-stream overlap of the FarSkip stack: with M the union of the busy intervals of the
           queue that runs the routed grouped GEMM and S the union of the other queue's, it prints
           |M n S| / |S| (share of side-stream work hidden under main-stream work) and |M n S| / |M|.
counters - mean counter value per dispatch for each kernel.  With --copy-gib, the plain device copy
           of that many GiB (the copy dispatch whose counter is closest to that size) calibrates
           FETCH_SIZE / WRITE_SIZE: the printed "scale" is (bytes the copy must move) / (bytes the
           counter reports), and every kernel's corrected HBM bytes are counter KiB x 1024 x scale.
traffic  - FETCH_SIZE and WRITE_SIZE from two runs joined per kernel, calibrated as above, in GB
           per dispatch (lines starting "traffic|" are read by bench.py).
Every summary starts with the digest of the library sources it was taken with.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import sys

LIB_PREFIX = "fsm::"
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")


# the sources the bf16 grouped GEMM (k_gemm_bf16, the stack's dominant kernel) is compiled from
GEMM_SOURCES = ("common.h", "gemm.hip", "tile_kit.h")


def source_digest(files=GEMM_SOURCES) -> str:
    """sha1 over the named HIP sources (names and contents), to tie a profile of the kernels built
    from them to a build."""
    h = hashlib.sha1()
    for f in sorted(files):
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _rows(path):
    with open(path, newline="") as f:
        yield from csv.DictReader(f)


def _col(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    lower = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in lower:
            return lower[n.lower()]
    raise KeyError(names)


def gemm_args(name: str):
    """Template arguments of a k_gemm_bf16 symbol as ints (BM, BN, waves_m, waves_n, epilogue, rows,
    ..., with true / false as 1 / 0), or None for other kernels."""
    i = name.find("k_gemm_bf16<")
    if i < 0:
        return None
    j = name.find(">", i)
    flags = {"true": 1, "false": 0}
    try:
        return tuple(flags[a.strip()] if a.strip() in flags else int(a)
                     for a in name[i + len("k_gemm_bf16<"):j].split(","))
    except ValueError:
        return None


def is_routed_gate_up(name: str) -> bool:
    """The routed (grouped or gathered rows) gate/up + SwiGLU product."""
    a = gemm_args(name)
    return a is not None and len(a) >= 6 and a[4] == 1 and a[5] in (0, 2)


def is_routed(name: str) -> bool:
    """Either routed product (grouped or gathered rows), as opposed to the shared expert / router."""
    a = gemm_args(name)
    return a is not None and len(a) >= 6 and a[5] in (0, 2)


def short(name: str, width: int = 90) -> str:
    name = name.replace("void ", "")
    return name if len(name) <= width else name[:width - 3] + "..."


def cmd_stats(path):
    print(f"# grouped GEMM source digest {source_digest()} (common.h, gemm.hip, tile_kit.h)")
    print(f"# rocprofv3 kernel statistics ({path.split('/')[-1]}), library kernels")
    print(f"{'kernel':<70} {'calls':>6} {'avg_us':>10} {'total_ms':>10} {'pct':>6}")
    for r in _rows(path):
        name = _col(r, "Name", "KernelName", "Kernel_Name")
        if LIB_PREFIX not in name:
            continue
        calls = int(float(_col(r, "Calls", "TotalCalls")))
        total_ns = float(_col(r, "TotalDurationNs", "Total_Duration_Ns", "TotalDuration"))
        avg_ns = float(_col(r, "AverageNs", "Average_Ns", "Average"))
        pct = float(_col(r, "Percentage", "Pct"))
        print(f"{short(name, 70):<70} {calls:>6} {avg_ns / 1e3:>10.1f} {total_ns / 1e6:>10.2f} {pct:>6.2f}")


def _union(iv):
    iv = sorted(iv)
    out = []
    for a, b in iv:
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return out


def _length(iv):
    return sum(b - a for a, b in iv)


def _intersect(x, y):
    i = j = 0
    tot = 0
    while i < len(x) and j < len(y):
        a = max(x[i][0], y[j][0])
        b = min(x[i][1], y[j][1])
        if b > a:
            tot += b - a
        if x[i][1] < y[j][1]:
            i += 1
        else:
            j += 1
    return tot


def overlap(main, side) -> dict:
    """Cross-stream overlap of two lists of (start, end) busy intervals (any one unit): the lengths
    of their unions |M| and |S|, of the intersection |M n S|, and the fractions |M n S| / |S| (the
    share of the side queue's work that ran while the main queue was busy) and |M n S| / |M|."""
    M, S = _union(main), _union(side)
    both = _intersect(M, S)
    lm, ls = _length(M), _length(S)
    return {"main": lm, "side": ls, "both": both,
            "side_hidden": both / ls if ls else None, "main_covered": both / lm if lm else None}


def cmd_trace(path, skip_first=0):
    print(f"# grouped GEMM source digest {source_digest()} (common.h, gemm.hip, tile_kit.h)")
    disp = []
    for r in _rows(path):
        name = _col(r, "Kernel_Name", "KernelName", "Name")
        q = _col(r, "Queue_Id", "QueueId", "Stream_Id")
        t0 = int(_col(r, "Start_Timestamp", "BeginNs", "Start"))
        t1 = int(_col(r, "End_Timestamp", "EndNs", "End"))
        disp.append((t0, t1, q, name))
    disp.sort()
    lib = [d for d in disp if LIB_PREFIX in d[3]]
    gemm = [d for d in lib if is_routed_gate_up(d[3])]
    if skip_first and len(gemm) > skip_first:
        t_begin = gemm[skip_first][0]
        lib = [d for d in lib if d[0] >= t_begin - 50_000_000]  # keep the rest of that step's head
    agg = collections.defaultdict(list)
    for t0, t1, q, name in lib:
        agg[(name, q)].append(t1 - t0)
    print(f"# dispatch trace summary ({path.split('/')[-1]}), library kernels"
          + (f", after the first {skip_first} routed gate/up launches" if skip_first else ""))
    print(f"{'kernel':<70} {'queue':>6} {'calls':>6} {'avg_us':>10} {'total_ms':>10}")
    for (name, q), ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        print(f"{short(name, 70):<70} {q:>6} {len(ds):>6} {sum(ds) / len(ds) / 1e3:>10.1f} {sum(ds) / 1e6:>10.2f}")
    # routed GEMMs (row modes 0 = grouped, 2 = gathered) run on the main queue
    main_q = {d[2] for d in lib if is_routed(d[3])}
    if len(main_q) != 1:
        print("# overlap: could not identify a single main queue")
        return
    mq = main_q.pop()
    ov = overlap([(t0, t1) for t0, t1, q, _ in lib if q == mq], [(t0, t1) for t0, t1, q, _ in lib if q != mq])
    if not ov["side"]:
        print("# overlap: no side-queue work (single stream)")
        return
    span = max(d[1] for d in lib) - min(d[0] for d in lib)
    print(f"# overlap: main queue {mq}; |M| = {ov['main'] / 1e6:.2f} ms, |S| = {ov['side'] / 1e6:.2f} ms, "
          f"|M n S| = {ov['both'] / 1e6:.2f} ms, span = {span / 1e6:.2f} ms")
    print(f"# overlap fraction |M n S|/|S| = {ov['side_hidden']:.4f}   |M n S|/|M| = {ov['main_covered']:.4f}")


def _per_dispatch(path):
    """{kernel: {counter: [per-dispatch value]}} (a counter reported per instance is summed)."""
    vals = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for r in _rows(path):
        name = _col(r, "Kernel_Name", "KernelName", "Name")
        cn = _col(r, "Counter_Name", "CounterName")
        v = float(_col(r, "Counter_Value", "CounterValue", "Value"))
        disp = _col(r, "Dispatch_Id", "DispatchId", "Correlation_Id")
        vals[name][cn][disp] += v
    return {n: {cn: list(d.values()) for cn, d in cs.items()} for n, cs in vals.items()}


def _calibrate(per, cn, copy_gib):
    """scale = expected KiB / measured KiB for the copy dispatch closest to copy_gib GiB."""
    want = copy_gib * 1024 * 1024
    best = None
    names = [n for n in per if "direct_copy" in n.lower()] or [n for n in per if "copy" in n.lower()]
    for n in names:
        cs = per[n]
        if cn not in cs:
            continue
        for v in cs[cn]:
            if v > 0 and (best is None or abs(v - want) < abs(best[0] - want)):
                best = (v, n)
    if best is None:
        return None, None
    return want / best[0], best


def cmd_counters(path, copy_gib=0.0):
    print(f"# grouped GEMM source digest {source_digest()} (common.h, gemm.hip, tile_kit.h)")
    per = _per_dispatch(path)
    scale = {}
    if copy_gib > 0:
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            sc, best = _calibrate(per, cn, copy_gib)
            if sc is not None:
                scale[cn] = sc
                print(f"# calibration: {cn} of the {copy_gib:g} GiB copy = {best[0]:.0f} KiB (expected "
                      f"{copy_gib * 1048576:.0f}) -> scale {sc:.4f}  [{short(best[1], 60)}]")
    print(f"# counters per dispatch ({path.split('/')[-1]}), library kernels: mean over dispatches")
    for name in sorted(per):
        if LIB_PREFIX not in name:
            continue
        parts = []
        for cn, v in sorted(per[name].items()):
            m = sum(v) / len(v)
            s = f"{cn}={m:.4g}"
            if cn in scale:
                s += f" ({m * 1024 * scale[cn] / 1e9:.3f} GB calibrated)"
            parts.append(s)
        n = len(next(iter(per[name].values())))
        print(f"{short(name, 70)}  n={n}  " + "  ".join(parts))


def cmd_traffic(fetch_path, write_path, copy_gib):
    print(f"# grouped GEMM source digest {source_digest()} (common.h, gemm.hip, tile_kit.h)")
    pf, pw = _per_dispatch(fetch_path), _per_dispatch(write_path)
    sf, bf = _calibrate(pf, "FETCH_SIZE", copy_gib)
    sw, bw = _calibrate(pw, "WRITE_SIZE", copy_gib)
    if sf is None or sw is None:
        print("# calibration copy not found")
        return 1
    print(f"# calibration ({copy_gib:g} GiB copy): FETCH_SIZE {bf[0]:.0f} KiB -> scale {sf:.4f}; "
          f"WRITE_SIZE {bw[0]:.0f} KiB -> scale {sw:.4f}")
    print("# per dispatch, calibrated HBM bytes: traffic|kernel|dispatches|fetch_GB|write_GB|total_GB")
    for name in sorted(set(pf) | set(pw)):
        if LIB_PREFIX not in name:
            continue
        f = pf.get(name, {}).get("FETCH_SIZE", [])
        w = pw.get(name, {}).get("WRITE_SIZE", [])
        if not f or not w:
            continue
        fg = sum(f) / len(f) * 1024 * sf / 1e9
        wg = sum(w) / len(w) * 1024 * sw / 1e9
        print(f"traffic|{name}|{len(f)}|{fg:.4f}|{wg:.4f}|{fg + wg:.4f}")
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("path")
    b = sub.add_parser("trace")
    b.add_argument("path")
    b.add_argument("--skip-first", type=int, default=0)
    c = sub.add_parser("counters")
    c.add_argument("path")
    c.add_argument("--copy-gib", type=float, default=0.0)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-gib", type=float, required=True)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        return cmd_stats(args.path)
    if args.cmd == "trace":
        return cmd_trace(args.path, args.skip_first)
    if args.cmd == "traffic":
        return cmd_traffic(args.fetch, args.write, args.copy_gib)
    return cmd_counters(args.path, args.copy_gib)


if __name__ == "__main__":
    sys.exit(main())
