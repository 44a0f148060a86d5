#!/usr/bin/env python3
"""Prefill throughput of the DSA hot path on one MI355X.

One step = dsa_indexer_topk followed by dsa_sparse_prefill over one prefill
chunk (indexer scores + exact top-k + causal masking + sparse absorbed-MLA
attention), inputs resident in HBM.  Default workload: N = 131,072 cached keys,
L = 2,048 queries (the newest positions, run as two 1,024-query blocks),
top_k = 2,048, indexer 32 heads x 128, attention 64 heads x 576/512, bf16.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C3]

Prints one JSON line (see the "roofline" and "cpu_baseline" objects).

    python bench.py --decode [--config C3]

times the decode step instead: the newest position's query (L = 1) selects its top-k
of the N cached keys (dsa_indexer_topk) and attends over them with the split-key
attention (dsa_sparse_decode); one JSON line of its own.

    python bench.py --batch {prefill8,ragged,decode64}

times one batched step over several sequences (dsa_indexer_topk_varlen, then
dsa_sparse_prefill_varlen) beside the same sequences run one call each.

    python bench.py --retrieval [--retrieval-n 1048576] [--retrieval-m 1024]

times the inner-product top-k over a corpus (dsa_retrieval_topk): M Gaussian queries
against N Gaussian corpus rows of 128 dims, top_k 1,024.

    python bench.py --pack KEEP [--config C3]

times the sparse attention alone, unpacked and with neighbour packing, on index rows where
each query keeps a fraction KEEP of its predecessor's keys.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "prefill tokens/sec (indexer+topk+sparse attn) at N=128K, top-k=2048; % roofline"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


def graph_ms_per_step(step, steps: int, warmup: int) -> float:
    """Capture step() once in a HIP graph (torch.cuda.graph) and time `steps` replays."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1000.0 / steps


# Source files that define each timed kernel; a traffic figure measured with hardware
# counters is reported only while these files are unchanged since the measurement.
KERNEL_SOURCES = {
    "score_filter": ["indexer.hip", "dsa_common.h", "dsa_internal.h", "../build.py"],
    "sparse_attention": ["attention.hip", "dsa_common.h", "dsa_internal.h", "../build.py"],
}


def kernel_source_hash(kernel: str) -> str:
    import hashlib
    h = hashlib.sha256()
    csrc = ROOT / "dsa_sparse_attention_indexer_amd" / "csrc"
    for name in KERNEL_SOURCES[kernel]:
        h.update((csrc / name).resolve().read_bytes())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.txt (FETCH_SIZE and
    WRITE_SIZE counter runs, scaled by a plain copy of known size), or None when the file
    is missing or the kernel's sources changed since it was measured."""
    f = ROOT / "profiles" / f"traffic_{kernel}_{workload}.txt"
    if not f.exists():
        return None
    fields = {}
    for line in f.read_text().splitlines():
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    try:
        if fields.get("source_sha256") != kernel_source_hash(kernel):
            return None
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError, OSError):
        return None


def workload_sizes(wl):
    """Algorithmic work of one step, per query row: (indexer flops, attention flops, attention bytes)."""
    rows = []
    for t in range(wl.L):
        p = wl.pos0 + t
        n_t = min(p, wl.N - 1) + 1
        k_valid = min(wl.top_k, n_t)
        f_idx = 2 * 32 * 128 * n_t
        f_attn = 2 * wl.H * (576 + 512) * k_valid
        b_attn = k_valid * 576 * 2 + 4 * wl.top_k + wl.H * 576 * 2 + wl.H * 512 * 2
        rows.append((f_idx, f_attn, b_attn))
    return rows


def cpu_baseline(wl, inp, target_s: float):
    """Time the fp64 oracle (indexer + top-k + attention) on a bounded row sample."""
    import numpy as np

    import dsa_inputs as di
    import oracle

    oracle.build(force=False)
    threads = oracle.default_threads()  # affinity CPUs, capped by OMP_NUM_THREADS (the host share of one GPU)

    def run(rows, n_threads):
        t0 = time.perf_counter()
        sel = oracle.topk(inp["q_idx"], inp["k_idx"], inp["w"], wl.pos0, wl.top_k, rows=rows,
                          n_threads=n_threads)
        idx = np.full((wl.L, wl.top_k), -1, np.int32)
        idx[rows] = sel
        oracle.attention(inp["q"], inp["kv"], idx, wl.pos0, di.SOFTMAX_SCALE, rows=rows, n_threads=n_threads)
        return time.perf_counter() - t0

    one = run(np.array([wl.L - 1], np.int64), 1)
    n_rows = int(max(threads, min(wl.L, round(target_s * threads / max(one, 1e-3)))))
    rows = np.unique(np.linspace(0, wl.L - 1, n_rows).round().astype(np.int64))
    secs = run(rows, threads)
    return {
        "value": round(len(rows) / secs, 3),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(rows)} of {wl.L} query rows evenly spaced over the chunk (full causal key "
                  f"range each), fp64 C oracle: full-sort top-k + sparse attention; {secs:.1f} s wall. "
                  f"Rows are independent, so tokens/s = rows / wall time extrapolates linearly to the "
                  f"whole chunk (about {wl.L / len(rows) * secs:.0f} s)",
        "host": host_description(threads),
    }


def host_description(threads: int) -> dict:
    """CPU model and counts of the host the oracle ran on."""
    model = ""
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "threads_used": threads,
            "why": "threads = CPUs in this process's affinity, capped by OMP_NUM_THREADS (the host CPU "
                   "share given to one GPU's job)"}


def selection_summary(st: dict, wl) -> dict:
    """Per-row selection figures of the last indexer call (dsa_indexer_topk_stats)."""
    rows = max(st["rows"], 1)
    return {
        "rows": st["rows"], "rows_all_keys": st["rows_all_keys"],
        "candidates_per_row": round(st["candidates"] / rows, 1), "candidates_max": st["candidates_max"],
        "candidates_per_top_k": round(st["candidates"] / rows / wl.top_k, 3),
        "band_per_row": round(st["band"] / rows, 1), "band_max": st["band_max"],
        "rows_fallback": st["rows_fallback"], "fallback_overflow": st["fallback_overflow"],
        "fallback_incomplete": st["fallback_incomplete"], "fallback_band": st["fallback_band"],
        "rows_failed": st["rows_failed"], "kth_radix": st["kth_radix"],
    }


# Kernels of the selection steps (key layout and statistics, threshold sample, row prep, exact
# select, fallback fold) and of the sparse attention: the byte-bound part of the step.
TOPK_ATTENTION_KERNELS = ["key_stats", "score_sample", "row_prep", "select", "fold", "sparse_attention"]


def topk_attention_hbm(kernels: dict, b_topk: float, b_attn: float):
    """Top-k selection plus sparse attention against the HBM roofline: their algorithmic bytes
    per step (B_topk = 20 L k, B_attn as in the attention roofline) over the time their kernels
    take per step.  None unless the select and attention kernels were timed."""
    if "select" not in kernels or "sparse_attention" not in kernels:
        return None
    names = [k for k in TOPK_ATTENTION_KERNELS if k in kernels]
    t_ms = sum(kernels[k]["ms_per_step"] for k in names)
    ach = (b_topk + b_attn) / (t_ms * 1e-3) / 1e9
    return {"bytes_per_step": int(b_topk + b_attn), "ms_per_step": round(t_ms, 4), "achieved": round(ach, 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "kernels": names}


def measured_ceilings(dsa, dev, mfma_iters: int = 4000, copy_mib: int = 2048, reps: int = 5):
    """What the GPU reaches on plain streams of the two kinds of work the path is bound by
    (dsa_ceiling_*): bf16 MFMA chains alone at one and two waves per SIMD, with constant and
    random operands, and a 16-byte streaming copy. Timed with the library's events."""
    import torch

    out = {}
    buf = torch.empty(dsa.ceiling_mfma_threads(2), dtype=torch.float32, device=dev)
    for wps in (1, 2):
        for rnd in (True, False):
            dsa.ceiling_mfma(buf, 50, rnd, wps)  # warm-up
            torch.cuda.synchronize()
            dsa.profile_set(["ceiling_mfma"])
            dsa.profile_read("ceiling_mfma")
            flops = sum(dsa.ceiling_mfma(buf, mfma_iters, rnd, wps) for _ in range(reps))
            torch.cuda.synchronize()
            ms, n = dsa.profile_read("ceiling_mfma")
            key = f"mfma_bf16_{'random' if rnd else 'constant'}_{wps}wave_per_simd_TFLOPs"
            out[key] = round(flops / (ms * 1e-3) / 1e12, 1)
    n16 = copy_mib * (1 << 20) // 16
    src = torch.ones(n16 * 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    sink = torch.empty(dsa.ceiling_stream_sink_words(), dtype=torch.int32, device=dev)
    nbytes = copy_mib * (1 << 20)
    for name, d, nt, moved in (("read_GBs", None, False, nbytes), ("read_nontemporal_GBs", None, True, nbytes),
                               ("copy_read_plus_write_GBs", dst, False, 2 * nbytes),
                               ("copy_nontemporal_read_plus_write_GBs", dst, True, 2 * nbytes)):
        dsa.ceiling_stream(src, d, sink, nt)
        torch.cuda.synchronize()
        dsa.profile_set(["ceiling_copy"])
        dsa.profile_read("ceiling_copy")
        for _ in range(reps):
            dsa.ceiling_stream(src, d, sink, nt)
        torch.cuda.synchronize()
        ms, n = dsa.profile_read("ceiling_copy")
        out[name] = round(moved * n / (ms * 1e-3) / 1e9, 1)
    dsa.profile_enable(False)
    out["note"] = (f"dsa_ceiling_mfma_bf16 (MFMA chains only, {mfma_iters} x 8 MFMAs per wave) and "
                   f"dsa_ceiling_stream ({copy_mib} MiB read, or read and written), {reps} launches each, HIP events")
    del buf, src, dst, sink
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="C3", help="C0..C4 (default C3, the headline workload)")
    ap.add_argument("--q-block", type=int, default=1024)
    ap.add_argument("--recency", action="store_true",
                    help="indexer keys scaled by 1 + s/N (scores favour recent keys) in place of the "
                         "configuration's own; not a headline measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="do not bracket kernels with events (the roofline object is then omitted)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain elementwise copy of MIB MiB (read MIB, write MIB) three "
                         "times, to scale the FETCH_SIZE / WRITE_SIZE counters, and exit")
    ap.add_argument("--decode", action="store_true",
                    help="time the decode step (L = 1 indexer + split-key attention) instead")
    ap.add_argument("--batch", choices=sorted(BATCHES),
                    help="time a batch of sequences through the varlen entry points instead")
    ap.add_argument("--retrieval", action="store_true",
                    help="time the inner-product top-k over a corpus (vector retrieval) instead")
    ap.add_argument("--retrieval-n", type=int, default=1 << 20)
    ap.add_argument("--retrieval-m", type=int, default=1024)
    ap.add_argument("--retrieval-k", type=int, default=1024)
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed (reported beside the eager step)")
    ap.add_argument("--pack", type=float, default=None, metavar="KEEP",
                    help="time the attention unpacked and neighbour-packed on rows sharing KEEP of their keys")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the MFMA-only and streaming-copy ceilings, print them, and exit")
    ap.add_argument("--no-ceilings", action="store_true", help="do not measure the ceilings in the default mode")
    ap.add_argument("--print-source-hash", metavar="KERNEL", choices=sorted(KERNEL_SOURCES),
                    help="print the source hash a traffic summary for KERNEL must carry, and exit")
    args = ap.parse_args()
    if args.print_source_hash:
        print(kernel_source_hash(args.print_source_hash))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path runs on one GPU (it would shard by query with no exchange); "
              "runs on several GPUs are not part of it. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import dsa_inputs as di
    import dsa_sparse_attention_indexer_amd as dsa

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}))
        return
    dsa.load_library()
    if args.ceilings:
        print(json.dumps({"measured_ceilings": measured_ceilings(dsa, dev)}), flush=True)
        return
    if args.batch:
        bench_batch(args, dev)
        return
    if args.retrieval:
        bench_retrieval(args, dev)
        return
    wl = di.CONFIGS[args.config]
    if args.recency:
        wl = di.replace(wl, name=wl.name + "-recency", indexer="recency")
    t0 = time.perf_counter()
    inp = di.make_inputs(wl)
    log(f"[bench] {wl.name}: inputs generated in {time.perf_counter() - t0:.1f} s")
    if args.decode:
        bench_decode(args, wl, inp, dev)
        return
    if args.pack is not None:
        bench_pack(args, wl, inp, dev)
        return

    def bf(a):
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)

    q_idx, k_idx, q, kv = bf(inp["q_idx"]), bf(inp["k_idx"]), bf(inp["q"]), bf(inp["kv"])
    w = torch.from_numpy(inp["w"]).to(dev)
    idx = torch.empty((wl.L, wl.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((wl.L, wl.H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dsa.workspace_bytes(wl.L, wl.N, wl.top_k, args.q_block), dtype=torch.uint8, device=dev)
    scale = float(np.float32(di.SOFTMAX_SCALE))

    def step():
        dsa.indexer_topk(q_idx, k_idx, w, wl.pos0, wl.top_k, q_block=args.q_block, out=idx, workspace=ws)
        dsa.sparse_prefill(q, kv, idx, wl.pos0, scale, q_block=args.q_block, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # In the timed region only the two kernels the roofline is computed for carry timing events
    # (events around every launch would add a few percent); the other kernels are timed in an
    # untimed pass afterwards.
    timing = not args.no_kernel_timing
    roof_kernels = ["score_filter", "sparse_attention"]
    if timing:
        dsa.profile_set(roof_kernels)
        for k in dsa.PROFILE_KERNELS:
            dsa.profile_read(k)
    torch.cuda.synchronize()  # barrier: one rank
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t_start = time.perf_counter()
    marks[0].record()
    for i in range(args.steps):
        step()
        marks[i + 1].record()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    ms_per_step = (t_end - t_start) * 1000.0 / args.steps
    step_ms = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    ms_median = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (
        step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    selection = selection_summary(dsa.indexer_stats(ws), wl)
    kernels = {}
    if timing:
        for k in roof_kernels:
            ms, n = dsa.profile_read(k)
            if n:
                kernels[k] = {"launches_per_step": n / args.steps, "ms_per_launch": ms / n,
                              "ms_per_step": ms / args.steps}
        extra = max(3, args.steps // 4)
        dsa.profile_set(None)
        for _ in range(extra):
            step()
        torch.cuda.synchronize()
        for k in dsa.PROFILE_KERNELS:
            ms, n = dsa.profile_read(k)
            if n and k not in roof_kernels:
                kernels[k] = {"launches_per_step": n / extra, "ms_per_launch": ms / n, "ms_per_step": ms / extra}
        dsa.profile_enable(False)
    # The same step captured once in a HIP graph and replayed (no timing events inside).
    graph_ms = graph_ms_per_step(step, args.steps, args.warmup) if args.graph else None

    value = wl.L / (ms_per_step / 1000.0)
    sizes = workload_sizes(wl)
    f_idx = sum(r[0] for r in sizes)
    f_attn = sum(r[1] for r in sizes)
    b_attn = sum(r[2] for r in sizes)
    b_topk = 20 * wl.L * wl.top_k
    t_roof_ms = (f_idx / (PEAK_BF16_TFLOPS * 1e12) + b_topk / (PEAK_HBM_GBS * 1e9)
                 + max(f_attn / (PEAK_BF16_TFLOPS * 1e12), b_attn / (PEAK_HBM_GBS * 1e9))) * 1e3

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(ms_median, 4),
        "ms_per_step_min_max": [round(step_ms[0], 4), round(step_ms[-1], 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: N={wl.N} cached keys, L={wl.L} newest queries, top_k={wl.top_k}, "
                        f"indexer 32x128 bf16 ({wl.indexer} keys), attention {wl.H} heads x 576/512 bf16, "
                        f"q_block={args.q_block}",
            "N": wl.N, "L": wl.L, "top_k": wl.top_k, "attn_heads": wl.H, "q_block": args.q_block,
            "parallelism": "single GPU",
        },
        "step_roofline_frac": round(t_roof_ms / ms_per_step, 4),
        "selection": selection,
    }
    if kernels:
        per = {}
        sf = kernels.get("score_filter")
        at = kernels.get("sparse_attention")
        if sf:
            n = sf["launches_per_step"]
            ach = f_idx / n / (sf["ms_per_launch"] * 1e-3) / 1e12
            per["score_filter"] = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                                   "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                                   "traffic": measured_traffic("score_filter", wl.name),
                                   "ms_per_launch": round(sf["ms_per_launch"], 4)}
        if at:
            n = at["launches_per_step"]
            ach = b_attn / n / (at["ms_per_launch"] * 1e-3) / 1e9
            per["sparse_attention"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                                       "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                                       "traffic": measured_traffic("sparse_attention", wl.name),
                                       "ms_per_launch": round(at["ms_per_launch"], 4)}
        dom = max(per, key=lambda k: kernels[k]["ms_per_step"]) if per else None
        if dom:
            r = dict(per[dom])
            r["kernel"] = dom
            result["roofline"] = r
        result["kernels"] = {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kernels.items()}
        if not args.no_ceilings:
            ceil = measured_ceilings(dsa, dev)
            result["measured_ceilings"] = ceil
            if "score_filter" in per:
                per["score_filter"]["frac_of_measured"] = round(
                    per["score_filter"]["achieved"] / ceil["mfma_bf16_random_1wave_per_simd_TFLOPs"], 4)
            if "sparse_attention" in per:
                per["sparse_attention"]["frac_of_measured"] = round(
                    per["sparse_attention"]["achieved"] / max(ceil["read_GBs"], ceil["read_nontemporal_GBs"]), 4)
        result["kernel_rooflines"] = per
        tah = topk_attention_hbm(kernels, b_topk, b_attn)
        if tah:
            result["topk_attention_hbm"] = tah
    if graph_ms is not None:
        result["graph"] = {"ms_per_step": round(graph_ms, 4), "tokens_per_s": round(wl.L / (graph_ms / 1000.0), 1)}
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(wl, inp, args.cpu_seconds)
        log(f"[bench] cpu baseline took {time.perf_counter() - t0:.1f} s")
    print(json.dumps(result), flush=True)


def bench_decode(args, wl, inp, dev):
    """Decode step at the configuration's cache: position N - 1 queries (L = 1)."""
    import numpy as np
    import torch

    import dsa_inputs as di
    import dsa_sparse_attention_indexer_amd as dsa

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    t = wl.L - 1
    pos = wl.pos0 + t
    q_idx, w = bf(inp["q_idx"][t:t + 1]), torch.from_numpy(inp["w"][t:t + 1].copy()).to(dev)
    q, k_idx, kv = bf(inp["q"][t:t + 1]), bf(inp["k_idx"]), bf(inp["kv"])
    idx = torch.empty((1, wl.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((1, wl.H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dsa.workspace_bytes(1, wl.N, wl.top_k, 0), dtype=torch.uint8, device=dev)
    cws = torch.empty(dsa.cached_workspace_bytes(1, wl.N, wl.top_k, 0), dtype=torch.uint8, device=dev)
    dws = torch.empty(max(dsa.decode_workspace_bytes(1, wl.H, wl.top_k, 0), 1), dtype=torch.uint8, device=dev)
    scale = float(np.float32(di.SOFTMAX_SCALE))
    # The cache holds the N-1 older keys; each step appends the newest one, then selects.
    cache = dsa.KeyCache(wl.N)
    cache.append(k_idx, wl.N - 1)

    def step():
        cache.n = wl.N - 1
        cache.append(k_idx)
        dsa.indexer_topk_cached(q_idx, k_idx, w, pos, wl.top_k, cache, out=idx, workspace=cws)
        dsa.sparse_decode(q, kv, idx, pos, scale, out=out, workspace=dws)

    def step_relayout():  # the same step laying out all N keys again
        dsa.indexer_topk(q_idx, k_idx, w, pos, wl.top_k, out=idx, workspace=ws)
        dsa.sparse_decode(q, kv, idx, pos, scale, out=out, workspace=dws)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1000.0 / args.steps

    ms_per_step = timed(step)
    relayout_ms = timed(step_relayout)
    # Per-kernel times in a pass of their own (events around every launch cost a few us a step).
    dsa.profile_enable(True)
    for k in dsa.PROFILE_KERNELS:
        dsa.profile_read(k)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kernels = {}
    for k in dsa.PROFILE_KERNELS:
        ms, n = dsa.profile_read(k)
        if n:
            kernels[k] = {"launches_per_step": round(n / args.steps, 4), "ms_per_launch": round(ms / n, 5)}
    dsa.profile_enable(False)
    graph_ms = graph_ms_per_step(step, args.steps, args.warmup) if args.graph else None
    n_t = pos + 1
    f_idx = 2 * 32 * 128 * n_t
    b_attn = wl.top_k * 576 * 2 + 4 * wl.top_k + wl.H * 576 * 2 + wl.H * 512 * 2
    result = {
        "metric": f"decode steps/sec (key-cache append + L=1 indexer+topk + split sparse attn) at N={wl.N}, "
                  f"top-k={wl.top_k}",
        "value": round(1000.0 / ms_per_step, 1),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "relayout_ms_per_step": round(relayout_ms, 5),
        "config": {"workload": f"{wl.name} decode: query at position {pos} of N={wl.N} cached keys (the newest "
                               f"appended to the indexer key cache each step), top_k={wl.top_k}, attention "
                               f"{wl.H} heads x 576/512 bf16, split keys",
                   "N": wl.N, "L": 1, "top_k": wl.top_k, "attn_heads": wl.H},
        "kernels": kernels,
    }
    if graph_ms is not None:
        result["graph"] = {"ms_per_step": round(graph_ms, 5), "steps_per_s": round(1000.0 / graph_ms, 1)}
    sp = kernels.get("attn_split")
    sf = kernels.get("score_filter")
    if sp:
        ach = b_attn / (sp["ms_per_launch"] * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                              "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "attn_split"}
    if sf:
        ach = f_idx / (sf["ms_per_launch"] * 1e-3) / 1e12
        result["indexer_roofline"] = {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                                      "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 5),
                                      "kernel": "score_filter"}
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        t0 = time.perf_counter()
        sel = oracle.topk(inp["q_idx"][t:t + 1], inp["k_idx"], inp["w"][t:t + 1], pos, wl.top_k)
        oracle.attention(inp["q"][t:t + 1], inp["kv"], sel, pos, di.SOFTMAX_SCALE)
        secs = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(1.0 / secs, 3), "unit": "steps/s", "cores": 1, "kind": "oracle",
                                  "sample": f"one decode step (1 query over {n_t} keys), fp64 C oracle: "
                                            f"full-sort top-k + sparse attention; {secs:.2f} s"}
    print(json.dumps(result), flush=True)


def bench_pack(args, wl, inp, dev):
    """Attention only: dsa_sparse_prefill vs dsa_sparse_prefill_packed on overlapping index rows."""
    import numpy as np
    import torch

    import dsa_inputs as di
    import dsa_sparse_attention_indexer_amd as dsa

    rng = di.make_rng(wl.seed + 77)
    idx_h = di.overlapping_topk_indices(rng, wl.L, wl.N, wl.top_k, wl.pos0, args.pack)
    pairs = idx_h[0::2][: wl.L // 2], idx_h[1::2][: wl.L // 2]
    union = np.mean([np.union1d(a[a >= 0], b[b >= 0]).size for a, b in zip(*pairs)])
    shared = float(np.mean([np.intersect1d(a, b).size for a, b in zip(*pairs)])) / wl.top_k

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, kv, idx = bf(inp["q"]), bf(inp["kv"]), torch.from_numpy(idx_h).to(dev)
    out = torch.empty((wl.L, wl.H, 512), dtype=torch.bfloat16, device=dev)
    scale = float(np.float32(di.SOFTMAX_SCALE))
    res = {}
    for pack in (False, True):
        for _ in range(args.warmup):
            dsa.sparse_prefill(q, kv, idx, wl.pos0, scale, out=out, pack=pack)
        torch.cuda.synchronize()
        dsa.profile_enable(True)
        dsa.profile_read("sparse_attention")
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dsa.sparse_prefill(q, kv, idx, wl.pos0, scale, out=out, pack=pack)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1000.0 / args.steps
        kms, n = dsa.profile_read("sparse_attention")
        dsa.profile_enable(False)
        res["packed" if pack else "unpacked"] = {"ms_per_step": round(ms, 4), "kernel_ms_per_step": round(kms / args.steps, 4),
                                                 "tokens_per_s": round(wl.L / (ms / 1000.0), 1)}
    result = {
        "metric": f"sparse attention tokens/sec with and without neighbour packing, {wl.name} shapes",
        "value": res["packed"]["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name} attention: L={wl.L} queries, top_k={wl.top_k}, {wl.H} heads; each index "
                               f"row keeps {args.pack} of the previous row's keys", "keep": args.pack},
        "pair_shared_fraction": round(shared, 4),
        "pair_union_rows": round(float(union), 1),
        "runs": res,
        "speedup": round(res["unpacked"]["ms_per_step"] / res["packed"]["ms_per_step"], 4),
    }
    print(json.dumps(result), flush=True)


def bench_retrieval(args, dev):
    """One step = dsa_retrieval_topk of M queries over an N-row corpus."""
    import numpy as np
    import torch

    import dsa_inputs as di
    import dsa_sparse_attention_indexer_amd as dsa

    M, N, k = args.retrieval_m, args.retrieval_n, args.retrieval_k
    t0 = time.perf_counter()
    rng = di.make_rng(90)
    qb = di.f32_to_bf16_bits(rng.standard_normal((M, 128), dtype=np.float32))
    xb = di.f32_to_bf16_bits(rng.standard_normal((N, 128), dtype=np.float32))
    log(f"[bench] retrieval: inputs generated in {time.perf_counter() - t0:.1f} s")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, x = bf(qb), bf(xb)
    out = torch.empty((M, k), dtype=torch.int32, device=dev)
    ws = torch.empty(dsa.retrieval_workspace_bytes(M, N, k), dtype=torch.uint8, device=dev)

    def step():
        dsa.retrieval_topk(q, x, k, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    dsa.profile_enable(True)
    for kname in dsa.PROFILE_KERNELS:
        dsa.profile_read(kname)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    kernels = {}
    for kname in dsa.PROFILE_KERNELS:
        kms, n = dsa.profile_read(kname)
        if n:
            kernels[kname] = {"launches_per_step": round(n / args.steps, 4), "ms_per_launch": round(kms / n, 5),
                              "ms_per_step": round(kms / args.steps, 5)}
    dsa.profile_enable(False)
    flops = 2.0 * M * N * 128
    result = {
        "metric": f"vector-retrieval queries/sec (exact inner-product top-{k}) over N={N} rows of 128 bf16",
        "value": round(M / (ms / 1000.0), 1),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"retrieval: M={M} Gaussian queries x N={N} Gaussian corpus rows, dim 128 bf16, "
                               f"top_k={k}", "M": M, "N": N, "top_k": k},
        "kernels": kernels,
    }
    sf = kernels.get("retr_filter")
    if sf:
        ach = flops / sf["launches_per_step"] / (sf["ms_per_launch"] * 1e-3) / 1e12
        result["roofline"] = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                              "kernel": "retr_filter"}
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        t0 = time.perf_counter()
        oracle.retrieval_topk(qb[:1], xb, k, n_threads=1)
        secs = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(1.0 / secs, 3), "unit": "queries/s", "cores": 1, "kind": "oracle",
                                  "sample": f"one query over all {N} rows, fp64 C oracle: full sort; {secs:.2f} s"}
    print(json.dumps(result), flush=True)


# Batches of sequences (N keys, L newest queries each; top_k 2048, 64 attention heads).
BATCHES = {
    # eight sequences of the 16K-key, 512-query chunk
    "prefill8": [(16384, 512)] * 8,
    # one chunk of each size, 2K .. 128K keys
    "ragged": [(131072, 2048), (65536, 1024), (16384, 512), (8192, 128), (2048, 64), (40000, 7)],
    # a decode step over 64 sequences, caches of 4K .. 32K keys
    "decode64": [(4096 + 448 * i, 1) for i in range(64)],
}


def bench_batch(args, dev):
    """One step = dsa_indexer_topk_varlen + dsa_sparse_prefill_varlen over the whole batch."""
    import numpy as np
    import torch

    import dsa_inputs as di
    import dsa_sparse_attention_indexer_amd as dsa

    top_k, H = 2048, 64
    specs = BATCHES[args.batch]
    t0 = time.perf_counter()
    seqs = []
    for i, (N, L) in enumerate(specs):
        wl = di.Workload(f"{args.batch}{i}", N, L, top_k, H, 50 + i, "concentrated")
        seqs.append((wl, di.make_inputs(wl)))
    log(f"[bench] batch {args.batch}: inputs generated in {time.perf_counter() - t0:.1f} s")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    cat = lambda key: np.concatenate([inp[key] for _, inp in seqs])
    q_idx, k_idx, q, kv = bf(cat("q_idx")), bf(cat("k_idx")), bf(cat("q")), bf(cat("kv"))
    w = torch.from_numpy(cat("w")).to(dev)
    cu_q = np.cumsum([0] + [wl.L for wl, _ in seqs]).astype(np.int64)
    cu_k = np.cumsum([0] + [wl.N for wl, _ in seqs]).astype(np.int64)
    pos0 = np.array([wl.pos0 for wl, _ in seqs], dtype=np.int64)
    T = int(cu_q[-1])
    splits = 0 if T < 512 else 1
    idx = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dsa.varlen_workspace_bytes(cu_q, cu_k, pos0, top_k), dtype=torch.uint8, device=dev)
    aws = torch.empty(max(dsa.prefill_varlen_workspace_bytes(cu_q, cu_k, pos0, H, top_k, splits), 1),
                      dtype=torch.uint8, device=dev)
    scale = float(np.float32(di.SOFTMAX_SCALE))

    def batched():
        dsa.indexer_topk_varlen(q_idx, k_idx, w, cu_q, cu_k, pos0, top_k, out=idx, workspace=ws)
        dsa.sparse_prefill_varlen(q, kv, idx, cu_q, cu_k, pos0, scale, splits=splits, out=out, workspace=aws)

    # The same work as one call per sequence (views into the packed tensors).
    one_ws = torch.empty(max(dsa.workspace_bytes(wl.L, wl.N, top_k) for wl, _ in seqs), dtype=torch.uint8,
                         device=dev)
    one_dws = torch.empty(max(max(dsa.decode_workspace_bytes(wl.L, H, top_k) for wl, _ in seqs), 1),
                          dtype=torch.uint8, device=dev)

    def per_sequence():
        for b, (wl, _) in enumerate(seqs):
            qs, ks = slice(cu_q[b], cu_q[b + 1]), slice(cu_k[b], cu_k[b + 1])
            dsa.indexer_topk(q_idx[qs], k_idx[ks], w[qs], wl.pos0, top_k, out=idx[qs], workspace=one_ws)
            if wl.L < 512:
                dsa.sparse_decode(q[qs], kv[ks], idx[qs], wl.pos0, scale, out=out[qs], workspace=one_dws)
            else:
                dsa.sparse_prefill(q[qs], kv[ks], idx[qs], wl.pos0, scale, out=out[qs])

    def timed(fn, kernels_too):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        if kernels_too:
            dsa.profile_enable(True)
            for k in dsa.PROFILE_KERNELS:
                dsa.profile_read(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1000.0 / args.steps
        kern = {}
        if kernels_too:
            for k in dsa.PROFILE_KERNELS:
                kms, n = dsa.profile_read(k)
                if n:
                    kern[k] = {"launches_per_step": round(n / args.steps, 4), "ms_per_launch": round(kms / n, 5),
                               "ms_per_step": round(kms / args.steps, 5)}
            dsa.profile_enable(False)
        return ms, kern

    ms_one, _ = timed(per_sequence, False)
    ms, kernels = timed(batched, True)
    graph_ms = graph_ms_per_step(batched, args.steps, args.warmup) if args.graph else None
    f_idx = sum(sum(r[0] for r in workload_sizes(wl)) for wl, _ in seqs)
    b_attn = sum(sum(r[2] for r in workload_sizes(wl)) for wl, _ in seqs)
    result = {
        "metric": f"batched prefill tokens/sec (indexer+topk+sparse attn), batch '{args.batch}'",
        "value": round(T / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.batch}: {len(seqs)} sequences (N, L) = "
                               f"{[(wl.N, wl.L) for wl, _ in seqs][:8]}{' ...' if len(seqs) > 8 else ''}, "
                               f"top_k={top_k}, indexer 32x128 bf16, attention {H} heads x 576/512 bf16, "
                               f"splits={splits}",
                   "sequences": len(seqs), "query_rows": T, "keys": int(cu_k[-1]), "top_k": top_k},
        "per_sequence_calls": {"ms_per_step": round(ms_one, 4), "tokens_per_s": round(T / (ms_one / 1000.0), 1)},
        "kernels": kernels,
    }
    if graph_ms is not None:
        result["graph"] = {"ms_per_step": round(graph_ms, 4), "tokens_per_s": round(T / (graph_ms / 1000.0), 1)}
    per = {}
    sf = kernels.get("score_filter")
    if sf:
        ach = f_idx / sf["launches_per_step"] / (sf["ms_per_launch"] * 1e-3) / 1e12
        per["score_filter"] = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                               "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                               "kernel": "score_filter"}
    at = kernels.get("sparse_attention") or kernels.get("attn_split")
    if at:
        ach = b_attn / at["launches_per_step"] / (at["ms_per_launch"] * 1e-3) / 1e9
        per["attention"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                            "kernel": "sparse_attention" if "sparse_attention" in kernels else "attn_split"}
    if per:
        dom = max(per, key=lambda k: kernels[per[k]["kernel"]]["ms_per_step"])
        result["roofline"] = per[dom]
        result["kernel_rooflines"] = per
    if not args.no_cpu_baseline:
        import oracle

        oracle.build(force=False)
        t0 = time.perf_counter()
        n_rows = 0
        for wl, inp in seqs[:8]:  # the newest query of up to 8 sequences
            t = wl.L - 1
            sel = oracle.topk(inp["q_idx"][t:t + 1], inp["k_idx"], inp["w"][t:t + 1], wl.pos0 + t, top_k)
            oracle.attention(inp["q"][t:t + 1], inp["kv"], sel, wl.pos0 + t, di.SOFTMAX_SCALE)
            n_rows += 1
        secs = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(n_rows / secs, 3), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the newest query of {n_rows} sequences, fp64 C oracle: full-sort "
                                            f"top-k + sparse attention; {secs:.2f} s"}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
