#!/usr/bin/env python3
"""Benchmark of the DFlash 2 path selector (dfs_select) on one MI355X.

One step = one dfs_select call over a whole batch of draft blocks (top-16 over the
vocabulary logits, the context gate, all pair scores and the walk), inputs
resident in HBM.  Prints one JSON line:
  value      draft blocks/s through dfs_select (blocks = sequences x one block each)
  roofline   the top-16 kernel (the dominant one): algorithmic bytes / its average
             time, against MI355X's 8 TB/s HBM peak
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, timed on
             this host's cores (a baseline, not the target)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/sec through dfs_select; top-16 HBM GB/s as % of peak"
HBM_PEAK_GBS = 8000.0
# Sources of the top-16 kernel; HBM traffic figures taken with rocprofv3 counters
# are reported only while these files hash to the value recorded with them.
TOPK_SOURCES = ["draft_selection_position_amd/csrc/topk.hip", "draft_selection_position_amd/csrc/dfs_device.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "topk_throughput_traffic.txt")


def topk_source_sha() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in TOPK_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """(fetch+write bytes per top-16 launch, record) from the committed counter summary, or None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256_16") != topk_source_sha() or rec.get("workload") != workload:
        return None
    return float(rec["hbm_bytes_per_launch"]), rec


def _kname(full: str) -> str:
    return full.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]


def summarize_rocprof(d: str) -> None:
    """Print per-kernel average durations and per-dispatch counters from a rocprofv3 csv directory."""
    import csv
    import glob

    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"## kernel stats ({os.path.relpath(path, d)})")
        print("| kernel | calls | avg us | min us | max us | % |")
        print("|---|---|---|---|---|---|")
        for r in csv.DictReader(open(path)):
            name = _kname(r["Name"])
            print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                  f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        agg = {}
        for r in csv.DictReader(open(path)):
            name = _kname(r["Kernel_Name"])
            key = (name, r["Counter_Name"], r.get("Grid_Size", ""))
            agg.setdefault(key, []).append(float(r["Counter_Value"]))
        print(f"## counters ({os.path.relpath(path, d)}), mean per dispatch")
        print("| kernel | counter | grid | dispatches | mean value |")
        print("|---|---|---|---|---|")
        for (name, cn, g), v in sorted(agg.items()):
            print(f"| {name} | {cn} | {g} | {len(v)} | {sum(v) / len(v):.1f} |")


def _affinity() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _oracle_worker(args):
    # One process of the CPU baseline: the oracle on some sequences, single-threaded.
    from threadpoolctl import threadpool_limits

    import oracle
    from workloads import make

    name, seqs = args
    with threadpool_limits(1):
        inp = make(name, seqs=seqs, threads=1)
        t0 = time.perf_counter()
        res = oracle.select(inp)
        dt = time.perf_counter() - t0
    return [(int(s), r.path.tolist(), r.margins.tolist()) for s, r in zip(seqs, res)], dt


def cpu_baseline(name: str, batch: int, target_cpu_s: float, workers: int) -> dict:
    """Time the oracle on a bounded sample of the workload's sequences (no GPU touched)."""
    import multiprocessing as mp

    probe, t1 = _oracle_worker((name, [0]))
    per_seq = max(t1, 1e-3)
    nseq = int(min(batch, max(workers, round(target_cpu_s / per_seq))))
    seqs = list(range(nseq))
    chunks = [seqs[i::workers] for i in range(workers) if seqs[i::workers]]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(len(chunks)) as pool:
        parts = pool.map(_oracle_worker, [(name, c) for c in chunks])
    wall = time.perf_counter() - t0
    rows = sorted([r for p, _ in parts for r in p])
    cpu_s = sum(dt for _, dt in parts)
    return {
        "value": nseq / wall,
        "unit": "blocks/s",
        "cores": len(chunks),
        "kind": "oracle",
        "sample": f"{nseq} of {batch} sequences of workload {name} (full V, L, d), "
                  f"{len(chunks)} worker processes x 1 thread, {cpu_s:.1f} CPU-s of oracle work "
                  f"(input generation excluded)",
        "single_core_blocks_per_s": 1.0 / per_seq,
        "_paths": {s: (p, m) for s, p, m in rows},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="throughput")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle CPU work of the baseline sample")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run device-to-device copies of this size (counter calibration)")
    ap.add_argument("--summarize-rocprof", metavar="DIR", help="print a summary of rocprofv3 csv output and exit")
    ap.add_argument("--graph", action="store_true",
                    help="also time dfs_select replayed from a captured HIP graph (one launch per step)")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs the selector on a single GPU; --gpus must be 1 "
              "(sequences are independent, so a multi-GPU run is batch sharding with no exchange)",
              file=sys.stderr)
        return 2

    import numpy as np

    from workloads import config_by_name, make

    cfg = config_by_name(args.workload)
    print(f"[bench] generating workload {cfg.name}: batch {cfg.batch} L {cfg.L} V {cfg.V} d {cfg.d}",
          file=sys.stderr, flush=True)
    inp = make(cfg)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline (before the GPU is touched)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg.name, cfg.batch, args.cpu_seconds, max(1, min(16, _affinity())))

    import torch

    import draft_selection_position_amd as dfs
    from tests.parity import upload

    dev = upload(inp)
    torch.cuda.synchronize()
    sel = dfs.Selector(cfg.batch, cfg.L, cfg.V, cfg.d, mode=cfg.walk, temperature=cfg.temperature,
                       seed=cfg.walk_seed,
                       logits_dtype=dev["logits"].dtype, act_dtype=dev["hidden"].dtype,
                       table_dtype=dev["A"].dtype)
    call = lambda: sel(dev["logits"], dev["hidden"], dev["prev_token"], dev["A"], dev["B"], dev["W_h"])  # noqa

    print(f"[bench] warmup {args.warmup}, timed {args.steps} dfs_select steps", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        call()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    blocks_per_s = cfg.batch / (ms_per_step * 1e-3)
    path = sel.path.cpu().numpy()

    # The dominant kernel alone: the top-16 pass over [batch*L, V], same stream.
    logits2d = dev["logits"].view(-1, cfg.V)
    rows = logits2d.shape[0]
    ws = torch.empty(max(1, dfs.topk_workspace_bytes(rows, cfg.V, logits2d.dtype)), dtype=torch.uint8,
                     device=logits2d.device)
    for _ in range(5):
        dfs.topk(logits2d, workspace=ws)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(args.steps):
        dfs.topk(logits2d, workspace=ws)
    ev1.record()
    torch.cuda.synchronize()
    topk_ms = ev0.elapsed_time(ev1) / args.steps
    topk_bytes = rows * cfg.V * logits2d.element_size()
    topk_gbs = topk_bytes / (topk_ms * 1e-3) / 1e9

    # Other steps alone, for the record.
    def timed(fn, n=max(20, args.steps // 4)):
        fn()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(n):
            fn()
        ev1.record()
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    hidden2d = dev["hidden"].view(-1, cfg.d)
    gate_ms = timed(lambda: dfs.gate(hidden2d, dev["W_h"]))
    idx, val = dfs.topk(logits2d, workspace=ws)
    g = dfs.gate(hidden2d, dev["W_h"])
    idx3, val3 = idx.view(cfg.batch, cfg.L, 16), val.view(cfg.batch, cfg.L, 16)
    pair_ms = timed(lambda: dfs.pair_scores(idx3, val3, dev["prev_token"], g, dev["A"], dev["B"]))

    graph_ms = None
    if args.graph:
        # One dfs_select captured into a graph on a side stream, then replayed: the
        # host submits one graph launch per step instead of the individual kernels.
        cs = torch.cuda.Stream()
        cs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cs):
            for _ in range(3):
                call()
        torch.cuda.current_stream().wait_stream(cs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        ev0.record()
        for _ in range(args.steps):
            graph.replay()
        ev1.record()
        torch.cuda.synchronize()
        graph_ms = ev0.elapsed_time(ev1) / args.steps
        if not torch.equal(sel.path.cpu(), torch.from_numpy(path)):
            raise RuntimeError("graph replay gave a different path than eager dfs_select")

    if args.calibrate_copy_mb > 0:
        n = args.calibrate_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device=logits2d.device).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    traffic = recorded_traffic(cfg.name)
    out = {
        "metric": METRIC,
        "value": blocks_per_s,
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": cfg.batch, "L": cfg.L, "V": cfg.V, "d": cfg.d, "k": 16,
                   "E": 256, "walk": cfg.walk, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": topk_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": topk_gbs / HBM_PEAK_GBS, "traffic": None if traffic is None else traffic[0],
                     "kernel": "topk_chunk_kernel", "bytes_per_launch": topk_bytes, "avg_ms": topk_ms},
        "step_ms": {"topk": topk_ms, "gate": gate_ms, "pair_scores": pair_ms, "select": ms_per_step},
        "host_wall_s": wall,
    }
    if graph_ms is not None:
        out["graph_replay"] = {"ms_per_step": graph_ms, "value": cfg.batch / (graph_ms * 1e-3)}
    if cpu is not None:
        paths = cpu.pop("_paths")
        mism = near = 0
        for s, (p, m) in paths.items():
            for t in range(cfg.L):
                if int(path[s, t]) != p[t]:
                    if m[t] < 1e-4:
                        near += 1
                    else:
                        mism += 1
                    break
        cpu["parity_sample"] = {"sequences": len(paths), "mismatched": mism, "near_tie_divergence": near}
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
