"""Benchmark of the paged BF16 KV-cache decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]

One step = for each of the 16 layers: paged_kv_append (RoPE + page write)
then paged_decode_attn (split phase + log-sum-exp combine), all on one HIP
stream, over a seeded synthetic batch already resident in HBM (default: 64
sequences x 2,048-token context x 16 layers, 4 GiB of KV in one page pool).
Prints ONE JSON line.  ``value`` is the KV bytes the attention must read per
step (K and V of every valid token, every layer) divided by the wall time of
the whole step.  The ``roofline`` entry is for the dominant kernel, the split
phase, timed with HIP events on the launch stream.  ``cpu_baseline`` is the
FP64 oracle (append + attention) timed on the host cores over a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "paged decode attn: KV-read HBM GB/s (% of MI355X peak); seq·layers/s"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_split_kernel_cfg3_counters.json")
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_cache_172_amd", "csrc", "kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def split_bytes_per_launch(ctx: np.ndarray, splits: int) -> int:
    """Algorithmic bytes of one split-phase launch (one layer): K and V of
    valid tokens, q' (BF16), the table entries read, and the partial results
    written (or the FP32 output when there is a single chunk)."""
    n = ctx.astype(np.int64)
    pages = -(-n // 16)
    kv = int(n.sum()) * 2048
    q = ctx.size * 4096
    table = int(pages.sum()) * 4
    outw = ctx.size * (8192 if splits == 1 else splits * 32 * 66 * 4)
    return kv + q + table + outw


def kernel_source_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(splits: int):
    """HBM bytes per split launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    try:
        with open(COUNTERS_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha") != kernel_source_sha() or c.get("splits") != splits:
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(batch, spec, q0, k0, v0, rope, budget_s: float):
    """Time the FP64 oracle (append + attention) on whole (layer, sequence)
    units of this workload: one unit on one thread to size the sample, then a
    bounded sample spread over the host threads."""
    import concurrent.futures
    import oracle
    from oracle import PoolView
    from tests.gpu_util import gather_units

    orc = oracle.default()
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    rng = np.random.default_rng(1720)
    L, B = spec.num_layers, spec.num_seqs
    all_units = [(int(rng.integers(L)), int(rng.integers(B))) for _ in range(4 * threads)]

    def run_unit(u, data):
        pages, bt, ctx, _ = data
        layer, s = u
        n = int(ctx[0])
        q = q0[layer, s][None].copy()
        pv = PoolView.from_pages(pages)
        orc.append(pv, bt, ctx, q, np.ascontiguousarray(k0[layer, s][None]),
                   np.ascontiguousarray(v0[layer, s][None]), rope[0], rope[1])
        orc.attn(pv, bt, ctx, q, 0.125)
        return n

    data = {u: gather_units(batch, [u]) for u in all_units}
    t0 = time.perf_counter()
    run_unit(all_units[0], data[all_units[0]])
    one = time.perf_counter() - t0
    n_units = int(max(threads, min(len(all_units), budget_s * threads / max(one, 1e-3))))
    n_units = max(threads, (n_units // threads) * threads)
    sample = all_units[:n_units]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        ns = list(ex.map(lambda u: run_unit(u, data[u]), sample))
    wall = time.perf_counter() - t0
    kv = sum(ns) * 2048
    return {
        "value": round(kv / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(sample)} (layer, sequence) units of this workload, each FP64 append "
                   f"+ attention over its full context, spread over {threads} host threads"),
        "seq_layers_per_s": round(len(sample) / wall, 3),
        "seconds": round(wall, 2),
        "one_unit_one_thread_s": round(one, 3),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this decode-step library has no multi-GPU "
              "path (one GPU's share is the benchmark); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_172_amd as pkv
    from paged_kv_cache_172_amd import pages as pg
    from paged_kv_cache_172_amd import workload as wl
    from paged_kv_cache_172_amd.runner import DecodeBatch, rope_table_host

    pkv.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    spec = wl.config_spec(a.config)
    log(f"[bench] config {a.config}: {spec.name}; building {spec.num_pages} pages on the GPU")
    pool = wl.make_device_pool(spec)
    q0, k0, v0 = wl.draw_new_tokens(spec)
    bt = spec.block_tables.copy()
    free_stats = None
    if len(spec.crossers):
        free = pg.FreeList(spec.free_pages, spec.num_pages)
        pg.lazy_page_step(bt, spec.ctx, free)
        free_stats = free.stats()
    rope = rope_table_host(wl.ROPE_THETA, wl.MAX_CONTEXT)
    batch = DecodeBatch(pool, bt, spec.ctx, q0, k0, v0, rope=rope, max_context_len=wl.MAX_CONTEXT)
    L = spec.num_layers
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def step(events=None):
        for layer in range(L):
            batch.append(layer, stream)
            if events is not None:
                events[layer][0].record(stream)
            batch.attn_split(layer, stream)
            if events is not None:
                events[layer][1].record(stream)
            batch.attn_combine(layer, stream)
            if events is not None:
                events[layer][2].record(stream)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({a.warmup} steps); timing {a.steps} steps")
    evs = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(L)]
           for _ in range(a.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(a.steps):
        step(evs[k])
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / a.steps
    split_ms = [e[0].elapsed_time(e[1]) for st in evs for e in st]
    comb_ms = [e[1].elapsed_time(e[2]) for st in evs for e in st]
    split_avg = statistics.fmean(split_ms)
    comb_avg = statistics.fmean(comb_ms)
    attn_med = statistics.median([s + c for s, c in zip(split_ms, comb_ms)])
    assert torch.isfinite(batch.out).all(), "non-finite attention output"

    kv_step = spec.kv_bytes_per_step()
    kv_layer = kv_step / L
    splits = batch.splits
    alg = split_bytes_per_launch(spec.ctx, splits)
    achieved = alg / (split_avg * 1e-3) / 1e9
    traffic = measured_traffic(splits)
    result = {
        "metric": METRIC,
        "value": round(kv_step / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {
            "workload": f"config {a.config}: {spec.name}",
            "num_seqs": spec.num_seqs, "num_layers": L,
            "context_tokens": int(spec.ctx.max()), "pool_pages": spec.num_pages,
            "kv_bytes_per_step": kv_step, "splits": splits, "storage_dtype": "bf16",
            "parallelism": "single GPU",
        },
        "frac_of_peak": round(kv_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "seq_layers_per_s": round(spec.num_seqs * L / (ms_per_step * 1e-3), 1),
        "attn_only": {
            "kv_gbps": round(kv_layer / (attn_med * 1e-3) / 1e9, 2),
            "frac_of_peak": round(kv_layer / (attn_med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "us_per_layer_median": round(attn_med * 1e3, 2),
            "seq_layers_per_s": round(spec.num_seqs / (attn_med * 1e-3), 1),
        },
        "kernels_us_avg": {"attn_split": round(split_avg * 1e3, 2),
                           "attn_combine": round(comb_avg * 1e3, 2)},
        "roofline": {
            "kernel": "attn_split_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg,
            "avg_launch_us": round(split_avg * 1e3, 2),
        },
    }
    if free_stats:
        result["free_list"] = free_stats
    if not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(batch, spec, q0, k0, v0, rope, a.cpu_budget_s)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
