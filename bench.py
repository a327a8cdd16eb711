"""Benchmark of the paged BF16 KV-cache decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]

One step = for each of the 16 layers, the append of the new token (RoPE +
page write) and the paged decode attention over the cache, over a seeded
synthetic batch already resident in HBM (default: 64 sequences x 2,048-token
context x 16 layers, 4 GiB of KV in one page pool).  The timed step issues
one paged_kv_append_decode_attn per layer (append and attention in one
launch); the same step as paged_kv_append + paged_decode_attn (two launches
per layer) is timed beside it.  Prints ONE JSON line.  ``value`` is the KV
bytes the attention must read per step (K and V of every valid token, every
layer) divided by the wall time of the whole step.  The ``roofline`` entry
is for the dominant kernel, the fused append + attention kernel, timed with
HIP events on the launch stream over back-to-back launches.  ``cpu_baseline``
is the FP64 oracle (append + attention) timed on the host cores over a
bounded sample of the same workload.
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
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_fused_kernel_cfg3_counters.json")
PREWARM_STEPS = 40    # untimed fused steps before the warmup (about 31 ms)
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


def append_bytes_per_launch(num_seqs: int) -> int:
    """Algorithmic bytes the fused kernel adds for the append: the new k and v
    rows read (8 heads x 64 BF16 each), the K and V rows written to the
    pages, and the two RoPE table rows (32 FP32 each); q is already counted
    by the attention."""
    return num_seqs * (2 * 1024 + 2 * 1024 + 2 * 128)


PREFILL_SEQS, PREFILL_TOKENS = 64, 2048


ROPE_TABLE_BYTES = 2 * 2048 * 32 * 4


def prefill_bytes_per_token(with_q: bool) -> int:
    """Algorithmic bytes of the prefill fill per prompt token: k and v rows
    read (1 KiB each), K' and V rows written into the pages (1 KiB each) and,
    with q, its row read and written back (4 KiB each).  The RoPE table is
    read once per launch (ROPE_TABLE_BYTES): rows are shared by every token
    at the same position."""
    return 4 * 1024 + (8 * 1024 if with_q else 0)


def time_prefill(torch, pkv, stream, rope_cos, rope_sin, reps: int):
    """The prefill page fill of 64 prompts x 2,048 tokens (one layer, q
    rotated) into a 256 MiB pool of its own, shuffled; average launch time
    from HIP events around back-to-back launches."""
    from paged_kv_cache_172_amd.runner import HALF_PAGE, PAGE_ELEMS
    dev = torch.device("cuda", 0)
    B, n = PREFILL_SEQS, PREFILL_TOKENS
    T = B * n
    P = T // 16
    g = torch.Generator(device=dev).manual_seed(172100)
    pages = torch.empty((P, 2, 8, 16, 64), dtype=torch.int16, device=dev)
    perm = torch.randperm(P, generator=g, device=dev).to(torch.int32)
    bt = perm.view(B, 128).contiguous()
    start = torch.zeros(B, dtype=torch.int32, device=dev)
    cu = (torch.arange(B + 1, device=dev, dtype=torch.int32) * n).contiguous()
    rows = lambda c: torch.randn((T, c), generator=g, device=dev).to(torch.bfloat16).view(torch.int16)
    q, k, v = rows(2048), rows(512), rows(512)
    base = pages.data_ptr()
    pool = pkv.make_pool(base, base + HALF_PAGE * 2, P, PAGE_ELEMS, 1024, 64)

    def launch():
        pkv.paged_kv_prefill(pool, bt, 128, start, cu, B, T, q, 2048, k, 512, v, 512,
                             rope_cos, rope_sin, rope_cos.shape[0], stream)

    for _ in range(2):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    alg = T * prefill_bytes_per_token(True) + ROPE_TABLE_BYTES
    gbps = alg / (us * 1e-6) / 1e9
    return {
        "workload": f"{B} prompts x {n} tokens, one layer, q rotated in place",
        "kernel": "append_kernel<true> (paged_kv_prefill)",
        "us_per_launch": round(us, 2),
        "tokens_per_s": round(T / (us * 1e-6), 1),
        "algorithmic_bytes_per_launch": alg,
        "gbps": round(gbps, 1),
        "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
    }


def time_continuous_batching(torch, stream, rope, reps: int):
    """The continuous-batching mix: 256 sequences x 16 layers, context lengths
    log-uniform in 16..2,048, 16 of them opening a page this step (lazy page
    step first).  The fused step, timed per layer, in four ways: the batch as
    given, ranked once per step by the library (paged_decode_attn_order, its
    launch inside the timed step) and followed by every layer's call
    (``given_order``); the batch as given with no order
    (``given_order_unranked``); sorted longest-first by the caller
    (``longest_first``); and laid out by the caller in the library's start
    order computed on the host (paged_decode_attn_order_host,
    ``host_order``).  The kernels' results do not depend on the order;
    with 2,048 (sequence, KV head) workgroups, twice what the GPU holds at
    once, the order sets the tail."""
    from paged_kv_cache_172_amd import pages as pg, workload as wl
    from paged_kv_cache_172_amd.runner import DecodeBatch
    spec = wl.config_spec(4)
    pool = wl.make_device_pool(spec)
    q0, k0, v0 = wl.draw_new_tokens(spec)
    bt = spec.block_tables.copy()
    if len(spec.crossers):
        pg.lazy_page_step(bt, spec.ctx, pg.FreeList(spec.free_pages, spec.num_pages))
    L = spec.num_layers
    kv_layer = spec.kv_bytes_per_step() / L
    res = {"workload": f"{spec.num_seqs} sequences x {L} layers, context log-uniform 16..2048 "
                       f"(sum {int(spec.ctx.sum())} tokens per layer)",
           "kv_bytes_per_layer": int(kv_layer)}
    longest = np.argsort(-spec.ctx, kind="stable")
    from paged_kv_cache_172_amd import _lib
    host_order = _lib.paged_decode_attn_order_host(spec.ctx, wl.MAX_CONTEXT,
                                                   _lib.paged_decode_attn_order_round())
    for name, perm, ranked in (("given_order", None, True), ("given_order_unranked", None, False),
                               ("longest_first", longest, False), ("host_order", host_order, False)):
        if perm is None:
            args = (bt, spec.ctx, q0, k0, v0)
        else:
            args = (np.ascontiguousarray(bt[:, perm]), np.ascontiguousarray(spec.ctx[perm]),
                    *(np.ascontiguousarray(x[:, perm]) for x in (q0, k0, v0)))
        b = DecodeBatch(pool, *args, rope=rope, max_context_len=wl.MAX_CONTEXT)
        # Untimed steps first, as many as the headline's: the first leg on
        # this pool keeps speeding up for about 20 steps (0.15 us per layer
        # more with 40 steps than with 10).
        for _ in range(PREWARM_STEPS):
            b.step_fused(stream, order=ranked)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            b.step_fused(stream, order=ranked)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / (reps * L) * 1e3
        res[name] = {"us_per_layer": round(us, 2), "kv_gbps": round(kv_layer / (us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(kv_layer / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "library_order": ranked}
        del b
    del pool
    torch.cuda.empty_cache()
    return res


def time_prefix_sharing(torch, pkv, stream, reps: int):
    """64 sequences of 2,048 tokens whose first 1,024 tokens are one shared
    prompt, tables built by the native pager (one layer): live pages with and
    without sharing, and the attention over the shared layout."""
    import numpy as np
    from paged_kv_cache_172_amd import pages as pg
    from paged_kv_cache_172_amd.runner import HALF_PAGE, PAGE_ELEMS
    dev = torch.device("cuda", 0)
    B, n, shared = 64, 2048, 1024
    pool_pages = B * n // 16          # credits: admission does not count on sharing
    pager = pg.Pager(pool_pages, 1)
    ids = [pager.submit(n, 1)[0] for _ in range(B)]
    assert pager.admit() == ids
    tables = np.full((B, 1, 128), -1, np.int32)
    pager.reserve(ids[0], shared, tables[0])
    for i in range(1, B):
        pager.share_prefix(ids[0], ids[i], shared, tables[i])
    assert pager.decode_step(ids, [n] * B, tables) == []
    st = pager.stats()
    g = torch.Generator(device=dev).manual_seed(172200)
    pool_t = torch.randn((pool_pages, 2, 8, 16, 64), generator=g, device=dev).to(torch.bfloat16)
    pool_t = pool_t.view(torch.int16)
    base = pool_t.data_ptr()
    pool = pkv.make_pool(base, base + HALF_PAGE * 2, pool_pages, PAGE_ELEMS, 1024, 64)
    bt = torch.from_numpy(np.ascontiguousarray(tables[:, 0])).to(dev)
    ctx = torch.full((B,), n, dtype=torch.int32, device=dev)
    q = torch.randn((B, 2048), generator=g, device=dev).to(torch.bfloat16).view(torch.int16)
    out = torch.empty((B, 2048), dtype=torch.float32, device=dev)

    def launch():
        pkv.paged_decode_attn_split(pool, bt, 128, ctx, B, n, q, 2048, 0.125, out, 2048, None, 0,
                                    stream)

    launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        launch()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    logical = B * n * 2048
    return {
        "workload": f"{B} sequences x {n} tokens, the first {shared} shared, one layer",
        "live_pages_shared": st["live_pages"],
        "live_pages_unshared": B * n // 16,
        "shared_refs": st["shared_refs"],
        "attn_us": round(us, 2),
        "logical_kv_gbps": round(logical / (us * 1e-6) / 1e9, 1),
        "hbm_kv_bytes": st["live_pages"] * 16 * 2048,
    }


def time_graph_step(torch, step, reps: int, layers: int):
    """The same step captured once in a HIP graph and replayed: the graph
    holds the step's launches and nothing else (no memory operations), and
    replaying it submits them all at once.  `step(stream)` enqueues one step
    on the stream it is given; capture and replay use a stream of their own
    (capture cannot run on the default stream)."""
    cap = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        step(cap)
    with torch.cuda.stream(cap):
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(cap)
        for _ in range(reps):
            g.replay()
        e1.record(cap)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del g
    return {"ms_per_step": round(ms, 4), "us_per_layer": round(ms / layers * 1e3, 2)}


def kernel_source_sha() -> str:
    """Hash of the kernel source's code: comments and the layout of
    whitespace do not count, so that editing a comment keeps the measured
    counters valid."""
    import re
    with open(KERNEL_SOURCE, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()[:16]


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


THREAD_CAP = 16      # a GPU machine's CPU share for one GPU


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(pages, bt_all, ctx_all, q0, k0, v0, rope, budget_s: float,
                 one_core_budget_s: float = 3.0, what: str = "step"):
    """Time the FP64 oracle (append + attention) on whole (layer, sequence)
    units of a workload, reading a host copy of its pool.

    Two figures, both with the same plain single-threaded oracle calls:
      - one core: units run one after another on one thread for about
        one_core_budget_s seconds;
      - N threads: a bounded sample (about budget_s seconds of CPU work, at
        most every unit once) spread over min(host cores, THREAD_CAP)
        threads, each unit one call.
    The oracle writes each unit's new K/V row into the host pool (the same
    bits the GPU wrote there), so repeated units do identical work."""
    import concurrent.futures
    import oracle
    from oracle import PoolView

    orc = oracle.default()
    host_cores = len(os.sched_getaffinity(0))
    threads = max(1, min(THREAD_CAP, host_cores))
    pool = PoolView.from_pages(pages)
    L, B = bt_all.shape[0], bt_all.shape[1]
    units = [(layer, s) for layer in range(L) for s in range(B)]
    np.random.default_rng(1720).shuffle(units)

    def run_unit(u):
        layer, s = u
        bt = np.ascontiguousarray(bt_all[layer, s][None])
        ctx = np.ascontiguousarray(ctx_all[s:s + 1])
        q = q0[layer, s][None].copy()
        orc.append(pool, bt, ctx, q, np.ascontiguousarray(k0[layer, s][None]),
                   np.ascontiguousarray(v0[layer, s][None]), rope[0], rope[1])
        orc.attn(pool, bt, ctx, q, 0.125)
        return int(ctx[0])

    # one core
    t0 = time.perf_counter()
    done, kv1 = 0, 0
    while done < len(units) and (done == 0 or time.perf_counter() - t0 < one_core_budget_s):
        kv1 += run_unit(units[done]) * 2048
        done += 1
    one_wall = time.perf_counter() - t0
    per_unit = one_wall / done
    # N threads, bounded sample
    n_units = int(min(len(units), max(threads, budget_s / max(per_unit, 1e-5))))
    sample = units[:n_units]
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        ns = list(ex.map(run_unit, sample))
    wall = time.perf_counter() - t0
    kv = sum(ns) * 2048
    return {
        "value": round(kv / wall / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(sample)} of the {len(units)} (layer, sequence) units of one {what}, "
                   f"each FP64 append + attention over its full context, on {threads} host "
                   f"threads (~{per_unit * len(sample):.2g} s of CPU work)"),
        "seq_layers_per_s": round(len(sample) / wall, 3),
        "seconds": round(wall, 3),
        "host_cores": host_cores,
        "thread_cap": THREAD_CAP,
        "cpu_model": cpu_model(),
        "one_core": {
            "value": round(kv1 / one_wall / 1e9, 4),
            "unit": "GB/s",
            "seq_layers_per_s": round(done / one_wall, 3),
            "units": done,
            "seconds": round(one_wall, 3),
        },
    }


def batch_cpu_baseline(batch, spec, q0, k0, v0, rope, budget_s, what="step"):
    pages = batch.pool_pages.cpu().numpy().view(np.uint16)
    return cpu_baseline(pages, batch.block_tables.cpu().numpy(), batch.context_lens_host, q0, k0,
                        v0, rope, budget_s, what=what)


def time_small_or_stress_config(torch, k: int, stream, rope, reps: int, cpu_budget_s):
    """Configs 1, 2 (latency of one layer's step; cache-resident, so not an
    HBM roofline) and 5 (1,024 sequences x 2,048 tokens, one layer, 4 GiB of
    KV; HBM-sized): the fused call, the two calls, and the attention alone,
    each as the average of back-to-back launches between two HIP events on
    the launch stream; with the oracle timed on the same workload."""
    from paged_kv_cache_172_amd import workload as wl
    from paged_kv_cache_172_amd.runner import DecodeBatch
    spec = wl.config_spec(k)
    if k == 5:
        pool = wl.make_device_pool(spec)
        q0, k0, v0 = wl.draw_new_tokens(spec)
    else:
        hw = wl.make_host_workload(spec)
        pool, q0, k0, v0 = hw.pages, hw.q, hw.k, hw.v
    b = DecodeBatch(pool, spec.block_tables, spec.ctx, q0, k0, v0, rope=rope,
                    max_context_len=wl.MAX_CONTEXT)
    del pool
    L = spec.num_layers
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    host_us = {}

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        t1 = time.perf_counter()
        e1.record(stream)
        torch.cuda.synchronize()
        # the host's own time to enqueue the calls (Python, ctypes, the
        # library's checks and the launch), per layer
        host_us[fn.__name__] = round((t1 - t0) / (reps * L) * 1e6, 2)
        return e0.elapsed_time(e1) / (reps * L) * 1e3      # us per layer

    def fused(s=stream):
        for layer in range(L):
            b.append_attn(layer, s)

    def unfused():
        for layer in range(L):
            b.append(layer, stream)
            b.attn(layer, stream)

    def attn():
        for layer in range(L):
            b.attn(layer, stream)

    def attn_two_phase():
        for layer in range(L):
            b.attn_split(layer, stream)
            b.attn_combine(layer, stream)

    us_f = timed(fused)
    us_u = timed(unfused)
    us_a = timed(attn)
    us_2 = timed(attn_two_phase)
    gfused = time_graph_step(torch, fused, reps, L)["us_per_layer"]
    host_main = dict(host_us)
    tight = None
    if k != 5 and int(spec.ctx.max()) < wl.MAX_CONTEXT:
        # the plan drawn from the batch's own longest context, which a serving
        # host knows: a 37-token sequence needs no split
        bt_ = DecodeBatch(b.pool_pages, spec.block_tables, spec.ctx, q0, k0, v0, rope=rope,
                          max_context_len=int(spec.ctx.max()))
        b_save, b = b, bt_
        tight = {"max_context_len": int(spec.ctx.max()), "splits": b.splits,
                 "fused_us_per_layer": round(timed(fused), 2),
                 "attn_us_per_layer": round(timed(attn), 2)}
        tight["host_enqueue_us_per_layer"] = {k: host_us[k] for k in ("fused", "attn")}
        b = b_save
        del bt_
    kv_layer = spec.kv_bytes_per_step() / L
    res = {
        "workload": f"config {k}: {spec.name}",
        "num_seqs": spec.num_seqs, "num_layers": L,
        "kv_bytes_per_layer": int(kv_layer),
        "splits": b.splits,
        "fused_us_per_layer": round(us_f, 2),
        "unfused_us_per_layer": round(us_u, 2),
        "attn_us_per_layer": round(us_a, 2),
        "attn_split_then_combine_us_per_layer": round(us_2, 2),
        "fused_graph_us_per_layer": gfused,
        "host_enqueue_us_per_layer": host_main,
        "kv_gbps_fused": round(kv_layer / (us_f * 1e-6) / 1e9, 1),
        "kv_gbps_attn": round(kv_layer / (us_a * 1e-6) / 1e9, 1),
    }
    if tight:
        res["plan_from_batch_max"] = tight
    if k == 5:
        alg = split_bytes_per_launch(spec.ctx, b.splits) + append_bytes_per_launch(spec.num_seqs)
        res["frac_of_peak_fused"] = round(kv_layer / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        res["frac_of_peak_attn"] = round(kv_layer / (us_a * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
        res["alg_frac_of_peak_fused"] = round(alg / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    else:
        res["note"] = "cache-resident: a latency, not an HBM roofline"
    if cpu_budget_s is not None:
        res["cpu_baseline"] = batch_cpu_baseline(b, spec, q0, k0, v0, rope, cpu_budget_s,
                                                 what="layer")
    del b
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--legs", default="all",
                    help="comma-separated measurement legs beside the headline step: prefill, "
                         "prefix, mix (config 4), configs (1, 2, 5); 'all' (default) or 'none'. "
                         "The headline step and its roofline are always timed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 8 device copies of 256 MiB (reference for HBM byte counters)")
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
    if a.copy_calibration:
        src = torch.ones(128 * 2 ** 20, dtype=torch.int16, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": 256 * 2 ** 20, "copies": 8}))
        return
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

    def step_fused(s=stream):
        for layer in range(L):
            batch.append_attn(layer, s)

    def step_unfused():
        for layer in range(L):
            batch.append(layer, stream)
            batch.attn(layer, stream)

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        """Wall time of reps calls of fn between two events on the stream
        (no events inside: an event record costs a few microseconds)."""
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(reps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps

    # Untimed pre-warm before the warmup proper: when sustained load starts,
    # the shader clock dips (to about 1.9 GHz, for about 10 ms, measured
    # between launches with the shader and constant clock counters) and then
    # holds 2.4 GHz.  A serving loop runs in the steady state, so the timed
    # steps start after the dip.
    for _ in range(PREWARM_STEPS):
        step_fused()
    for _ in range(a.warmup):
        step_unfused()
        step_fused()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({a.warmup} steps); timing {a.steps} steps")
    # Timed regions in order of importance: on a long run the GPU's kernel
    # times drift up by about 1 %, so the headline is taken first.  The
    # appends rotate q in place and rewrite the same slots, so every step
    # does identical work whatever the order.
    ms_per_step = timed(step_fused, a.steps)
    assert torch.isfinite(batch.out).all(), "non-finite attention output"
    # The distribution of steps, after the headline: an event recorded
    # between consecutive steps on the stream (no synchronize in between),
    # median and p10/p90 over the same number of steps.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(a.steps):
        step_fused()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(a.steps))
    # The timed step is nothing but the dominant kernel, L launches back to
    # back on one stream between two HIP events, so its average launch
    # duration is the step time / L (it matches the profiler's kernel time).
    # The plain split kernel is timed the same way, on its own.
    fused_avg = ms_per_step / L
    graph_leg = time_graph_step(torch, step_fused, a.steps, L)
    split_avg = timed(lambda: [batch.attn_split(layer, stream) for layer in range(L)], a.steps) / L
    ms_unfused = timed(step_unfused, a.steps)

    legs = {"prefill", "prefix", "mix", "configs"} if a.legs == "all" else \
        set() if a.legs == "none" else set(a.legs.split(","))
    prefill = (time_prefill(torch, pkv, stream, batch.rope_cos, batch.rope_sin, max(3, a.steps // 2))
               if "prefill" in legs else None)
    prefix = time_prefix_sharing(torch, pkv, stream, max(3, a.steps)) if "prefix" in legs else None
    mix = time_continuous_batching(torch, stream, rope, max(3, a.steps // 2)) if "mix" in legs else None

    kv_step = spec.kv_bytes_per_step()
    kv_layer = kv_step / L
    splits = batch.splits
    if splits > 1:
        log("[bench] note: this plan also launches the combine phase after each split phase")
    alg_split = split_bytes_per_launch(spec.ctx, splits)
    alg = alg_split + append_bytes_per_launch(spec.num_seqs)
    achieved = alg / (fused_avg * 1e-3) / 1e9
    traffic = measured_traffic(splits)
    result = {
        "metric": METRIC,
        "value": round(kv_step / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "prewarm_steps": PREWARM_STEPS,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "graph_step": graph_leg,
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
            "step": "paged_kv_append_decode_attn per layer",
            "parallelism": "single GPU",
        },
        "frac_of_peak": round(kv_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "seq_layers_per_s": round(spec.num_seqs * L / (ms_per_step * 1e-3), 1),
        "unfused_step": {
            "ms_per_step": round(ms_unfused, 4),
            "kv_gbps": round(kv_step / (ms_unfused * 1e-3) / 1e9, 2),
            "calls": "paged_kv_append + paged_decode_attn per layer",
        },
        "attn_only": {
            "kernel": "attn_split_kernel<false, false>",
            "kv_gbps": round(kv_layer / (split_avg * 1e-3) / 1e9, 2),
            "frac_of_peak": round(kv_layer / (split_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "alg_frac_of_peak": round(alg_split / (split_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "us_per_layer": round(split_avg * 1e3, 2),
            "seq_layers_per_s": round(spec.num_seqs / (split_avg * 1e-3), 1),
            "in_kernel_merge": splits > 1,
        },
        "roofline": {
            "kernel": "attn_split_kernel<true, true> (fused append + attention)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg,
            "avg_launch_us": round(fused_avg * 1e3, 2),
        },
    }
    for key, leg in (("prefill_fill", prefill), ("prefix_sharing", prefix),
                     ("continuous_batching", mix)):
        if leg is not None:
            result[key] = leg
    if free_stats:
        result["free_list"] = free_stats
    if not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = batch_cpu_baseline(batch, spec, q0, k0, v0, rope, a.cpu_budget_s)
    del batch, pool
    torch.cuda.empty_cache()
    others = {}
    for k in ((1, 2, 5) if "configs" in legs else ()):
        if k == a.config:
            continue
        log(f"[bench] config {k}")
        others[f"config{k}"] = time_small_or_stress_config(
            torch, k, stream, rope, reps=(200 if k < 5 else max(5, a.steps // 2)),
            cpu_budget_s=None if a.no_cpu_baseline else (3.0 if k < 5 else 6.0))
    if others:
        result["other_configs"] = others
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
