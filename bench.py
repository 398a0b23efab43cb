"""Benchmark of the paged FP8 MQA logits + threshold Top-k select hot path.

One step = one pmqa_fused_logits_select call over the whole batch of a
synthetic workload: one kernel launch that scores every visible (row, KV
position) pair, selects candidates and ties against the row thresholds, and
finishes every tile (fit test, radix-select repair, ranges and exact Top-k),
with every input already resident in HBM.  Each step gets its own pre-zeroed
counters and pristine thresholds (prepared before the timed region) and cycles
through `--replicas` copies of the KV pool, so no step finds its pool in the
256 MiB Infinity Cache.

Prints one JSON line:
  value          pairs/s: sum over rows of visible KV positions, per second
  rows_per_s     rows selected (and finalized) per second
  roofline       the call's kernel (the only launch of a step): algorithmic HBM
                 bytes per launch over its average launch time -- one HIP event
                 pair on the launch stream around the timed steps, divided by
                 the step count -- against 8 TB/s; traffic from the committed
                 rocprofv3 FETCH_SIZE / WRITE_SIZE summary when it was taken on
                 this kernel source
  cpu_baseline   the float64 CPU oracle on a bounded sample of the workload

    python bench.py [--steps K] [--warmup W] [--workload 3|4|5|prefill] [--path fused|unfused]
                    [--main-leg]   also time the same kernel without the finish stage
"""
import argparse
import hashlib
import itertools
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_fp8_mqa_amd as pm  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
GOLDEN = os.path.join(ROOT, "tests", "golden")
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SRC = os.path.join(ROOT, "paged_fp8_mqa_amd", "csrc", "pmqa_device.hip")
METRIC = "scored (row,KV position) pairs/sec and rows top-k selected/sec; % roofline"


def kernel_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def load_thresholds(cfg, wl):
    d = json.load(open(os.path.join(GOLDEN, f"thresholds_cfg{cfg}.json")))
    if d["fingerprint"] != W.fingerprint(wl):
        raise SystemExit(f"workload {wl.name} does not match its stored thresholds (generator drift)")
    return np.array(d["threshold_bits"], dtype=np.int32).view(np.float32)


def algorithmic_bytes(wl, path):
    """HBM bytes one launch must move at least: every visible KV position's 132
    bytes once per request, q and weights, the row thresholds/counters/ranges,
    and (unfused) the logits write and read."""
    kv = int(wl.seq_lens.astype(np.int64).sum()) * 132
    qw = wl.q.size + wl.weights.size * 4
    rows = wl.rows * (4 + 8 + 8)
    pairs = int(wl.row_ends().sum())
    extra = 8 * pairs if path == "unfused" else 0
    return kv + qw + rows + extra


def traffic_from_profiles(cfg, path):
    """Measured HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source."""
    f = os.path.join(PROFILES, "fused_traffic.json")
    if not os.path.exists(f):
        return None
    d = json.load(open(f))
    e = d.get(f"cfg{cfg}_{path}")
    if not e or e.get("kernel_src_sha") != kernel_hash():
        return None
    return e.get("hbm_bytes_per_launch")


def cpu_baseline(wl, thresholds, budget_s):
    """The oracle (float64 scores, full-sort Top-k) on the workload's requests in
    order, starting over after the last, until about budget_s seconds of CPU
    work."""
    import oracle
    from oracle.select import select_with_repair
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    ends = wl.row_ends()
    pairs = 0
    rows = 0
    reqs = 0
    live = [b for b in range(wl.batch) if int(wl.seq_lens[b]) > 0]
    t0 = time.perf_counter()
    for i in itertools.count():
        b = live[i % len(live)]
        L = int(wl.seq_lens[b])
        k, s = oracle.gather_request(wl.kv_fused, wl.block_tables[b], L, wl.block_size, 128)
        sc = oracle.request_scores(wl.q[b], k, s, wl.weights[b * wl.next_n:(b + 1) * wl.next_n])
        for t in range(wl.next_n):
            r = b * wl.next_n + t
            e = int(ends[r])
            select_with_repair(sc[t, :e].astype(np.float32), e, thresholds[r], wl.top_k, wl.capacity)
            pairs += e
            rows += 1
        reqs += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": pairs / dt, "unit": "pairs/s", "cores": int(cores), "kind": "oracle",
            "rows_per_s": rows / dt,
            "sample": f"{reqs} requests of {wl.name} in order, {reqs / len(live):.2f} passes over its {len(live)} "
                      f"non-empty requests ({pairs} pairs, {rows} rows) in {dt:.1f}s"}


def calibration_copy(args, dev):
    """With --calib-copy-mib: one plain elementwise kernel that reads and writes
    exactly that many MiB (torch's same-dtype copy_ may go to a DMA engine
    instead of a kernel), the yardstick for the HBM byte counters."""
    if not args.calib_copy_mib:
        return
    src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def bench_prefill(args, dev):
    """The prefill chunk through pmqa_prefill_select: one launch per step over
    prefill-shaped rows (tiles of 4 rows of one request, causal row ends).  Its
    keys (2.3 MB) stay in the caches across the tiles that share a request, so
    the bound is the FP8 MFMA work, 16384 FLOP per (row, key) pair."""
    wl = W.prefill_chunk()
    d = json.load(open(os.path.join(GOLDEN, "thresholds_prefill_chunk.json")))
    if d["fingerprint"] != W.prefill_fingerprint(wl):
        raise SystemExit("prefill workload does not match its stored thresholds (generator drift)")
    thr0 = np.array(d["threshold_bits"], dtype=np.int32).view(np.float32)
    R, T = wl.rows, wl.tiles
    pairs = int(np.maximum(wl.row_ends, 0).astype(np.int64).sum())
    q = torch.from_numpy(wl.q).to(dev)
    w = torch.from_numpy(wl.weights).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    treq = torch.from_numpy(wl.tile_requests).to(dev)
    re_ = torch.from_numpy(wl.row_ends).to(dev)
    kv = torch.from_numpy(wl.kv_fused).to(dev).view(wl.num_blocks, wl.block_size, 1, 132)
    total = args.warmup + args.steps
    thr_all = torch.from_numpy(np.tile(thr0, (total, 1))).to(dev)
    cnt_all = torch.zeros(total, R, 2, dtype=torch.int32, device=dev)
    cand = torch.empty(R, wl.top_k + wl.capacity, 2, dtype=torch.int32, device=dev)
    arrivals = torch.zeros(T, dtype=torch.int32, device=dev)
    ranges = torch.empty(2, R, dtype=torch.int32, device=dev)
    topk = torch.empty(R, wl.top_k, dtype=torch.int32, device=dev)
    ws = pm.make_workspace("fused", T, wl.tile_rows, wl.max_context, dev)
    stream = torch.cuda.current_stream()

    def step(i):
        pm.prefill_select(q, kv, w, bt, treq, re_, wl.tile_rows, wl.max_context, thr_all[i], cnt_all[i], cand,
                          wl.capacity, wl.top_k, arrivals, ranges, topk, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for j in range(args.steps):
        step(args.warmup + j)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    assert int(arrivals.abs().sum()) == 0, "arrivals not left zeroed"
    repaired = int((thr_all[-1].cpu().numpy().view(np.int32) != thr0.view(np.int32)).sum())
    calibration_copy(args, dev)
    flops = 2.0 * 64 * 128 * pairs
    tflops = flops / (ms_step / 1e3) / 1e12
    kv_bytes = int(wl.seq_lens.astype(np.int64).sum()) * 132
    out = {
        "metric": METRIC, "value": pairs / (ms_step / 1e3), "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3 x fp8_e4m3 -> f32", "data": "synthetic (seeded generators, workloads/)",
        "config": {"workload": wl.name, "path": "prefill", "tiles": T, "tile_rows": wl.tile_rows, "rows": R,
                   "pairs": pairs, "top_k": wl.top_k, "capacity": wl.capacity, "block_size": wl.block_size,
                   "parallelism": "single GPU"},
        "rows_per_s": R / (ms_step / 1e3),
        "repaired_rows": repaired,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / FP8_PEAK_TFLOPS, "traffic": None, "kernel": "fused_kernel<4>",
                     "launch_us": ms_step * 1e3, "flop_per_launch": flops,
                     "kv_bytes_per_launch_once": kv_bytes},
        "kernel_src_sha": kernel_hash(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = prefill_cpu_baseline(wl, thr0, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def prefill_cpu_baseline(wl, thresholds, budget_s):
    """The oracle on the prefill chunk's tiles in order, starting over after the
    last, until about budget_s seconds of CPU work."""
    import oracle
    from oracle.select import select_with_repair
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        cores = os.cpu_count()
    pairs = rows = tiles = 0
    t0 = time.perf_counter()
    for j in itertools.count():
        i = j % wl.tiles
        rs = list(range(i * wl.tile_rows, (i + 1) * wl.tile_rows))
        sc = oracle.prefill_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.tile_requests, wl.row_ends,
                                   wl.tile_rows, wl.block_size, wl.max_context, rows=rs)
        for r in rs:
            e = int(wl.row_ends[r])
            if e > 0:
                select_with_repair(sc[r, :e].astype(np.float32), e, thresholds[r], wl.top_k, wl.capacity)
                pairs += e
                rows += 1
        tiles += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": pairs / dt, "unit": "pairs/s", "cores": int(cores), "kind": "oracle", "rows_per_s": rows / dt,
            "sample": f"{tiles} tiles of {wl.name} in order, {tiles / wl.tiles:.2f} passes over its {wl.tiles} "
                      f"tiles ({pairs} pairs, {rows} rows) in {dt:.1f}s"}


def bench_logits(args, dev):
    """--path logits: pmqa_mqa_logits(_typed) alone on the workload, with the
    precisions of --dtypes (output,epi,acc).  HBM-bound: every visible key's
    132 bytes once per request, q and weights, and the logits written (4 or 2
    bytes per pair)."""
    wl = W.make(int(args.workload))
    names = args.dtypes.split(",")
    dt = {"f32": torch.float32, "f16": torch.float16}
    out_dt, epi_dt, acc_dt = (dt[n] for n in names)
    pairs = int(wl.row_ends().sum())
    q = torch.from_numpy(wl.q).to(dev)
    w = torch.from_numpy(wl.weights).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    kv_host = torch.from_numpy(wl.kv_fused)
    kvs = [kv_host.to(dev).view(wl.num_blocks, wl.block_size, 1, 132) for _ in range(args.replicas)]
    out = torch.empty(wl.rows, pm.padded_seq_len(wl.max_seq_len), dtype=out_dt, device=dev)

    def step(i):
        pm.mqa_logits(q, kvs[i % len(kvs)], w, bt, sl, wl.max_seq_len, out=out, output_dtype=out_dt,
                      epi_dtype=epi_dt, acc_dtype=acc_dt)

    for i in range(args.warmup):
        step(i)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for j in range(args.steps):
        step(args.warmup + j)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    out_bytes = 2 if out_dt == torch.float16 else 4
    alg = int(wl.seq_lens.astype(np.int64).sum()) * 132 + wl.q.nbytes + wl.weights.nbytes + pairs * out_bytes
    achieved = alg / (ms_step / 1e3) / 1e9
    line = {
        "metric": "scored (row,KV position) pairs/sec; % roofline (logits only)",
        "value": pairs / (ms_step / 1e3), "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"fp8_e4m3 x fp8_e4m3 -> acc {names[2]}, epilogue {names[1]}, out {names[0]}",
        "data": "synthetic",
        "config": {"workload": wl.name, "path": "logits", "dtypes": {"output": names[0], "epi": names[1],
                                                                      "acc": names[2]},
                   "pairs": pairs, "rows": wl.rows, "kv_replicas": args.replicas, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_launch": alg,
                     "kernel": "logits_kernel<%d>" % wl.next_n, "launch_us": ms_step * 1e3},
        "kernel_src_sha": kernel_hash(),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


FP4_PEAK_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA


def bench_fp4(args, dev):
    """--path fp4: pmqa_fp4_mqa_logits on the MXFP4 pool of the workload's
    shape (decode batch 3 or MTP batch 4), with --dtypes output,epi
    (default bf16,f32).  HBM-bound: every visible key's 68 bytes (64 value
    bytes, 4 scale bytes) once per request, q and its scales, weights, and the
    logits written."""
    wl = W.fp4_config(int(args.workload))
    names = args.dtypes.split(",") if args.dtypes != "f32,f32,f32" else ["bf16", "f32"]
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    out_dt, epi_dt = dt[names[0]], dt[names[1]]
    pairs = int(wl.row_ends().sum())
    q = torch.from_numpy(wl.q).to(dev)
    qsf = torch.from_numpy(wl.q_sf).to(dev)
    w = torch.from_numpy(wl.weights).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    kv_host = torch.from_numpy(wl.kv_fused)
    kvs = [kv_host.to(dev).view(wl.num_blocks, wl.block_size, 1, 68) for _ in range(args.replicas)]
    out = torch.empty(wl.rows, pm.padded_seq_len(wl.max_seq_len), dtype=out_dt, device=dev)

    def step(i):
        pm.fp4_mqa_logits(q, qsf, kvs[i % len(kvs)], w, bt, sl, wl.max_seq_len, out=out, output_dtype=out_dt,
                          epi_dtype=epi_dt)

    for i in range(args.warmup):
        step(i)
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for j in range(args.steps):
        step(args.warmup + j)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    out_bytes = 4 if out_dt == torch.float32 else 2
    alg = (int(wl.seq_lens.astype(np.int64).sum()) * 68 + wl.q.nbytes + wl.q_sf.nbytes + wl.weights.nbytes
           + pairs * out_bytes)
    achieved = alg / (ms_step / 1e3) / 1e9
    flops = 2.0 * 64 * 128 * pairs
    line = {
        "metric": "scored (row,KV position) pairs/sec; % roofline (MXFP4 logits)",
        "value": pairs / (ms_step / 1e3), "unit": "pairs/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"mxfp4 x mxfp4 -> f32 acc, epilogue {names[1]}, out {names[0]}",
        "data": "synthetic",
        "config": {"workload": wl.name, "path": "fp4", "dtypes": {"output": names[0], "epi": names[1]},
                   "pairs": pairs, "rows": wl.rows, "kv_replicas": args.replicas, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_launch": alg,
                     "kernel": "fp4_logits_kernel<%d>" % wl.next_n, "launch_us": ms_step * 1e3,
                     "mfma_frac": flops / (ms_step / 1e3) / 1e12 / FP4_PEAK_TFLOPS},
        "kernel_src_sha": kernel_hash(),
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="4", choices=["3", "4", "5", "prefill"])
    ap.add_argument("--path", default="fused", choices=["fused", "unfused", "logits", "fp4"])
    ap.add_argument("--dtypes", default="f32,f32,f32",
                    help="--path logits: output,epi,acc precisions, each f32 or f16; --path fp4: output,epi, "
                         "each f32, f16 or bf16 (default bf16,f32)")
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (for HBM counter calibration)")
    ap.add_argument("--main-leg", action="store_true",
                    help="also time the steps without the finish stage (the main pass alone; another launch "
                         "configuration of the same kernel, so it stays out of the default run)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    pm.lib()
    if args.workload == "prefill":
        return bench_prefill(args, dev)
    if args.path == "logits":
        return bench_logits(args, dev)
    if args.path == "fp4":
        return bench_fp4(args, dev)
    args.workload = int(args.workload)

    wl = W.make(args.workload)
    thr0 = load_thresholds(args.workload, wl)
    R, B = wl.rows, wl.batch
    ends = wl.row_ends()
    pairs = int(ends.sum())

    q = torch.from_numpy(wl.q).to(dev)
    w = torch.from_numpy(wl.weights).to(dev)
    bt = torch.from_numpy(wl.block_tables).to(dev)
    sl = torch.from_numpy(wl.seq_lens).to(dev)
    kv_host = torch.from_numpy(wl.kv_fused)
    kvs = [kv_host.to(dev).view(wl.num_blocks, wl.block_size, 1, 132) for _ in range(args.replicas)]
    del kv_host

    total = args.warmup + args.steps
    thr_all = torch.from_numpy(np.tile(thr0, (total, 1))).to(dev)
    cnt_all = torch.zeros(total, R, 2, dtype=torch.int32, device=dev)
    cand = torch.empty(R, wl.top_k + wl.capacity, 2, dtype=torch.int32, device=dev)
    arrivals = torch.zeros(B, dtype=torch.int32, device=dev)
    ranges = torch.empty(2, R, dtype=torch.int32, device=dev)
    topk = torch.empty(R, wl.top_k, dtype=torch.int32, device=dev)
    ws = pm.make_workspace("fused" if args.path == "fused" else "indexer_topk", B, wl.next_n, wl.max_seq_len, dev)
    logits = None
    if args.path == "unfused":
        logits = torch.empty(R, pm.padded_seq_len(wl.max_seq_len), dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream()

    def step(i, finish=True):
        kv = kvs[i % len(kvs)]
        fin = dict(arrivals=arrivals, ranges=ranges, topk_idx=topk, workspace=ws) if finish else {}
        if args.path == "fused":
            pm.fused_logits_select(q, kv, w, bt, sl, wl.max_seq_len, thr_all[i], cnt_all[i], cand, wl.capacity,
                                   wl.top_k, **fin)
        else:
            pm.mqa_logits(q, kv, w, bt, sl, wl.max_seq_len, out=logits)
            pm.indexer_topk(logits, sl, wl.next_n, wl.max_seq_len, thr_all[i], cnt_all[i], cand, wl.capacity,
                            wl.top_k, **fin)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    thr_pristine = torch.from_numpy(np.tile(thr0, (total, 1))).to(dev)

    def reset():
        cnt_all.zero_()
        thr_all.copy_(thr_pristine)

    def timed(finish):
        """Mean time per step over the timed steps: one event pair around all of
        them on the launch stream (events between steps would add their own
        gaps)."""
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for j in range(args.steps):
            step(args.warmup + j, finish)
        stop.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / args.steps

    ms_step = timed(True)
    assert int(arrivals.abs().sum()) == 0, "arrivals not left zeroed"
    repaired = int((thr_all[-1].cpu().numpy().view(np.int32) != thr0.view(np.int32)).sum())

    main_ms_mean = None
    if args.main_leg:
        # the same steps with the finish stage off: the main pass alone (fresh
        # counters, same KV replicas in the same order)
        reset()
        for i in range(args.warmup):
            step(i, finish=False)
        main_ms_mean = timed(False)

    # per-call spread, as context: an event pair around each call
    reset()
    for i in range(args.warmup):
        step(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for j in range(args.steps):
        ev[j][0].record(stream)
        step(args.warmup + j)
        ev[j][1].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])


    calibration_copy(args, dev)

    alg = algorithmic_bytes(wl, args.path)
    call_s = ms_step / 1e3
    achieved = alg / call_s / 1e9
    flops = 2.0 * 64 * 128 * pairs
    out = {
        "metric": METRIC,
        "value": pairs / (ms_step / 1e3),
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 -> f32",
        "data": "synthetic (seeded generators, workloads/)",
        "config": {"workload": wl.name, "path": args.path, "batch": B, "next_n": wl.next_n,
                   "block_size": wl.block_size, "top_k": wl.top_k, "capacity": wl.capacity,
                   "pairs": pairs, "rows": R, "kv_replicas": args.replicas, "parallelism": "single GPU"},
        "rows_per_s": R / (ms_step / 1e3),
        "repaired_rows": repaired,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_from_profiles(args.workload, args.path),
                     "algorithmic_bytes_per_launch": alg,
                     "kernel": ("fused_kernel<%d>" % wl.next_n) if args.path == "fused"
                               else "logits_kernel + select_kernel",
                     "launch_us": ms_step * 1e3,
                     "mfma_frac": flops / call_s / 1e12 / FP8_PEAK_TFLOPS},
        "call_us": {"mean": ms_step * 1e3,
                    "per_call_events": {"p10": float(np.percentile(launch_ms, 10)) * 1e3,
                                        "p50": float(np.percentile(launch_ms, 50)) * 1e3,
                                        "p90": float(np.percentile(launch_ms, 90)) * 1e3}},
        "kernel_src_sha": kernel_hash(),
    }
    if main_ms_mean is not None:
        out["main_pass_us"] = main_ms_mean * 1e3
        out["finish_stage_us"] = (ms_step - main_ms_mean) * 1e3
        out["main_pass_frac"] = alg / (main_ms_mean / 1e3) / 1e9 / HBM_PEAK_GBS
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, thr0, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
