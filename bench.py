#!/usr/bin/env python3
"""Throughput benchmark of the sparse MLA paged decode on one MI355X.

A step is one call of mla_sparse_decode (index resolution, gather, dequant,
QK^T, online softmax, PV, epilogue and -- when the plan splits the top-k
list -- the LSE combine) over one batch of synthetic input already resident
in HBM.  Steps rotate over several input sets (same cache pool, different Q
and index lists) so the bytes touched per rotation exceed the 256 MB
Infinity Cache.  The steps are captured once into a HIP graph (one pass over
the input sets) and replayed, as a serving loop would; timing uses HIP events
recorded on the launch stream around the replays.  The graph's output is
checked against an eager call.

Prints one JSON line on stdout.  Default workload: B=64, topk=512, 64 heads,
65,536-token sequences over a 16,384-page pool with 1% outlier channels.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16/fp16 MFMA peak
FLOP_PER_TOKEN = 2 * 64 * 512 + 2 * 64 * 448   # QK^T + PV per valid (query, token)
Q_BYTES = 64 * 512 * 2
OUT_BYTES = 64 * 448 * 2 + 64 * 4
TOKEN_BYTES = 584
APPEND_BYTES_PER_TOKEN = 512 * 2 + 4 + 4 + TOKEN_BYTES   # latent + seq id + position + record


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def workload_stats(w):
    """Valid entries, attended count and algorithmic bytes of one step."""
    lens = w.seq_lens.astype(np.int64)[:, None]
    idx = w.topk_idx.astype(np.int64)
    valid = (idx >= 0) & (idx < lens)
    n_valid = int(valid.sum())
    pages = set()
    for b in range(w.batch):
        lp = np.unique(idx[b][valid[b]] // 256)
        pages.update((b, int(p)) for p in lp)
    byts = (w.batch * (Q_BYTES + OUT_BYTES + 4) + TOKEN_BYTES * n_valid + 4 * w.batch * w.topk
            + 4 * len(pages))
    return dict(n_valid=n_valid, attended=64 * n_valid, bytes=byts, kv_bytes=TOKEN_BYTES * n_valid,
                flops=FLOP_PER_TOKEN * n_valid)


def cpu_baseline(w, seconds):
    """Time the fp64 CPU oracle on passes over the same workload (set 0), with
    every BLAS thread, then (for a fifth of the time) with one thread."""
    from oracle.mla_oracle import sparse_mla_decode as oracle_decode
    st = workload_stats(w)

    def rate(budget):
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle_decode(w.q_bits, w.kv_pages, w.page_table, w.topk_idx, w.seq_lens, w.softmax_scale)
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget or passes >= 1000:
                return st["attended"] * passes / el, passes, el

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                      or [1])
    except Exception:  # threadpoolctl missing: report the process's CPU affinity
        threadpool_limits = None
        threads = len(os.sched_getaffinity(0))
    value, passes, el = rate(seconds)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            one = rate(max(1.0, seconds / 5))[0]
    return {"value": value, "unit": "attended (query*head*token)/s",
            "cores": int(threads), "kind": "oracle",
            "value_1_thread": one,
            "sample": f"{passes} full pass(es) of the timed workload's first input set "
                      f"({w.batch} queries, {st['n_valid']} valid entries) in {el:.1f} s; "
                      f"numpy float64 with {threads} BLAS thread(s), then 1 thread"}


def copy_bandwidth(dev, mib=1024, reps=5):
    """Device-to-device copy rate (read + write bytes per second): the
    practical HBM ceiling on this GPU, reported beside the 8 TB/s peak."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    return 2 * n / sec / 1e9


def cold_calls(step, n_sets, stream, dev, calls=50, flush_mb=512):
    """Per-call duration (HIP events on the launch stream) of single eager
    calls, each after a flush write that evicts L2 and the Infinity Cache."""
    import torch
    flush = torch.empty(flush_mb << 18, dtype=torch.int32, device=dev)
    times = []
    with torch.cuda.stream(stream):
        for i in range(calls):
            flush.fill_(i)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(i % n_sets, stream)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
    del flush
    t = np.array(times)
    return {"median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
            "p90_us": float(np.percentile(t, 90)), "calls": calls, "flush_mb": flush_mb,
            "launch": "eager, one call per flush"}


def bench_append(dev, kv, pt, seq_len, steps, stream, traffic_json=None):
    """Time mla_kv_append writing the last `per_seq` positions of every
    sequence (a prefill-sized append of 4,096 tokens per sequence) into the
    resident pool; HIP events on the launch stream around `steps` calls."""
    import torch
    import sparse_mla_decode_page_amd as mlasd
    B = pt.shape[0]
    per_seq = 4096
    n = B * per_seq
    g = torch.Generator(device="cpu").manual_seed(99)
    lat = (torch.randn((n, 512), generator=g) * 2.0).to(torch.bfloat16).to(dev)
    seq = torch.arange(B, dtype=torch.int32).repeat_interleave(per_seq).to(dev)
    pos = (torch.arange(per_seq, dtype=torch.int32) + (seq_len - per_seq)).repeat(B).to(dev)
    with torch.cuda.stream(stream):
        for _ in range(3):
            mlasd.mla_kv_append(lat, seq, pos, pt, kv, stream=stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            mlasd.mla_kv_append(lat, seq, pos, pt, kv, stream=stream)
        e1.record(stream)
    stream.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    byts = n * APPEND_BYTES_PER_TOKEN
    gbs = byts / (us * 1e-6) / 1e9
    traffic = None
    if traffic_json and os.path.exists(traffic_json):
        try:
            traffic = json.load(open(traffic_json)).get(f"append_{B}x{per_seq}", {}).get("bytes_per_launch")
        except Exception:
            traffic = None
    return {"tokens_per_launch": n, "us_per_launch": us, "tokens_per_s": n / (us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                         "algorithmic_bytes_per_launch": byts},
            "workload": f"{B} sequences x {per_seq} new tokens into the resident pool"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # The GPU needs some 20-30 ms of continuous work before its clocks settle:
    # with 20 warm-up steps the timed replays of c3 run 1 us (c4 2.3 us) slower
    # than in the steady state a serving loop runs in.  1,000 steps cost about
    # 50 ms.  Single cold calls are timed separately (config.cold_call).
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", type=int, default=3, help="workload index 0..4")
    ap.add_argument("--nsplit", type=int, default=0, help="force top-k slices per query (0 = plan)")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = enough to exceed MALL)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="per-launch HBM bytes measured with rocprofv3 counters")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager calls only (for counter-collection runs)")
    ap.add_argument("--op", choices=["decode", "append"], default="decode",
                    help="append: time only the cache-append kernel")
    ap.add_argument("--no-append", action="store_true", help="skip the cache-append measurement")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the flushed single-call timing and the copy ceiling (profiling runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 8 plain device-to-device copies of MIB MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_mla_decode_page_amd as mlasd
    from gen.synth import CONFIG_NAMES, make_config, rotation_sets

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy > 0:
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 8}), flush=True)
        return
    mlasd.load_library()

    t0 = time.perf_counter()
    w = make_config(args.config)
    st = workload_stats(w)
    n_sets = args.sets or int(min(64, max(1, math.ceil(640e6 / st["bytes"]))))
    sets = rotation_sets(w, n_sets, seed=777 + args.config)
    log(f"workload {CONFIG_NAMES[args.config]}: {n_sets} input sets built in {time.perf_counter() - t0:.1f} s")

    kv = torch.from_numpy(w.kv_pages).to(dev)
    pt = torch.from_numpy(w.page_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    side = torch.cuda.Stream(dev)
    if args.op == "append":
        if int(w.seq_lens.min()) < 4096:
            print("--op append needs every sequence >= 4096 tokens (config 1-3)", file=sys.stderr)
            sys.exit(2)
        res = bench_append(dev, kv, pt, int(w.seq_lens.min()), args.steps, side, args.traffic_json)
        res["metric"] = "cache append: tokens/s"
        print(json.dumps(res), flush=True)
        return
    dsets = []
    for s in sets:
        dsets.append(dict(
            q=torch.from_numpy(s.q_bits.view(np.int16)).view(torch.bfloat16).to(dev),
            idx=torch.from_numpy(s.topk_idx).to(dev),
            out=torch.empty((w.batch, 64, 448), dtype=torch.bfloat16, device=dev),
            lse=torch.empty((w.batch, 64), dtype=torch.float32, device=dev)))
    stats = [workload_stats(s) for s in sets]
    nsplit, split_len, head_groups = mlasd.plan(w.batch, w.topk, args.nsplit)
    nsplit_arg = args.nsplit if args.nsplit > 0 else None

    def step(i, stream):
        d = dsets[i % n_sets]
        mlasd.mla_sparse_decode(d["q"], kv, pt, d["idx"], lens, w.softmax_scale, out=d["out"],
                                lse=d["lse"], stream=stream, nsplit=nsplit_arg)

    # eager warm-up on the capture stream (sizes the library's split scratch)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for i in range(max(args.warmup, n_sets)):
            step(i, side)
    side.synchronize()
    ref0 = (dsets[0]["out"].clone(), dsets[0]["lse"].clone())
    if not torch.isfinite(ref0[1]).any():
        raise RuntimeError("non-finite output in warm-up")

    # eager timing (includes host launch overhead per call)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    n_eager = min(args.steps, 4 * n_sets)
    with torch.cuda.stream(side):
        ev0.record(side)
        for i in range(n_eager):
            step(i, side)
        ev1.record(side)
    side.synchronize()
    eager_ms = ev0.elapsed_time(ev1) / n_eager

    if args.no_graph:
        res = {"metric": "eager only", "ms_per_step": eager_ms, "steps": n_eager,
               "config": {"workload": CONFIG_NAMES[args.config], "nsplit": nsplit}}
        print(json.dumps(res), flush=True)
        return

    # one graph = one pass over all input sets; replayed until >= steps
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(n_sets):
            step(i, side)
    reps = max(1, math.ceil(args.steps / n_sets))
    with torch.cuda.stream(side):
        for _ in range(max(1, args.warmup // n_sets)):
            graph.replay()
        side.synchronize()
        ev0.record(side)
        for _ in range(reps):
            graph.replay()
        ev1.record(side)
    side.synchronize()
    steps_done = reps * n_sets
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps_done
    if not (torch.equal(dsets[0]["out"], ref0[0]) and torch.equal(dsets[0]["lse"], ref0[1])):
        raise RuntimeError("graph replay output differs from the eager call")
    args.steps = steps_done

    cold = None if args.no_cold else cold_calls(step, n_sets, side, dev)
    copy_gbs = None if args.no_cold else copy_bandwidth(dev)

    order = [i % n_sets for i in range(args.steps)]
    attended = sum(stats[k]["attended"] for k in order) / args.steps
    byts = sum(stats[k]["bytes"] for k in order) / args.steps
    kvb = sum(stats[k]["kv_bytes"] for k in order) / args.steps
    flops = sum(stats[k]["flops"] for k in order) / args.steps
    sec = ms_step / 1e3
    achieved = byts / sec / 1e9

    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            key = f"config{args.config}_nsplit{nsplit}_hg{head_groups}"
            if key in tj:
                traffic = tj[key]["bytes_per_launch"]
        except Exception:
            traffic = None

    res = {
        "metric": "sparse-MLA decode: attended (query*head*token)/s + achieved HBM GB/s vs peak",
        "value": attended / sec,
        "unit": "attended (query*head*token)/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": CONFIG_NAMES[args.config],
            "batch": w.batch, "heads": 64, "topk": w.topk,
            "valid_entries_per_step": stats[0]["n_valid"],
            "nsplit": nsplit, "split_len": split_len, "head_groups": head_groups,
            "input_sets": n_sets,
            "launch": "HIP graph replay (one graph = one pass over the input sets)",
            "eager_ms_per_step": eager_ms,
            "cold_call": cold,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "copy_gbs": copy_gbs,
            "frac_of_copy": achieved / copy_gbs if copy_gbs else None,
            "algorithmic_bytes_per_step": byts,
            "kv_gbs": kvb / sec / 1e9,
            "mfma_tflops": flops / sec / 1e12,
            "mfma_frac": flops / sec / 1e12 / BF16_PEAK_TFLOPS,
            "timed": "decode kernel" + (" + LSE combine kernel" if nsplit > 1 else ""),
        },
    }
    if not args.no_append and int(w.seq_lens.min()) >= 4096:
        # runs after the decode timing: it overwrites the pool's tail records
        res["kv_append"] = bench_append(dev, kv, pt, int(w.seq_lens.min()), 50, side, args.traffic_json)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
