#!/usr/bin/env python3
"""Throughput benchmark of the sparse MLA paged decode on one MI355X.

A step is one call of mla_sparse_decode (index resolution, gather, dequant,
QK^T, online softmax, PV, epilogue and -- when the plan splits the top-k
list -- the LSE combine) over one batch of synthetic input already resident
in HBM.  Steps rotate over several input sets (same cache pool, different Q
and index lists) so the bytes touched per rotation exceed the 256 MB
Infinity Cache.  Exactly --steps steps are captured into one HIP graph and
replayed, as a serving loop would; timing uses HIP events recorded on the
launch stream around the replay.  The graph's output is checked against an
eager call.

Every standard workload (c0..c4) is timed in the same run; the headline line
is the largest one, c4 (B=256, top-k 512, log-uniform lengths up to 131,072
tokens), and the others appear under "per_config".  Prints one JSON line on
stdout; progress goes to stderr.

Other modes: --config N times one workload only; --batch/--topk/--seq-len
time a custom uniform-length workload; --summarize-counters DIR turns
rocprofv3 FETCH_SIZE / WRITE_SIZE runs into profiles/traffic.json entries.
"""
import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E peak
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 / fp16 MFMA peak
FLOP_PER_TOKEN = 2 * 64 * 512 + 2 * 64 * 448   # QK^T + PV per valid (query, token)
Q_BYTES = 64 * 512 * 2
OUT_BYTES = 64 * 448 * 2 + 64 * 4
TOKEN_BYTES = 584
APPEND_BYTES_PER_TOKEN = 512 * 2 + 4 + 4 + TOKEN_BYTES   # latent + seq id + position + record
WARMUP_FLOOR_S = 0.05           # untimed GPU work before timing, whatever --warmup says
HEADLINE = 4
METRIC = "sparse-MLA decode: attended (query·head·token)/s + achieved HBM GB/s vs peak"
KERNEL_SOURCES = ["sparse_mla_decode_page_amd/csrc/mlasd_decode.hip", "sparse_mla_decode_page_amd/csrc/mlasd_combine.hip"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_hash():
    """Hash of the decode kernels' source: counter figures are only reported
    while the kernels they were taken on are unchanged."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
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


def read_traffic(path, key):
    """Counter bytes per step for `key`, or None when absent or taken on
    other kernel sources."""
    if not os.path.exists(path):
        return None
    try:
        e = json.load(open(path)).get(key)
    except Exception:
        return None
    if not e or e.get("kernel_hash") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


def bench_append(dev, kv, pt, seq_len, steps, stream):
    """Time mla_kv_append writing the last 4,096 positions of every sequence
    (a prefill-sized append) into the resident pool; HIP events on the launch
    stream around `steps` calls."""
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
    return {"tokens_per_launch": n, "us_per_launch": us, "tokens_per_s": n / (us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": byts},
            "workload": f"{B} sequences x {per_seq} new tokens into the resident pool"}


def bench_topk(dev, stream, steps, batch=64, max_len=65536, k=512, parts=None):
    """Time mla_topk_select on `batch` rows of `max_len` fp32 scores (all
    positions candidates): HIP events on the launch stream around `steps`
    calls captured in one graph.  The stream's scratch is reserved for the
    library's plan (or the forced `parts`); the one-workgroup-per-row plan
    is timed beside it."""
    import torch
    import sparse_mla_decode_page_amd as mlasd
    from gen.synth import indexer_scores
    sc = torch.from_numpy(indexer_scores(31, batch, max_len)).to(dev)
    lens = torch.full((batch,), max_len, dtype=torch.int32, device=dev)
    idx = torch.empty((batch, k), dtype=torch.int32, device=dev)
    n_parts, nbytes = mlasd.topk_plan(batch, max_len, parts or 0)
    mlasd.reserve(nbytes, stream=stream)

    def timed(pa):
        with torch.cuda.stream(stream):
            for _ in range(3):
                mlasd.mla_topk_select(sc, lens, k, out=idx, stream=stream, parts=pa)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(steps):
                mlasd.mla_topk_select(sc, lens, k, out=idx, stream=stream, parts=pa)
        with torch.cuda.stream(stream):
            g.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
        stream.synchronize()
        del g
        return e0.elapsed_time(e1) * 1e3 / steps

    us = timed(parts)
    us_one = timed(1) if n_parts > 1 else us
    byts = batch * max_len * 4 + batch * k * 4 + batch * 4
    gbs = byts / (us * 1e-6) / 1e9
    return {"workload": f"{batch} queries x {max_len} fp32 scores, k={k}", "us_per_launch": us,
            "parts_per_row": n_parts, "us_per_launch_one_workgroup_per_row": us_one,
            "rows_per_s": batch / (us * 1e-6),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": byts},
            "launch": f"HIP graph replay of {steps} calls"}


def bench_chain(dev, wb, steps):
    """Time top-k selection chained before the decode in one captured graph
    on workload c3's cache: 64 rows of 65,536 fp32 scores -> topk_idx ->
    decode, `steps` times, HIP events on the launch stream."""
    import torch
    import sparse_mla_decode_page_amd as mlasd
    from gen.synth import indexer_scores
    w = wb.w
    sc = torch.from_numpy(indexer_scores(33, w.batch, int(w.seq_lens.max()))).to(dev)
    idx = torch.empty((w.batch, w.topk), dtype=torch.int32, device=dev)
    n_parts, nbytes = mlasd.topk_plan(w.batch, sc.shape[1])
    mlasd.reserve(nbytes, stream=wb.stream)   # the decode's split scratch, grown if the selection needs more
    q = wb.dsets[0]["q"]
    out = torch.empty((w.batch, 64, 448), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.batch, 64), dtype=torch.float32, device=dev)
    stream = wb.stream

    def step():
        mlasd.mla_topk_select(sc, wb.lens, w.topk, out=idx, stream=stream)
        mlasd.mla_sparse_decode(q, wb.kv, wb.pt, idx, wb.lens, w.softmax_scale, out=out, lse=lse, stream=stream)

    with torch.cuda.stream(stream):
        for _ in range(3):
            step()
    stream.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(steps):
            step()
    with torch.cuda.stream(stream):
        g.replay()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
    stream.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del g
    return {"workload": f"top-k of {w.batch} x {int(w.seq_lens.max())} fp32 scores (k={w.topk}), then the "
                        f"decode of workload c3 on the selected entries",
            "us_per_step": us, "topk_parts_per_row": n_parts,
            "launch": f"HIP graph replay of {steps} chained steps"}


class Workbench:
    """One workload on the device: rotating input sets, the step function,
    and the graph of exactly `steps` steps."""

    def __init__(self, w, dev, nsplit, name, head_groups=0):
        import torch
        import sparse_mla_decode_page_amd as mlasd
        from gen.synth import rotation_sets
        self.mlasd, self.torch = mlasd, torch
        self.w, self.dev, self.name = w, dev, name
        st = workload_stats(w)
        self.n_sets = int(min(64, max(1, math.ceil(640e6 / st["bytes"]))))
        t0 = time.perf_counter()
        self.sets = rotation_sets(w, self.n_sets, seed=777 + w.batch)
        self.stats = [workload_stats(s) for s in self.sets]
        self.kv = torch.from_numpy(w.kv_pages).to(dev)
        self.pt = torch.from_numpy(w.page_table).to(dev)
        self.lens = torch.from_numpy(w.seq_lens).to(dev)
        self.dsets = []
        for s in self.sets:
            self.dsets.append(dict(
                q=torch.from_numpy(s.q_bits.view(np.int16)).view(torch.bfloat16).to(dev),
                idx=torch.from_numpy(s.topk_idx).to(dev),
                out=torch.empty((w.batch, 64, 448), dtype=torch.bfloat16, device=dev),
                lse=torch.empty((w.batch, 64), dtype=torch.float32, device=dev)))
        self.nsplit_arg = nsplit if nsplit > 0 else None
        self.hg_arg = head_groups if head_groups > 0 else None
        ns, sl, hg = mlasd.plan(w.batch, w.topk, nsplit)
        if head_groups > 0:   # the plan with the head groups forced
            sl = max(32, -(-w.topk // max(1, nsplit or ns)) // 32 * 32 if nsplit else sl)
            hg = head_groups
        self.plan = (ns, sl, hg)
        self.stream = torch.cuda.Stream(dev)
        mlasd.reserve(mlasd.workspace_size(w.batch, w.topk, nsplit, head_groups), stream=self.stream)
        log(f"{name}: {self.n_sets} input sets ready in {time.perf_counter() - t0:.1f} s, "
            f"plan (nsplit, split_len, head_groups) = {self.plan}")

    def step(self, i, stream):
        d = self.dsets[i % self.n_sets]
        self.mlasd.mla_sparse_decode(d["q"], self.kv, self.pt, d["idx"], self.lens, self.w.softmax_scale,
                                     out=d["out"], lse=d["lse"], stream=stream, nsplit=self.nsplit_arg,
                                     head_groups=self.hg_arg)

    def run(self, steps, warmup, graph=True):
        torch = self.torch
        side = self.stream
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            for i in range(self.n_sets):
                self.step(i, side)
        side.synchronize()
        ref0 = (self.dsets[0]["out"].clone(), self.dsets[0]["lse"].clone())
        if not torch.isfinite(ref0[1]).any():
            raise RuntimeError(f"{self.name}: non-finite output")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        if not graph:
            with torch.cuda.stream(side):
                for i in range(warmup):
                    self.step(i, side)
                side.synchronize()
                ev0.record(side)
                for i in range(steps):
                    self.step(i, side)
                ev1.record(side)
            side.synchronize()
            return dict(ms_step=ev0.elapsed_time(ev1) / steps, warmup_steps=warmup,
                        order=[i % self.n_sets for i in range(steps)])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for i in range(steps):
                self.step(i, side)
        # untimed warm-up, enqueued back to back so the clocks settle: at
        # least --warmup steps and WARMUP_FLOOR_S of GPU work
        with torch.cuda.stream(side):
            ev0.record(side)
            g.replay()
            ev1.record(side)
            ev1.synchronize()
            t_one = ev0.elapsed_time(ev1) / 1e3
            reps = max(math.ceil(max(warmup - steps, 0) / steps), math.ceil((WARMUP_FLOOR_S - t_one) / t_one), 0)
            ev0.record(side)
            for _ in range(reps):
                g.replay()
            ev1.record(side)
            ev1.synchronize()
            warm = steps * (reps + 1)
            t_warm = t_one + ev0.elapsed_time(ev1) / 1e3
            torch.cuda.synchronize()
            ev0.record(side)
            g.replay()
            ev1.record(side)
        side.synchronize()
        torch.cuda.synchronize()
        ms_step = ev0.elapsed_time(ev1) / steps
        if not (torch.equal(self.dsets[0]["out"], ref0[0]) and torch.equal(self.dsets[0]["lse"], ref0[1])):
            raise RuntimeError(f"{self.name}: graph replay output differs from the eager call")
        del g
        return dict(ms_step=ms_step, warmup_steps=warm, warmup_s=t_warm,
                    order=[i % self.n_sets for i in range(steps)])

    def summary(self, r, config_key):
        order = r["order"]
        n = len(order)
        attended = sum(self.stats[k]["attended"] for k in order) / n
        byts = sum(self.stats[k]["bytes"] for k in order) / n
        kvb = sum(self.stats[k]["kv_bytes"] for k in order) / n
        flops = sum(self.stats[k]["flops"] for k in order) / n
        sec = r["ms_step"] / 1e3
        achieved = byts / sec / 1e9
        ns, sl, hg = self.plan
        traffic = read_traffic(os.path.join(ROOT, "profiles", "traffic.json"), f"{config_key}_nsplit{ns}_hg{hg}")
        return {
            "us_per_step": r["ms_step"] * 1e3,
            "attended_per_s": attended / sec,
            "algorithmic_bytes_per_step": byts,
            "achieved_gbs": achieved,
            "frac": achieved / HBM_PEAK_GBS,
            "kv_gbs": kvb / sec / 1e9,
            "mfma_tflops": flops / sec / 1e12,
            "mfma_frac": flops / sec / 1e12 / MFMA_PEAK_TFLOPS,
            "traffic_bytes_per_step": traffic,
            "valid_entries_per_step": self.stats[0]["n_valid"],
            "plan": {"nsplit": ns, "split_len": sl, "head_groups": hg},
            "input_sets": self.n_sets,
            "warmup_steps_run": r["warmup_steps"],
        }


def summarize_counters(d, config_key, out_json):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (counter_collection
    CSVs under d/fetch, d/write, and the copy calibration under d/cal_fetch,
    d/cal_write) into per-step HBM bytes for `config_key`."""
    def per_kernel(sub, counter):
        files = glob.glob(os.path.join(d, sub, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {os.path.join(d, sub)}")
        acc = {}
        for fn in files:
            for row in csv.DictReader(open(fn)):
                if row.get("Counter_Name") != counter:
                    continue
                k = row["Kernel_Name"]
                acc.setdefault(k, []).append(float(row["Counter_Value"]))
        return {k: (float(np.mean(v)), len(v)) for k, v in acc.items()}

    cf = per_kernel("cal_fetch", "FETCH_SIZE")
    cw = per_kernel("cal_write", "WRITE_SIZE")
    copy_kib = json.load(open(os.path.join(d, "cal_bytes.json")))["calibrate_copy_bytes"] / 1024.0
    fk = max(cf.values(), key=lambda v: v[0])[0]
    wk = max(cw.values(), key=lambda v: v[0])[0]
    f_factor, w_factor = copy_kib / fk, copy_kib / wk
    fetch = per_kernel("fetch", "FETCH_SIZE")
    write = per_kernel("write", "WRITE_SIZE")
    per = {}
    lines = []
    for k in sorted(set(fetch) | set(write)):
        if "mlasd" not in k:
            continue
        fr = fetch.get(k, (0.0, 0))
        wr = write.get(k, (0.0, 0))
        rd, wt = fr[0] * 1024 * f_factor, wr[0] * 1024 * w_factor
        per[k] = rd + wt
        lines.append(f"{k:42s} {fr[1]:6d} {fr[0]:14.1f} {wr[0]:14.1f} {rd / 1e6:9.2f} {wt / 1e6:9.2f}")
    total = sum(per.values())
    tj = json.load(open(out_json)) if os.path.exists(out_json) else {}
    tj[config_key] = {"bytes_per_launch": total, "per_kernel_bytes": per, "fetch_factor": f_factor,
                      "write_factor": w_factor, "kernel_hash": kernel_hash()}
    with open(out_json, "w") as f:
        json.dump(tj, f, indent=1)
    print(f"calibration: FETCH_SIZE factor {f_factor:.3f}, WRITE_SIZE factor {w_factor:.3f}")
    print(f"{'kernel':42s} {'disp':>6s} {'FETCH KiB':>14s} {'WRITE KiB':>14s} {'read MB':>9s} {'write MB':>9s}")
    print("\n".join(lines))
    print(f"HBM bytes per step (all kernels of one call, calibrated): {total / 1e6:.2f} MB")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps before timing (at least 50 ms of GPU work is run regardless)")
    ap.add_argument("--config", type=int, default=-1, help="time workload 0..4 only (-1: all, headline c4)")
    ap.add_argument("--batch", type=int, default=0, help="custom workload: queries")
    ap.add_argument("--topk", type=int, default=512, help="custom workload: top-k width")
    ap.add_argument("--seq-len", type=int, default=65536, help="custom workload: tokens per sequence")
    ap.add_argument("--nsplit", type=int, default=0,
                    help="force top-k slices per query (0 = plan); with --op topk, parts per row")
    ap.add_argument("--head-groups", type=int, default=0, help="force workgroups per slice's heads (0 = plan)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls (counter-collection runs)")
    ap.add_argument("--no-append", action="store_true", help="skip the cache-append measurement")
    ap.add_argument("--op", choices=["decode", "append", "topk"], default="decode",
                    help="append: time only the cache-append kernel (on workload c3's pool); "
                         "topk: time only the top-k selection (--batch rows, default 64, of "
                         "--seq-len scores, default 65,536; k = --topk)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the flushed single-call timing and the copy ceiling (profiling runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 8 plain device-to-device copies of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-counters", default="", metavar="DIR",
                    help="turn rocprofv3 counter runs under DIR into profiles/traffic.json (needs --key)")
    ap.add_argument("--key", default="", help="traffic.json key for --summarize-counters")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.key, os.path.join(ROOT, "profiles", "traffic.json"))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this library runs on a single "
              "GPU and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_mla_decode_page_amd as mlasd
    from gen.synth import CONFIG_NAMES, build_workload, make_config

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

    if args.op == "append":
        w = make_config(3)
        kv = torch.from_numpy(w.kv_pages).to(dev)
        pt = torch.from_numpy(w.page_table).to(dev)
        res = bench_append(dev, kv, pt, int(w.seq_lens.min()), args.steps, torch.cuda.Stream(dev))
        res["metric"] = "cache append: tokens/s"
        print(json.dumps(res), flush=True)
        return
    if args.op == "topk":
        res = bench_topk(dev, torch.cuda.Stream(dev), args.steps, batch=args.batch or 64,
                         max_len=args.seq_len, k=args.topk, parts=args.nsplit or None)
        res["metric"] = "top-k selection: query rows/s"
        print(json.dumps(res), flush=True)
        return

    if args.batch > 0:
        lens = np.full(args.batch, args.seq_len)
        name = f"custom: B={args.batch} topk={args.topk} seq_len={args.seq_len}"
        todo = [("custom", name, lambda: build_workload(4242, lens, args.topk, name=name,
                                                        num_pages=int(lens.sum() // 256 + args.batch + 8)))]
        head_key = "custom"
    else:
        idx = [args.config] if args.config >= 0 else [0, 1, 2, 3, 4]
        todo = [(f"config{i}", CONFIG_NAMES[i], (lambda i=i: make_config(i))) for i in idx]
        head_key = f"config{args.config if args.config >= 0 else HEADLINE}"

    per = {}
    head = None
    for key, name, build in todo:
        t0 = time.perf_counter()
        w = build()
        log(f"{key}: workload built in {time.perf_counter() - t0:.1f} s")
        wb = Workbench(w, dev, args.nsplit, key, args.head_groups)
        r = wb.run(args.steps, args.warmup, graph=not args.no_graph)
        s = wb.summary(r, key)
        s["workload"] = name
        per[key] = s
        log(f"{key}: {s['us_per_step']:.2f} us/step, {s['attended_per_s']:.3e} attended/s, "
            f"{s['achieved_gbs']:.0f} GB/s = {s['frac']:.3f} of peak")
        if key == head_key:
            head = dict(wb=wb, r=r, s=s, w=w)
            if not args.no_cold:
                s["cold_call"] = cold_calls(wb.step, wb.n_sets, wb.stream, dev)
        if key == "config3" and not args.no_append:
            per["kv_append"] = bench_append(dev, wb.kv, wb.pt, int(w.seq_lens.min()), 50, wb.stream)
            per["topk_select"] = bench_topk(dev, wb.stream, 50)
            per["topk_then_decode"] = bench_chain(dev, wb, 50)
        if key != head_key:
            del wb
            torch.cuda.empty_cache()

    s, w = head["s"], head["w"]
    copy_gbs = None if args.no_cold else copy_bandwidth(dev)
    res = {
        "metric": METRIC,
        "value": s["attended_per_s"],
        "unit": "attended (query*head*token)/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": s["warmup_steps_run"],
        "ms_per_step": s["us_per_step"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 + bf16 MFMA operands, fp32 accumulate (fp8 e4m3 + UE8M0 cache)",
        "data": "synthetic (seeded; stands in for the pages' DeepSeek-V4-Flash caches)",
        "config": {
            "workload": s["workload"],
            "batch": w.batch, "heads": 64, "topk": w.topk,
            "valid_entries_per_step": s["valid_entries_per_step"],
            "plan": s["plan"],
            "input_sets": s["input_sets"],
            "launch": "HIP graph replay of exactly `steps` steps over rotating input sets",
            "warmup_requested": args.warmup,
            "cold_call": s.get("cold_call"),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": s["achieved_gbs"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": s["frac"],
            "traffic": s["traffic_bytes_per_step"],
            "copy_gbs": copy_gbs,
            "frac_of_copy": s["achieved_gbs"] / copy_gbs if copy_gbs else None,
            "algorithmic_bytes_per_step": s["algorithmic_bytes_per_step"],
            "kv_gbs": s["kv_gbs"],
            "mfma_tflops": s["mfma_tflops"],
            "mfma_frac": s["mfma_frac"],
            "timed": "decode kernel" + (" + LSE combine kernel" if s["plan"]["nsplit"] > 1 else "")
                     + " (HIP events on the launch stream around the graph replay)",
        },
        "per_config": per,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
