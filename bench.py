#!/usr/bin/env python3
"""Throughput of paged MLA decode on one MI355X: TFLOPS and HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2]

One step is one decode call over the whole batch of the workload: the split-KV
kernel then the LSE combine, on inputs already resident in HBM.  The tile
scheduler runs once per decode step and its metadata is reused by every layer
(the pages' call pattern), so it is timed separately on the host
(``metadata_us``); ``with_metadata`` reports the rate when every step also
rebuilds and uploads the metadata.  The cache is rotated over enough copies
that the bytes read between two uses of one copy exceed 1 GiB, four times the
256 MB Infinity Cache: a step's rows are never served from what earlier steps
left there.

Algorithmic work (what the method must do, not padded work):
  FLOP  = sum over (query row, visible key) of 2 * (d_qk + d_v)
  bytes = every visible cache row once per request (d_qk * 2 B, or 656 B for
          an FP8-with-scale row; the value is inside it) + q, O (bf16) and LSE
          (fp32) of the computed heads + block-table entries (or indices) read
          + sequence lengths.
The split workspace traffic is overhead and is not counted.

Prints one JSON line.  ``ms_per_step`` is the whole decode (split-KV then
combine) over K steps timed back to back between two HIP events; the combine
is timed alone the same way and the split-KV time is the difference.
``step_ms`` gives the min and median of at least 100 single steps, each its
own graph replay between two events (rotating over the cache copies).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged MLA decode TFLOPS + HBM GB/s (h_q=128, d_qk=576, d_v=512) on 1 GPU"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "mla_paged_kv_amd", "csrc")


def kernel_sources():
    """Every source of the library: the kernels, the launchers, the host and
    device schedulers (which set the split partial traffic) and the C ABI."""
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".h", ".hip", ".cpp")))


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in kernel_sources():
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def algorithmic_work(case, batches=None) -> dict:
    """Integer accounting of the work the method must do (see module
    docstring), over every request or over the requests in ``batches``."""
    s_q, d_qk, d_v = case["s_q"], case["d_qk"], case["d_v"]
    bsel = list(range(case["q"].shape[0])) if batches is None else list(batches)
    B = len(bsel)
    row_bytes = 656 if case.get("kv_fp8") else d_qk * 2
    if case["sparse"]:
        heads = case["active_h_q"]
        idx = case["indices"][bsel]
        nrows = case["kvcache"].shape[0] * case["kvcache"].shape[1]
        valid = ((idx >= 0) & (idx < nrows)).sum().item()
        flop = valid * heads * 2 * (d_qk + d_v)
        kv_bytes = valid * row_bytes
        meta_bytes = idx.numel() * 4
        keys = valid
    else:
        heads = case["h_q"]
        sl = [int(case["cache_seqlens"][b]) for b in bsel]
        keys = 0
        for L in sl:
            for i in range(s_q):
                keys += max(0, min(L, L - s_q + i + 1)) if case["causal"] else L
        flop = keys * heads * 2 * (d_qk + d_v)
        kv_bytes = sum(sl) * row_bytes
        meta_bytes = sum((L + 63) // 64 for L in sl) * 4 + B * 4
    q_bytes = B * s_q * heads * d_qk * 2
    o_bytes = B * s_q * heads * (d_v * 2 + 4)
    return dict(flop=flop, bytes=kv_bytes + q_bytes + o_bytes + meta_bytes, kv_bytes=kv_bytes,
                keys=keys)


def _oracle_rate(case, min_seconds: float, max_passes: int, batches=None):
    """(TFLOPS, passes, seconds) of the oracle over whole passes of the
    workload, or of the requests in ``batches`` only."""
    import oracle
    work = algorithmic_work(case, batches)
    passes, t0 = 0, time.perf_counter()
    while True:
        if case["sparse"]:
            oracle.ref_decode_sparse(case["q"], case["kvcache"], case["indices"], case["d_v"],
                                     case["softmax_scale"], heads=range(case["active_h_q"]),
                                     batches=batches)
        else:
            oracle.ref_decode_paged(case["q"], case["kvcache"], case["block_table"],
                                    case["cache_seqlens"], case["d_v"], case["causal"],
                                    case["softmax_scale"], batches=batches)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    return work["flop"] * passes / dt / 1e12, passes, dt


def cpu_baseline(case, min_seconds: float, max_passes: int = 64) -> dict:
    """The FP64 oracle as it stands, on the host cores: whole passes of the
    workload until ``min_seconds`` have elapsed with every BLAS thread, then a
    bounded sample (the first requests, about a quarter of that time) with one
    thread."""
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        cores = max([p["num_threads"] for p in blas] or [os.cpu_count() or 1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = os.cpu_count() or 1
    rate, passes, dt = _oracle_rate(case, min_seconds, max_passes)
    out = {"value": round(rate, 6), "unit": "TFLOPS", "cores": int(cores), "kind": "oracle",
           "sample": f"whole workload x {passes} pass(es), {dt:.1f} s, float64 numpy "
                     f"(BLAS threads {cores}, host cpus {os.cpu_count()})"}
    if threadpool_limits is not None:
        # one thread: requests 0, 1, ... (cycling) one at a time until a
        # quarter of the time budget is spent (at least one request)
        B = int(case["q"].shape[0])
        flop, n, t1 = 0, 0, time.perf_counter()
        with threadpool_limits(limits=1, user_api="blas"):
            while True:
                _oracle_rate(case, 0.0, 1, batches=[n % B])
                flop += algorithmic_work(case, [n % B])["flop"]
                n += 1
                if time.perf_counter() - t1 >= min_seconds / 4 or n >= 64 * B:
                    break
        d1 = time.perf_counter() - t1
        out["single_thread"] = {"value": round(flop / d1 / 1e12, 6), "unit": "TFLOPS", "cores": 1,
                                "kind": "oracle",
                                "sample": f"{n} requests (cycling over the {B}), {d1:.1f} s, float64 "
                                          f"numpy, BLAS threads 1"}
    return out


COPY_PROBE_BYTES = 256 << 20  # read once and written once by the copy probe


def copy_probe(torch, dev, reps: int = 3):
    """A plain copy of known size (COPY_PROBE_BYTES read, the same written),
    run only under counter collection: its FETCH_SIZE / WRITE_SIZE readings
    scale the counters of the decode kernels to bytes."""
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


ROTATE_BYTES = 1 << 30  # bytes read between two uses of one cache copy
MAX_COPIES = 16


def rotation_copies(step_bytes: int) -> int:
    """Cache copies so that the other copies' steps read >= ROTATE_BYTES
    between two uses of one copy."""
    return max(2, min(MAX_COPIES, 1 + math.ceil(ROTATE_BYTES / max(step_bytes, 1))))


def bench_workload(k, steps: int, warmup: int, replays: int = 100,
                   probe: bool = False) -> dict:
    import torch

    import mla_paged_kv_amd as mla
    from synth.configs import make_config

    case = make_config(k)
    work = algorithmic_work(case)
    dev = torch.device("cuda", 0)
    q = case["q"].to(dev)
    kv0 = case["kvcache"].to(dev)
    copies = rotation_copies(work["bytes"])
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    bt = case["block_table"].to(dev)
    sl = case["cache_seqlens"].to(dev)
    idx = case["indices"].to(dev) if case["sparse"] else None

    def get_meta():
        if case["sparse"]:
            return mla.mla_get_metadata(case["cache_seqlens"], case["s_q"], case["h_q"],
                                        topk=case["topk"], active_h_q=case["active_h_q"], device=dev)
        return mla.mla_get_metadata(case["cache_seqlens"], case["s_q"], case["h_q"], device=dev)

    t0 = time.perf_counter()
    for _ in range(20):
        meta = get_meta()
    torch.cuda.synchronize()
    metadata_us = (time.perf_counter() - t0) / 20 * 1e6

    # the same schedule built on the device (one single-workgroup kernel)
    if case["sparse"]:
        dmeta = lambda: mla.mla_get_metadata_device(  # noqa: E731
            None, case["s_q"], case["h_q"], topk=case["topk"], active_h_q=case["active_h_q"],
            batch=int(case["q"].shape[0]), device=dev)
    else:
        dmeta = lambda: mla.mla_get_metadata_device(sl, case["s_q"], case["h_q"])  # noqa: E731
    dmeta()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        dmeta()
    e1.record()
    torch.cuda.synchronize()
    metadata_device_us = e0.elapsed_time(e1) / 20 * 1e3

    B, s_q, h_q = case["q"].shape[:3]
    out = torch.empty((B, s_q, h_q, case["d_v"]), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=dev)
    ws_bytes = meta.workspace_bytes(case["d_v"])
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def split(kv, m):
        if case["sparse"]:
            mla.mla_decode_sparse(q, kv, idx, case["d_v"], m, softmax_scale=case["softmax_scale"],
                                  workspace=ws, out=out, lse=lse, stage="split")
        else:
            mla.mla_decode_paged(q, kv, bt, sl, case["d_v"], m, causal=case["causal"],
                                 softmax_scale=case["softmax_scale"], workspace=ws, out=out,
                                 lse=lse, stage="split")

    def combine(m):
        mla.mla_combine(m, out, lse, ws, case["d_v"])

    for i in range(warmup):
        split(kvs[i % copies], meta)
        combine(meta)
    torch.cuda.synchronize()
    if probe:
        copy_probe(torch, dev)

    # The timed loops run as HIP-graph replays (torch.cuda.CUDAGraph over the
    # library's launches, captured once, default-priority stream): no host
    # work between the kernels, as in a serving loop that captures its decode
    # step.  Each graph holds exactly `steps` iterations; it is replayed
    # untimed for at least `settle_s` seconds (a short workload's few
    # milliseconds otherwise catch the clock still ramping up from idle),
    # then once between two events.
    settle_s = 0.2

    def capture(body):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        torch.cuda.synchronize()
        return g

    def replay_ms(g):
        t_settle = time.perf_counter()
        while True:
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t_settle >= settle_s:
                break
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def steps_body():
        for i in range(steps):
            split(kvs[i % copies], meta)
            combine(meta)

    def combine_body():
        for _ in range(steps):
            combine(meta)

    # whole decode steps (split-KV then combine), back to back
    g_step = capture(steps_body)
    ms_step = replay_ms(g_step)
    # per-kernel durations.  An event recorded between the two kernels of a
    # step adds a dispatch gap of several microseconds to both intervals, and
    # split-KV launches back to back with nothing between them run slower
    # than in the step loop.  So the combine is timed alone (`steps` launches
    # back to back) and the split-KV kernel is the whole step minus that:
    # the durations rocprofv3 reports for the launches of the step loop.
    comb_ms = 0.0
    if meta.num_split_units > 0:  # else the combine launches nothing
        g_comb = capture(combine_body)
        comb_ms = replay_ms(g_comb)
        del g_comb
    split_ms = ms_step - comb_ms
    del g_step

    # single steps: one graph per cache copy, replayed in rotation, each
    # replay timed on its own
    graphs = []
    for c in range(copies):
        graphs.append(capture(lambda c=c: (split(kvs[c], meta), combine(meta))))
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(replays)]
    for i in range(copies):
        graphs[i].replay()
    torch.cuda.synchronize()
    for i in range(replays):
        evs[i][0].record()
        graphs[i % copies].replay()
        evs[i][1].record()
    torch.cuda.synchronize()
    singles = sorted(a.elapsed_time(b) for a, b in evs)
    step_stats = {"replays": replays, "min": round(singles[0], 5),
                  "median": round(singles[len(singles) // 2], 5),
                  "max": round(singles[-1], 5)}
    del graphs

    # rate with the scheduler and its upload inside every step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        m = get_meta()
        split(kvs[i % copies], m)
        combine(m)
    torch.cuda.synchronize()
    ms_with_meta = (time.perf_counter() - t0) * 1e3 / steps

    ai = work["flop"] / work["bytes"]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if ai >= ridge else "hbm"
    if bound == "hbm":
        achieved = work["bytes"] / (split_ms * 1e-3) / 1e9
        peak, unit = PEAK_HBM_GBS, "GB/s"
    else:
        achieved = work["flop"] / (split_ms * 1e-3) / 1e12
        peak, unit = PEAK_BF16_TFLOPS, "TFLOP/s"
    res = dict(
        case=case, work=work, ms_step=ms_step, split_ms=split_ms, combine_ms=comb_ms,
        tflops=work["flop"] / (ms_step * 1e-3) / 1e12,
        gbs=work["bytes"] / (ms_step * 1e-3) / 1e9,
        metadata_us=metadata_us, metadata_device_us=metadata_device_us, ms_with_meta=ms_with_meta,
        roofline=dict(bound=bound, achieved=round(achieved, 2), peak=peak, unit=unit,
                      frac=round(achieved / peak, 4), traffic=None),
        sched=dict(num_parts=meta.num_parts, row_blocks=meta.row_blocks,
                   max_splits=meta.max_splits, split_units=meta.num_split_units,
                   workspace_mb=round(ws_bytes / 2**20, 2)),
        copies=copies, step_stats=step_stats,
    )
    return res


def prefill_work(case) -> dict:
    """Sparse prefill: FLOP over (query token, head, valid index); bytes = the
    KV rows once (they are shared by the queries) + q, out, lse, max_logits,
    indices."""
    idx = case["indices"]
    valid = ((idx >= 0) & (idx < case["s_kv"])).sum().item()
    s_q, h_q, d_qk, d_v = case["s_q"], case["h_q"], case["d_qk"], case["d_v"]
    flop = valid * h_q * 2 * (d_qk + d_v)
    byts = case["s_kv"] * d_qk * 2 + s_q * h_q * (d_qk * 2 + d_v * 2 + 8) + idx.numel() * 4
    return dict(flop=flop, bytes=byts, kv_bytes=case["s_kv"] * d_qk * 2, keys=valid)


def bench_prefill(steps: int, warmup: int, probe: bool = False) -> dict:
    """The sparse prefill chunk: one mla_sparse_prefill call per step."""
    import torch

    import mla_paged_kv_amd as mla
    from synth.configs import make_config
    import numpy as np

    case = make_config("p")
    work = prefill_work(case)
    dev = torch.device("cuda", 0)
    q, kv0, idx = case["q"].to(dev), case["kv"].to(dev), case["indices"].to(dev)
    copies = rotation_copies(work["bytes"])
    kvs = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    meta = mla.mla_get_metadata(np.zeros(case["s_q"], np.int32), 1, case["h_q"], topk=case["topk"],
                                device=dev)
    out = torch.empty((case["s_q"], case["h_q"], case["d_v"]), dtype=torch.bfloat16, device=dev)
    mx = torch.empty((case["s_q"], case["h_q"]), dtype=torch.float32, device=dev)
    lse = torch.empty_like(mx)
    ws = torch.empty(max(meta.workspace_bytes(case["d_v"]), 256), dtype=torch.uint8, device=dev)

    def run(i):
        mla.mla_sparse_prefill(q, kvs[i % copies], idx, case["softmax_scale"], dv=case["d_v"],
                               meta=meta, workspace=ws, out=out, max_logits=mx, lse=lse)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    if probe:
        copy_probe(torch, dev)
    # untimed calls for at least 0.2 s first, as for the decode timings
    t_settle = time.perf_counter()
    i = 0
    while time.perf_counter() - t_settle < 0.2:
        run(i)
        i += 1
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tflops = work["flop"] / (ms * 1e-3) / 1e12
    return dict(workload=case["name"], ms_per_step=round(ms, 5), tflops=round(tflops, 2),
                kernels_ms={"splitkv+combine": round(ms, 5)},
                algorithmic={"flop": work["flop"], "bytes": work["bytes"]},
                roofline=dict(bound="mfma", achieved=round(tflops, 2), peak=PEAK_BF16_TFLOPS,
                              unit="TFLOP/s", frac=round(tflops / PEAK_BF16_TFLOPS, 4), traffic=None),
                schedule=dict(num_parts=meta.num_parts, row_blocks=meta.row_blocks,
                              max_splits=meta.max_splits, split_units=meta.num_split_units),
                cache_copies_rotated=copies,
                note="split-KV and combine of one call, timed together")


# name stems of the split-KV kernels (one of them runs per workload)
SPLIT_KERNELS = ("mla_splitkv", "mla_decode", "mla_narrow")


def traffic_path(k) -> str:
    return os.path.join(ROOT, "profiles", f"splitkv_traffic_workload{k}.json")


def load_traffic(k):
    """HBM bytes per launch of the split-KV kernel from the committed counter
    summary of workload k, if it was taken on the current kernel source."""
    path = traffic_path(k)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def _counter_rows(path: str, counter: str):
    import csv
    rows = []
    with open(path, newline="") as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def ingest_counters(k: int, fetch_csv: str, write_csv: str, command: str) -> dict:
    """Turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) of ``bench.py --workload k --copy-probe`` into HBM bytes per
    split-KV launch (the pair kernel ``mla_splitkv``, the decode kernel
    ``mla_decode`` or the narrow kernel ``mla_narrow``, whichever the workload
    runs).  Each counter is scaled by bytes / reading of the copy
    probe in the same run (the neg kernel over COPY_PROBE_BYTES)."""
    out = {"workload": k, "kernel_hash": kernel_hash(), "command": command}
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _counter_rows(path, counter)
        split = [v for n, v in rows if any(k in n for k in SPLIT_KERNELS)]
        probe = [v for n, v in rows if "neg_kernel" in n]
        if not split or not probe:
            raise SystemExit(f"{path}: no split-KV or copy-probe dispatches with {counter}")
        kib = sum(split) / len(split)
        probe_kib = sorted(probe)[len(probe) // 2]
        factor = (COPY_PROBE_BYTES / 1024) / probe_kib
        out[name] = {"counter": counter, "dispatches": len(split), "kib_per_launch": round(kib, 1),
                     "probe_kib": round(probe_kib, 1), "probe_factor": round(factor, 4),
                     "bytes_per_launch": int(kib * 1024 * factor)}
    out["traffic_bytes_per_launch"] = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    with open(traffic_path(k), "w") as fh:
        json.dump(out, fh, indent=1)
        fh.write("\n")
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replays", type=int, default=100,
                    help="single steps timed one by one for step_ms (min / median)")
    ap.add_argument("--workload", default="2", choices=["1", "2", "3", "4", "5", "4f", "5f", "p"],
                    help="seeded workload (2 = varlen decode, h_q=128: the headline; 4f/5f: "
                         "FP8-cache variants of 4/5; p: the sparse prefill chunk)")
    ap.add_argument("--others", default="3,4,5,4f,5f,p",
                    help="extra workloads timed into 'other_workloads' ('' for none)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run the known-size copy used to scale HBM counters (profiling only)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two counter runs of --workload into the committed "
                         "traffic summary and exit")
    ap.add_argument("--ingest-command", default="", help="command recorded with --ingest-counters")
    args = ap.parse_args()

    if args.ingest_counters:
        print(json.dumps(ingest_counters(args.workload, *args.ingest_counters, args.ingest_command)))
        return

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only: sharding the decode over "
                                   "several GPUs is described, not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.workload == "p":  # the prefill chunk alone (profiling runs)
        o = bench_prefill(args.steps, args.warmup, probe=args.copy_probe)
        o["roofline"]["traffic"] = load_traffic("p")
        print(json.dumps(dict(o, kernel_source_hash=kernel_hash())), flush=True)
        return
    k = int(args.workload) if args.workload.isdigit() else args.workload
    r = bench_workload(k, args.steps, args.warmup, replays=args.replays, probe=args.copy_probe)
    case = r["case"]
    r["roofline"]["traffic"] = load_traffic(k)
    line = {
        "metric": METRIC,
        "value": round(r["tflops"], 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_step"], 5),
        "step_ms": r["step_stats"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case["name"], "batch": int(case["q"].shape[0]),
                   "s_q": case["s_q"], "h_q": case["h_q"], "d_qk": case["d_qk"],
                   "d_v": case["d_v"], "causal": case["causal"],
                   "visible_keys": r["work"]["keys"], "parallelism": "single GPU"},
        "hbm_gbps": round(r["gbs"], 1),
        "frac_mfma_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
        "frac_hbm_peak": round(r["gbs"] / PEAK_HBM_GBS, 4),
        "kernels_ms": {"splitkv": round(r["split_ms"], 5), "combine": round(r["combine_ms"], 5)},
        "metadata_us": round(r["metadata_us"], 1),
        "metadata_device_us": round(r["metadata_device_us"], 1),
        "with_metadata": {"ms_per_step": round(r["ms_with_meta"], 5),
                          "tflops": round(r["work"]["flop"] / (r["ms_with_meta"] * 1e-3) / 1e12, 3)},
        "schedule": r["sched"],
        "algorithmic": {"flop": r["work"]["flop"], "bytes": r["work"]["bytes"]},
        "cache_copies_rotated": r["copies"],
        "roofline": r["roofline"],
        "kernel_source_hash": kernel_hash(),
    }
    others = {}
    for k in [x.strip() for x in args.others.split(",") if x.strip()]:
        if k == str(args.workload):
            continue
        if k == "p":
            others["p"] = bench_prefill(max(10, args.steps // 5), 3)
            others["p"]["roofline"]["traffic"] = load_traffic("p")
            torch.cuda.empty_cache()
            continue
        o = bench_workload(k, max(10, args.steps // 2), max(3, args.warmup // 2),
                           replays=args.replays)
        o["roofline"]["traffic"] = load_traffic(k)
        others[str(k)] = {
            "workload": o["case"]["name"], "ms_per_step": round(o["ms_step"], 5),
            "step_ms": o["step_stats"], "cache_copies_rotated": o["copies"],
            "tflops": round(o["tflops"], 2), "hbm_gbps": round(o["gbs"], 1),
            "frac_mfma_peak": round(o["tflops"] / PEAK_BF16_TFLOPS, 4),
            "frac_hbm_peak": round(o["gbs"] / PEAK_HBM_GBS, 4),
            "kernels_ms": {"splitkv": round(o["split_ms"], 5), "combine": round(o["combine_ms"], 5)},
            "metadata_device_us": round(o["metadata_device_us"], 1),
            "kv_format": "fp8 with scale (656 B/row)" if o["case"].get("kv_fp8") else "bf16",
            "roofline": o["roofline"], "schedule": o["sched"],
        }
        del o
        torch.cuda.empty_cache()
    if others:
        line["other_workloads"] = others
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
