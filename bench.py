#!/usr/bin/env python3
"""Throughput of Prof-K exact top-k on one MI355X.

Workload: one flat fp32 tensor of N = 2^30 Pareto(alpha = 1.5, x_m = 1) values
(seed 0, generated on the host by workloads.py and copied to HBM before
timing), exact top-k for k in {2^5, 2^10, 2^15, 2^19}, eps = 1e-3.  One
"step" is the whole k sweep: four exact top-k calls over the resident tensor,
each including its sampling, threshold, filter, refinement and the host's wait
for the count R that the device publishes.  Each k is timed over K calls back
to back (HIP events on the stream around them; the host calls in turn, each
returning once its run-time check is known, so the next call queues behind the
previous refinement); `value` = 4 N / (sum over k of the mean call time).

Also printed (same JSON line):
  per_k        ms, Gelem/s and algorithmic GB/s (4N bytes per call) per k
  roofline     the filter kernel: algorithmic bytes (4N read + 8R written) per
               launch / its launch time from HIP events recorded by the library
               around the filter on the same stream; peak 8 TB/s
  batched      1024 rows x 2^20, top-64 per row (same tensor, reshaped)
  cpu_baseline the CPU oracle (plain C heap top-k) on a bounded sample
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KS = (1 << 5, 1 << 10, 1 << 15, 1 << 19)
EPS = 1e-3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--log2n", type=int, default=30, help="input size (default: the 2^30 workload)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched variant")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FILTER_FETCH_CSV", "FILTER_WRITE_CSV", "COPY_FETCH_CSV",
                                                         "COPY_WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs into the traffic record")
    return ap.parse_args()


def filter_source_hash() -> str:
    p = os.path.join(ROOT, "sampling_threshold_filtering_amd", "csrc", "k_filter.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_record(n: int):
    """HBM bytes per filter launch from the committed rocprofv3 counter summary, if it
    was taken on the current filter source and at this size; else None."""
    p = os.path.join(ROOT, "profiles", "filter_traffic_pareto_2p30.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("filter_source_sha256_16") != filter_source_hash() or rec.get("N") != n:
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 1 << 30


def calibrate_copy():
    """A plain device copy of known size, profiled with the same counters as the filter."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 3}), flush=True)


def _pmc_rows(path, name_pattern):
    """(kernel name, counter value) rows of a rocprofv3 counter_collection.csv."""
    import csv
    import re
    out = []
    with open(path) as f:
        for row in csv.DictReader(f):
            name = row.get("Kernel_Name") or row.get("Kernel-Name") or ""
            if re.search(name_pattern, name):
                out.append(float(row.get("Counter_Value") or row.get("Counter-Value")))
    return out


def summarize_pmc(paths):
    """Scale the filter's FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what the same
    counters read for a copy of known size, and write the traffic record."""
    ff, fw, cf, cw = paths
    f_fetch = _pmc_rows(ff, "filter_kernel")
    f_write = _pmc_rows(fw, "filter_kernel")
    c_fetch = _pmc_rows(cf, "copyBuffer")
    c_write = _pmc_rows(cw, "copyBuffer")
    kib = 1024.0
    fetch_scale = COPY_BYTES / (max(c_fetch) * kib)
    write_scale = COPY_BYTES / (max(c_write) * kib)
    fetch = float(np.mean(f_fetch)) * kib * fetch_scale
    write = float(np.mean(f_write)) * kib * write_scale
    N = 1 << 30
    rec = {"N": N, "filter_source_sha256_16": filter_source_hash(),
           "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
           "bytes_per_launch": round(fetch + write), "fetch_scale": round(fetch_scale, 4),
           "write_scale": round(write_scale, 4), "filter_dispatches": [len(f_fetch), len(f_write)],
           "read_bytes_algorithmic": 4 * N}
    out = os.path.join(ROOT, "profiles", "filter_traffic_pareto_2p30.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def cpu_baseline(x: np.ndarray):
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    threads = max(1, min(16, cores))
    n = x.size
    sample = x[:n]
    oracle.topk(sample[: 1 << 20], 32, nthreads=threads)  # warm the library and pages
    t0 = time.perf_counter()
    for k in KS:
        oracle.topk(sample, k, nthreads=threads)
    dt = time.perf_counter() - t0
    return {"value": round(len(KS) * n / dt / 1e9, 4), "unit": "Gelem/s", "cores": threads, "kind": "oracle",
            "sample": f"the same 2^{n.bit_length() - 1}-value tensor, k sweep {list(KS)}, "
                      f"{dt:.2f} s total; plain C heap top-k, {threads} threads"}


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see the sharding notes of the design document); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import sampling_threshold_filtering_amd as stf
    from workloads import generate

    N = 1 << args.log2n
    t_gen = time.perf_counter()
    x = generate("pareto", N, seed=0)
    gen_s = time.perf_counter() - t_gen
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    xd = torch.from_numpy(x).to(dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    opts = stf.make_options(timing=1)

    per_k = {}
    filt_bytes = 0.0
    filt_ms = 0.0
    total_ms = 0.0
    retries = 0
    for k in KS:
        out = (torch.empty(k, dtype=torch.float32, device=dev), torch.empty(k, dtype=torch.int64, device=dev))
        for _ in range(args.warmup):
            stf.topk(xd, k, eps=EPS, seed=0, options=opts, out=out)
        torch.cuda.synchronize()
        # K calls back to back, bracketed by events on the stream (each call waits
        # only for its run-time check; the next one is enqueued behind it)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(args.steps):
            _, _, st = stf.topk(xd, k, eps=EPS, seed=s, options=opts, stats=True, out=out)
            filt_ms += st["filter_ms"]
            filt_bytes += 4.0 * N + 8.0 * st["R"][-1]
            retries += st["attempts"] - 1
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        total_ms += ms
        per_k[str(k)] = {"ms": round(ms, 4), "gelem_s": round(N / ms / 1e6, 2),
                         "alg_GBps": round(4.0 * N / ms / 1e6, 1),
                         "frac_of_hbm_peak": round(4.0 * N / ms / 1e6 / HBM_PEAK_GBPS, 4)}
    torch.cuda.synchronize()

    n_filter = args.steps * len(KS)
    achieved = filt_bytes / n_filter / (filt_ms / n_filter / 1e3) / 1e9
    traffic = traffic_record(N)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": "filter_kernel", "filter_ms_avg": round(filt_ms / n_filter, 4),
                "bytes_per_launch_alg": round(filt_bytes / n_filter)}

    batched = None
    if not args.no_batched and N >= (1 << 20) * 16:
        B = min(1024, N >> 20)
        xb = xd[: B << 20].view(B, 1 << 20)
        for _ in range(max(1, args.warmup)):
            stf.topk_batched(xb, 64, eps=EPS, seed=0)
        torch.cuda.synchronize()
        nb = max(1, args.steps // 2)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(nb):
            stf.topk_batched(xb, 64, eps=EPS, seed=s)
        e1.record(stream)
        e1.synchronize()
        bt = [e0.elapsed_time(e1) / nb]
        bms = float(np.mean(bt))
        batched = {"rows": B, "row_len": 1 << 20, "k": 64, "ms": round(bms, 4),
                   "gelem_s": round((B << 20) / bms / 1e6, 2)}

    cpu = None if args.no_cpu else cpu_baseline(x)

    value = len(KS) * N / (total_ms / 1e3) / 1e9
    line = {
        "metric": "Gelem/s + % of HBM peak, exact top-k N=2^30 fp32, k=2^5..2^19, 1 GPU",
        "value": round(value, 2),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"Pareto(1.5) fp32 flat tensor N=2^{args.log2n}, seed 0, exact top-k k sweep "
                               f"{list(KS)}, eps=1e-3", "N": N, "ks": list(KS), "eps": EPS},
        "hbm_frac_alg": round(4.0 * N * len(KS) / (total_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
        "per_k": per_k,
        "retries": retries,
        "roofline": roofline,
        "batched": batched,
        "cpu_baseline": cpu,
        "host_gen_s": round(gen_s, 2),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
