#!/usr/bin/env python3
"""Throughput of Prof-K exact top-k on one MI355X.

Headline workload: flat fp32 tensors of N = 2^30 Pareto(alpha = 1.5, x_m = 1)
values (three input tensors, seeds 0, 1, 2, generated on the host by
workloads.py and copied to HBM before timing), exact top-k for k in {2^5, 2^10,
2^15, 2^19}, eps = 1e-3.  One "step" is the whole k sweep: four exact top-k
calls, each including its sampling, threshold, filter, refinement and the host's
wait for the count R that the device publishes.  Each k is timed over K calls
back to back (HIP events on the stream around them; the host calls in turn, each
returning once its run-time check is known, so the next call queues behind the
previous refinement), the calls rotating over the input tensors; `value` =
4 N / (sum over k of the mean call time).  The sample size follows the rule
calibrated on MI355X (--s-rule 2: Algorithm 1 of the page with the cost ratio
that `--calibrate-s` measures); the same sweep under the library's default
(k N)^(1/3) rule is printed beside it.

Also printed (same JSON line):
  per_k        ms, Gelem/s and algorithmic GB/s (4N bytes per call) per k
  roofline     the filter kernel: algorithmic bytes (4N read + 8R written) per
               launch / its launch time from HIP events recorded by the library
               around the filter on the same stream (in a second pass over the
               same calls, so that the events do not enter `value`); peak 8 TB/s
  read_ceiling one dwordx4 non-temporal read of the 2^30 buffer and nothing else
               (profk_read_ceiling), best of a blocks-per-CU sweep: the practical
               ceiling of the filter on this device
  configs      every other workload of the hot-path scope: uniform 2^22 k = 32;
               normal and uniform 2^26 with k in {32, 1024, 32768}; the SAE pool
               (4096 x 12288, k = 131072); the two radix-adversarial readings at
               2^30 with k = 2^19 and eps = 1e-4, plus the forced-overflow run
               (M = k: six failed attempts, then the exact full selection) and
               the exact full selection alone.  Inputs below 2^27 values rotate
               over copies totalling at least 768 MB, so that the 256 MB last-
               level cache does not serve the reads.  Each entry gives ms per call,
               Gelem/s, the fraction of the one-read roofline (4N bytes at 8 TB/s)
               and the workspace the library held.
  batched      1024 rows x 2^20, top-64 per row (input tensor 0, reshaped)
  large        N = 4.3e9 (beyond 32-bit indexing), k in {2^10, 2^18, 2^22}
  cpu_baseline the CPU oracle (plain C heap top-k) on a bounded sample, with
               the threads it used, and a single-thread figure
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
S_RULE_NAMES = {0: "cube-root (k N)^(1/3), S in [2^15, 2^17]", 1: "Algorithm 1, page cost ratio",
                2: "Algorithm 1, cost ratio measured on MI355X, S in [2^12, 2^17]"}
KS = (1 << 5, 1 << 10, 1 << 15, 1 << 19)
EPS = 1e-3


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # untimed calls per k before the timed ones: the filter's per-die shares settle over
    # about ten calls after the library starts (measured: 620-625 us per filter pass in
    # calls 2-5 at 2^30 values, ~600 us from call 10 on)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--log2n", type=int, default=30, help="input size (default: the 2^30 workload)")
    ap.add_argument("--s-rule", type=int, default=2, choices=(0, 1, 2),
                    help="sample-size rule: 0 the (kN)^(1/3) rule clamped to [2^15, 2^17] (the library default), "
                         "1 Algorithm 1 with the page's cost ratio, 2 Algorithm 1 with the ratio measured on "
                         "MI355X (default here)")
    ap.add_argument("--inputs", type=int, default=3,
                    help="input tensors of the headline workload (Pareto seeds 0, 1, ...); calls rotate over them")
    ap.add_argument("--only", default="",
                    help="comma list of parts to run (flat, ceiling, configs, c1, c2, c3, c5, t7, batched, large, cpu); "
                         "default all.  c1/c2/c3/c5/t7 select single entries of configs, e.g. for a profile")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-batched", action="store_true", help="skip the batched variant")
    ap.add_argument("--no-large", action="store_true", help="skip the N = 4.3e9 (beyond 2^32) measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    ap.add_argument("--calibrate-s", metavar="OUT_JSON",
                    help="sweep the sample size S over an (N, k) grid, fit the cost model of the sample-size "
                         "rule and write the measurements and the fit to OUT_JSON")
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
    """The CPU oracle on the host cores of this machine: the multi-thread heap top-k over
    the whole k sweep of the 2^30 input for about 10 s, and the single-thread one on a
    2^26-value prefix for about 10 s (both scaled to Gelem/s)."""
    import oracle
    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count() or 1
    threads = max(1, min(16, host_cores))
    n = x.size
    oracle.topk(x[: 1 << 20], 32, nthreads=threads)  # warm the library and pages

    def run(sample, nthreads, budget):
        t0 = time.perf_counter()
        reps = 0
        while True:  # whole k sweeps until about `budget` seconds of CPU work
            for k in KS:
                oracle.topk(sample, k, nthreads=nthreads)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= budget or reps >= 32:
                return reps, dt

    reps, dt = run(x, threads, 10.0)
    m = 1 << 26
    reps1, dt1 = run(x[:m], 1, 10.0)
    return {"value": round(reps * len(KS) * n / dt / 1e9, 4), "unit": "Gelem/s", "cores": threads,
            "host_cores": host_cores, "kind": "oracle",
            "sample": f"the 2^{n.bit_length() - 1}-value Pareto tensor (seed 0), k sweep {list(KS)} repeated {reps} "
                      f"times, {dt:.2f} s; plain C heap top-k on {threads} threads (the box has {host_cores} "
                      f"host cores available)",
            "single_thread": {"value": round(reps1 * len(KS) * m / dt1 / 1e9, 4), "unit": "Gelem/s", "cores": 1,
                              "sample": f"its first 2^26 values, k sweep {list(KS)} repeated {reps1} times, "
                                        f"{dt1:.2f} s on one thread"}}


# ---------------------------------------------------------------------------
# Sample-size calibration ("Prof-K: Probabilistic One-Pass Filtering for Efficient
# Top-k Selection", App. E.1 "Sample Size"; §4 "Choice of the Sample Size", Eq. 13
# and Proposition 7).  The overhead beyond the scan is modelled as
#   C(S) = c + (g + b) S + d(k) M*(S)
# with one intercept c per (N, k), one sampling cost g + b and one buffer cost d(k)
# per k; the ratio 1/r(k) = d(k) / (g + b) is what the cost-model S rule takes.
# The grid is the page's (S = 2^12 .. 2^18 capped at N/32, exact (t*, M*) at
# eps = 1e-3, standard normal inputs, k = 2^5 .. 2^17) with N up to 2^30 and k = 2^19
# added.  Besides the page's per-k least-squares fit, one constant 1/r (and the
# floor S_min) is fitted by direct search: the value whose Proposition-7 rule gives
# the lowest mean latency relative to the best grid point (the rule without the
# page's S_min floor for k/N > 2^-10, as the library's MI355X rule takes it).
CAL_LOG2N = (22, 24, 26, 28, 30)
CAL_KS = (1 << 5, 1 << 8, 1 << 11, 1 << 14, 1 << 17, 1 << 19)
CAL_LOG2S = tuple(range(12, 19))
CAL_CALLS = 10


def _time_calls(stf, torch, xd, k, opts, calls, warmup, stream, out):
    for w in range(warmup):
        stf.topk(xd, k, eps=EPS, seed=1000 + w, options=opts, out=out)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    fms, rs, att = 0.0, 0.0, 0
    e0.record(stream)
    for s in range(calls):
        _, _, st = stf.topk(xd, k, eps=EPS, seed=s, options=opts, stats=True, out=out)
        fms += st["filter_ms"]
        rs += st["R"][-1] if st["R"] else 0
        att += st["attempts"]
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / calls, fms / calls, rs / calls, att / calls


def _fit_cost_model(rows):
    """Least squares of overhead = c[N,k] + gb * S + d[k] * M over the rows whose
    sampler runs its one-pass form (S <= 2^17 and S <= N/64; beyond that the
    threshold select and the top-up change the per-sample cost)."""
    use = [r for r in rows if (1 << 14) <= r["S"] <= (1 << 17) and 64 * r["S"] <= r["N"]]
    cfgs = sorted({(r["N"], r["k"]) for r in use})
    ks = sorted({r["k"] for r in use})
    ncol = len(cfgs) + 1 + len(ks)
    A = np.zeros((len(use), ncol))
    y = np.zeros(len(use))
    for i, r in enumerate(use):
        A[i, cfgs.index((r["N"], r["k"]))] = 1.0
        A[i, len(cfgs)] = r["S"]
        A[i, len(cfgs) + 1 + ks.index(r["k"])] = r["M"]
        y[i] = r["overhead_ms"] * 1e6  # ns
    coef, *_ = np.linalg.lstsq(A, y, rcond=None)
    pred = A @ coef
    gb = float(coef[len(cfgs)])
    d = {k: float(coef[len(cfgs) + 1 + j]) for j, k in enumerate(ks)}
    ss_res = float(np.sum((y - pred) ** 2))
    ss_tot = float(np.sum((y - y.mean()) ** 2))
    call_ns = np.array([r["ms"] * 1e6 for r in use])
    inv_r = {k: (d[k] / gb if gb > 0 and d[k] > 0 else 0.0) for k in ks}
    return {"sampling_ns_per_elem": gb, "buffer_ns_per_slot": {str(k): v for k, v in d.items()},
            "inv_r": {str(k): v for k, v in inv_r.items()},
            "r2_overhead": 1.0 - ss_res / ss_tot if ss_tot > 0 else None,
            "mean_rel_err_of_call": float(np.mean(np.abs(y - pred) / call_ns)),
            "mean_rel_err_of_overhead": float(np.mean(np.abs(y - pred) / np.maximum(y, 1.0))),
            "rows_fitted": len(use)}


def _prop7_s(N, k, z, inv_r, s_min, s_max):
    """Algorithm 1 lines 3-4 for a constant 1/r, without the floor for k/N > 2^-10
    (the measurement's own copy: it only scores sample sizes on the measured grid)."""
    if inv_r <= 0.0:
        S = s_min
    else:
        kappa = z * z + 0.5
        s1 = (z * inv_r) ** (2.0 / 3.0) * (k * N) ** (1.0 / 3.0)
        s2 = (kappa * N * inv_r) ** 0.5
        S = max(s_min, min(s_max, int(max(s1, s2))))
    return min(S, max(1, N // 128))


def _fit_constant_ratio(rows, z):
    """Direct search for one 1/r and S_min: the rule's latency, interpolated in log2 S
    between grid points, relative to the best grid latency, averaged over (N, k)."""
    grid = {}
    for r in rows:
        grid.setdefault((r["N"], r["k"]), {})[r["S"]] = r["ms"]
    best = None
    for s_min in (1 << 12, 1 << 13, 1 << 14):
        for inv_r in np.geomspace(0.002, 1.0, 61):
            ratios = []
            for (N, k), m in grid.items():
                ss = sorted(m)
                S = _prop7_s(N, k, z, inv_r, s_min, 1 << 17)
                lat = float(np.interp(np.log2(S), np.log2(ss), [m[v] for v in ss]))
                ratios.append(lat / min(m.values()))
            cand = (float(np.mean(ratios)), float(inv_r), s_min, float(np.max(ratios)))
            if best is None or cand[0] < best[0]:
                best = cand
    return {"inv_r": best[1], "s_min": best[2], "s_max": 1 << 17, "mean_latency_ratio_to_best": best[0],
            "worst_latency_ratio_to_best": best[3]}


def calibrate_s(path: str, calls: int = CAL_CALLS):
    import torch

    import sampling_threshold_filtering_amd as stf
    from workloads import generate

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nmax = 1 << max(CAL_LOG2N)
    x = torch.from_numpy(generate("normal", nmax, seed=0)).to(dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    rows = []
    for ln in CAL_LOG2N:
        N = 1 << ln
        xd = x[:N]
        for k in CAL_KS:
            out = (torch.empty(k, dtype=torch.float32, device=dev), torch.empty(k, dtype=torch.int64, device=dev))
            for ls in CAL_LOG2S:
                S = 1 << ls
                if S > N // 32:
                    continue
                opts = stf.make_options(timing=1, s_override=S)
                p = stf.solve(N, k, EPS, options=opts)
                if p["direct_exact"]:
                    continue
                ms, fms, r_mean, att = _time_calls(stf, torch, xd, k, opts, calls, 2, stream, out)
                row = {"N": N, "k": k, "S": S, "t": p["t"], "M": p["M"], "ms": ms, "filter_ms": fms,
                       "overhead_ms": ms - fms, "R_mean": r_mean, "attempts_mean": att}
                rows.append(row)
                print(json.dumps(row), flush=True)
    z = stf.solve(1 << 30, 32, EPS)["z_a"]
    fit = _fit_cost_model(rows)
    const = _fit_constant_ratio(rows, z)
    print(json.dumps({"fit": fit, "constant_ratio_fit": const}), flush=True)
    # latency at the S each rule of the library picks, next to the best grid point
    rules = {"cube_root": {"s_rule": 0}, "cost_model_page": {"s_rule": 1}, "mi355x": {"s_rule": 2}}
    picks = []
    for ln in CAL_LOG2N:
        N = 1 << ln
        xd = x[:N]
        for k in CAL_KS:
            out = (torch.empty(k, dtype=torch.float32, device=dev), torch.empty(k, dtype=torch.int64, device=dev))
            grid = [r for r in rows if r["N"] == N and r["k"] == k]
            if not grid:
                continue
            best = min(grid, key=lambda r: r["ms"])
            rec = {"N": N, "k": k, "best_grid_S": best["S"], "best_grid_ms": best["ms"]}
            for name, kw in rules.items():
                opts = stf.make_options(timing=1, **kw)
                p = stf.solve(N, k, EPS, options=opts)
                ms, _, r_mean, _ = _time_calls(stf, torch, xd, k, opts, calls, 2, stream, out)
                rec[name] = {"S": p["S"], "ms": ms, "R_mean": r_mean, "direct_exact": p["direct_exact"]}
            picks.append(rec)
            print(json.dumps(rec), flush=True)
    res = {"workload": "standard normal fp32, seed 0, prefixes of one 2^30 tensor", "eps": EPS, "calls": calls,
           "grid": rows, "fit": fit, "constant_ratio_fit": const, "rules": picks}
    with open(path, "w") as f:
        json.dump(res, f, indent=1)

LARGE_N = 4_300_000_000
LARGE_KS = (1 << 10, 1 << 18, 1 << 22)


def bench_large(stf, torch, dev, stream, args, opts):
    """Inputs beyond 2^32 values (the page's Table 4: N = 4.3e9, k = 2^10, 2^18, 2^22):
    standard normal fp32 drawn on the device by torch's seeded generator (seed 0),
    exact top-k through the segmented path, mean call time over the timed calls."""
    free = torch.cuda.mem_get_info(dev)[0]
    if free < 4 * LARGE_N + (2 << 30):
        return None
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    x = torch.randn(LARGE_N, dtype=torch.float32, device=dev, generator=gen)
    res = {"N": LARGE_N, "input": "standard normal fp32, torch.randn on the device, seed 0"}
    for k in LARGE_KS:
        out = (torch.empty(k, dtype=torch.float32, device=dev), torch.empty(k, dtype=torch.int64, device=dev))
        for _ in range(max(1, args.warmup)):
            stf.topk(x, k, eps=EPS, seed=0, options=opts, out=out)
        torch.cuda.synchronize()
        n = max(1, args.steps // 2)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for s in range(n):
            _, _, st = stf.topk(x, k, eps=EPS, seed=s, options=opts, out=out, stats=True)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / n
        res[str(k)] = {"ms": round(ms, 4), "gelem_s": round(LARGE_N / ms / 1e6, 2),
                       "frac_of_hbm_peak": round(4.0 * LARGE_N / ms / 1e6 / HBM_PEAK_GBPS, 4),
                       "segments": st["segments"]}
    del x
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


INPUT_DIGESTS = {}  # name -> digest of every host-generated input tensor (see digest())


def digest(name: str, x: np.ndarray) -> None:
    """Record a SHA-256 of the tensor's bytes, taken as the SHA-256 of the concatenated
    SHA-256 digests of its 2^24-value chunks (so that the chunks hash on several threads)."""
    from concurrent.futures import ThreadPoolExecutor
    b = np.ascontiguousarray(x).reshape(-1).view(np.uint8)
    step = 4 << 24
    parts = [b[i:i + step] for i in range(0, b.size, step)]
    with ThreadPoolExecutor(max_workers=16) as ex:
        ds = list(ex.map(lambda c: hashlib.sha256(memoryview(c)).digest(), parts))
    INPUT_DIGESTS[name] = hashlib.sha256(b"".join(ds)).hexdigest()[:16]


def progress(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_calls(stf, torch, bufs, k, eps, opts, calls, warmup, stream, out):
    """Mean ms per exact call over `calls` calls back to back, rotating over `bufs`
    (seed = call number), after `warmup` untimed calls."""
    for w in range(warmup):
        stf.topk(bufs[w % len(bufs)], k, eps=eps, seed=w, options=opts, out=out)
    torch.cuda.synchronize()
    e0, e1 = _events(torch)
    e0.record(stream)
    for c in range(calls):
        stf.topk(bufs[c % len(bufs)], k, eps=eps, seed=c, options=opts, out=out)
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / calls


MALL_DEFEAT_BYTES = 768 << 20  # > 512 MB: twice the 256 MB last-level cache, and more


def rotation(torch, xd):
    """Device copies of xd totalling at least MALL_DEFEAT_BYTES when xd is smaller than
    that (the same values at other addresses), else [xd]."""
    n = xd.numel()
    c = -(-MALL_DEFEAT_BYTES // (4 * n))
    if c <= 1:
        return [xd]
    big = torch.empty((c, n), dtype=torch.float32, device=xd.device)
    big.copy_(xd.unsqueeze(0).expand(c, n))
    return [big[i] for i in range(c)]


def out_pair(torch, dev, k):
    return torch.empty(k, dtype=torch.float32, device=dev), torch.empty(k, dtype=torch.int64, device=dev)


def entry(N, k, eps, ms, p, copies):
    return {"N": N, "k": k, "eps": eps, "ms": round(ms, 4), "gelem_s": round(N / ms / 1e6, 2),
            "frac_of_roofline": round(4.0 * N / ms / 1e6 / HBM_PEAK_GBPS, 4), "S": p["S"], "t": p["t"], "M": p["M"],
            "input_copies": copies}


def read_ceiling(stf, torch, xd, stream, reps=10):
    """profk_read_ceiling on xd for 1, 2, 3, 4 blocks per CU: GB/s of one read."""
    fold = torch.zeros(1, dtype=torch.int64, device=xd.device)
    sweep = {}
    for bpc in (1, 2, 3, 4):
        for _ in range(3):
            stf.read_ceiling(xd, bpc, out=fold)
        torch.cuda.synchronize()
        e0, e1 = _events(torch)
        e0.record(stream)
        for _ in range(reps):
            stf.read_ceiling(xd, bpc, out=fold)
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        sweep[str(bpc)] = {"us": round(ms * 1e3, 1), "GBps": round(4.0 * xd.numel() / ms / 1e6, 1)}
    best = max(sweep, key=lambda b: sweep[b]["GBps"])
    return {"kernel": "read_ceiling_kernel (dwordx4 non-temporal, 4 float4 per lane per tile, the filter's order)",
            "N": xd.numel(), "best_blocks_per_cu": int(best), "GBps": sweep[best]["GBps"],
            "frac_of_peak": round(sweep[best]["GBps"] / HBM_PEAK_GBPS, 4), "sweep": sweep}


def bench_configs(stf, torch, dev, stream, args, opts, want, keep):
    """The other workloads of the hot-path scope, each at its own sizes; `keep` collects
    (name, tensor, k, eps, options) for the workspace pass."""
    from workloads import generate, sae_pool
    res = {}
    calls = max(args.steps, 30)
    warm = max(args.warmup, 5)
    if "c1" in want:
        N, k = 1 << 22, 32
        xh = generate("uniform", N, seed=0)
        digest("uniform_2p22", xh)
        bufs = rotation(torch, torch.from_numpy(xh).to(dev))
        ms = time_calls(stf, torch, bufs, k, EPS, opts, calls, warm, stream, out_pair(torch, dev, k))
        res["uniform_2p22"] = {"32": entry(N, k, EPS, ms, stf.solve(N, k, EPS, options=opts), len(bufs))}
        progress("uniform 2^22", round(ms, 4), "ms")
        keep.append(("uniform_2p22/32", bufs[0], k, EPS, opts))
    if "c2" in want:
        N = 1 << 26
        for kind in ("normal", "uniform"):
            xh = generate(kind, N, seed=0)
            digest(f"{kind}_2p26", xh)
            bufs = rotation(torch, torch.from_numpy(xh).to(dev))
            r = {}
            for k in (32, 1024, 32768):
                ms = time_calls(stf, torch, bufs, k, EPS, opts, calls, warm, stream, out_pair(torch, dev, k))
                r[str(k)] = entry(N, k, EPS, ms, stf.solve(N, k, EPS, options=opts), len(bufs))
                progress(kind, "2^26 k", k, round(ms, 4), "ms")
                keep.append((f"{kind}_2p26/{k}", bufs[0], k, EPS, opts))
            res[f"{kind}_2p26"] = r
        a = [res["normal_2p26"][str(k)]["ms"] for k in (32, 1024, 32768)]
        b = [res["uniform_2p26"][str(k)]["ms"] for k in (32, 1024, 32768)]
        res["normal_vs_uniform_2p26_ms_ratio"] = [round(x / y, 3) for x, y in zip(a, b)]
    if "c3" in want:
        N, k = 50331648, 131072
        xh = sae_pool(0).reshape(-1)
        digest("sae_pool_4096x12288", xh)
        bufs = rotation(torch, torch.from_numpy(xh).to(dev))
        ms = time_calls(stf, torch, bufs, k, EPS, opts, calls, warm, stream, out_pair(torch, dev, k))
        res["sae_pool_4096x12288"] = {"131072": entry(N, k, EPS, ms, stf.solve(N, k, EPS, options=opts), len(bufs))}
        progress("sae pool", round(ms, 4), "ms")
        keep.append(("sae_pool_4096x12288/131072", bufs[0], k, EPS, opts))
    if "c5" in want:
        N, k, eps = 1 << 30, 1 << 19, 1e-4
        for kind in ("adv_levels", "adv_noise"):
            xh = generate(kind, N, seed=0)
            digest(f"{kind}_2p30", xh)
            xd = torch.from_numpy(xh).to(dev)
            del xh
            out = out_pair(torch, dev, k)
            ms = time_calls(stf, torch, [xd], k, eps, opts, args.steps, args.warmup, stream, out)
            e = entry(N, k, eps, ms, stf.solve(N, k, eps, options=opts), 1)
            keep.append((f"{kind}_2p30/{k}", xd, k, eps, opts))
            if kind == "adv_levels":
                # forced overflow: M = k fails every attempt (R > M), then the exact full selection
                fo = stf.make_options(s_rule=opts.s_rule, force_M=k)
                _, _, st = stf.topk(xd, k, eps=eps, seed=0, options=fo, stats=True, out=out)
                fms = time_calls(stf, torch, [xd], k, eps, fo, 3, 1, stream, out)
                ex = stf.make_options(s_rule=opts.s_rule, force_fallback=1)
                xms = time_calls(stf, torch, [xd], k, eps, ex, 3, 1, stream, out)
                e["forced_overflow_M_eq_k"] = {"ms": round(fms, 4), "attempts": st["attempts"],
                                               "fallback": st["fallback"], "R_first_attempt": st["R"][0]}
                e["exact_full_selection_ms"] = round(xms, 4)
            res[f"{kind}_2p30"] = {str(k): e}
            progress(kind, "2^30", e)
    if "t7" in want:
        # the page's distribution sweep (Table 7): uniform [0,1) for reference, then
        # uniform [1,2), uniform [128.6, 128.7], log-normal, exponential, Cauchy, at 2^27
        # (rotated past the MALL) and 2^30 values, k in {2^8, 2^13}, eps = 1e-3
        t7 = {}
        for log2n in (27, 30):
            N = 1 << log2n
            for kind in ("uniform", "uniform12", "narrow", "lognormal", "exponential", "cauchy"):
                xh = generate(kind, N, seed=0)
                digest(f"{kind}_2p{log2n}", xh)
                xd = torch.from_numpy(xh).to(dev)
                del xh
                bufs = rotation(torch, xd)
                r = {}
                for k in (1 << 8, 1 << 13):
                    c, w = (args.steps, args.warmup) if log2n >= 30 else (calls, warm)
                    ms = time_calls(stf, torch, bufs, k, EPS, opts, c, w, stream, out_pair(torch, dev, k))
                    r[str(k)] = entry(N, k, EPS, ms, stf.solve(N, k, EPS, options=opts), len(bufs))
                t7[f"{kind}_2p{log2n}"] = r
                progress("table 7", kind, f"2^{log2n}", {k: v["ms"] for k, v in r.items()})
                del bufs, xd
                torch.cuda.empty_cache()
            for k in ("256", "8192"):
                ref = t7[f"uniform_2p{log2n}"][k]["ms"]
                t7.setdefault(f"ms_over_uniform_2p{log2n}", {})[k] = {
                    kind: round(t7[f"{kind}_2p{log2n}"][k]["ms"] / ref, 3)
                    for kind in ("uniform12", "narrow", "lognormal", "exponential", "cauchy")}
        res["table7_distributions"] = t7
    return res


def main():
    args = parse()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_s:
        calibrate_s(args.calibrate_s)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(see the sharding notes of the design document); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import sampling_threshold_filtering_amd as stf
    from workloads import generate

    parts = {"flat", "ceiling", "configs", "c1", "c2", "c3", "c5", "t7", "batched", "large", "cpu"}
    want = set(p.strip() for p in args.only.split(",") if p.strip()) or set(parts)
    if not want <= parts:
        sys.exit(f"--only: unknown parts {sorted(want - parts)}")
    if "configs" in want:
        want |= {"c1", "c2", "c3", "c5", "t7"}
    if args.no_cpu:
        want.discard("cpu")
    if args.no_batched:
        want.discard("batched")
    if args.no_large:
        want.discard("large")
    need_pareto = bool(want & {"flat", "ceiling", "batched", "cpu"})

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    N = 1 << args.log2n
    opts = stf.make_options(s_rule=args.s_rule)
    opts_t = stf.make_options(timing=1, s_rule=args.s_rule)
    keep = []

    x0 = None
    xds = []
    gen_s = 0.0
    if need_pareto:
        t_gen = time.perf_counter()
        for i in range(max(1, args.inputs) if "flat" in want else 1):
            x = generate("pareto", N, seed=i)
            digest(f"pareto_2p{args.log2n}_seed{i}", x)
            if i == 0:
                x0 = x
            xds.append(torch.from_numpy(x).to(dev))
            del x
        gen_s = time.perf_counter() - t_gen
        torch.cuda.synchronize()

    per_k, other_rule, roofline, value, total_ms, retries = None, None, None, None, None, 0
    if "flat" in want:
        per_k = {}
        filt_bytes = filt_ms = total_ms = 0.0
        # warm-up steps: whole sweeps over the k values first (the first ~20 calls on a
        # fresh process run 1-1.5% slower while the GPU settles), then per k below
        for w in range(args.warmup):
            for k in KS:
                stf.topk(xds[w % len(xds)], k, eps=EPS, seed=2000 + w, options=opts, out=out_pair(torch, dev, k))
        torch.cuda.synchronize()
        for k in KS:
            out = out_pair(torch, dev, k)
            # K calls back to back, bracketed by events on the stream (each call waits
            # only for its run-time check; the next one is enqueued behind it).  No stats
            # are requested here: building them on the host delays the next call's launch.
            ms = time_calls(stf, torch, xds, k, EPS, opts, args.steps, args.warmup, stream, out)
            # the filter's own launch time, from HIP events the library records around it,
            # and the attempts of the same calls (a separate pass: neither is part of the
            # timed calls above)
            for c in range(args.steps):
                _, _, st = stf.topk(xds[c % len(xds)], k, eps=EPS, seed=c, options=opts_t, stats=True, out=out)
                retries += st["attempts"] - 1
                filt_ms += st["filter_ms"]
                filt_bytes += 4.0 * N + 8.0 * st["R"][-1]
            total_ms += ms
            progress("pareto 2^30 k", k, round(ms, 4), "ms")
            per_k[str(k)] = {"ms": round(ms, 4), "gelem_s": round(N / ms / 1e6, 2),
                             "alg_GBps": round(4.0 * N / ms / 1e6, 1),
                             "frac_of_hbm_peak": round(4.0 * N / ms / 1e6 / HBM_PEAK_GBPS, 4)}
            keep.append((f"pareto_2p30/{k}", xds[0], k, EPS, opts))
        torch.cuda.synchronize()
        value = len(KS) * N / (total_ms / 1e3) / 1e9
        # the same sweep with the library's default sample-size rule, for comparison
        if args.s_rule != 0:
            other_rule = {}
            o0 = stf.make_options(s_rule=0)
            for k in KS:
                ms = time_calls(stf, torch, xds, k, EPS, o0, args.steps, args.warmup, stream, out_pair(torch, dev, k))
                other_rule[str(k)] = {"ms": round(ms, 4), "S": stf.solve(N, k, EPS, options=o0)["S"]}
        n_filter = args.steps * len(KS)
        achieved = filt_bytes / n_filter / (filt_ms / n_filter / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_record(N),
                    "kernel": "filter_kernel", "filter_ms_avg": round(filt_ms / n_filter, 4),
                    "bytes_per_launch_alg": round(filt_bytes / n_filter)}

    ceiling = read_ceiling(stf, torch, xds[0], stream) if "ceiling" in want else None
    if ceiling:
        progress("read ceiling", ceiling["GBps"], "GB/s")
    if ceiling and roofline:
        roofline["frac_of_read_ceiling"] = round(roofline["achieved"] / ceiling["GBps"], 4)

    batched = None
    if "batched" in want and N >= (1 << 20) * 16:
        B = min(1024, N >> 20)
        xb = xds[0][: B << 20].view(B, 1 << 20)
        bopts = stf.make_options(s_rule=args.s_rule)
        for _ in range(max(1, args.warmup)):
            stf.topk_batched(xb, 64, eps=EPS, seed=0, options=bopts)
        torch.cuda.synchronize()
        nb = max(1, args.steps // 2)
        e0, e1 = _events(torch)
        e0.record(stream)
        for c in range(nb):
            stf.topk_batched(xb, 64, eps=EPS, seed=c, options=bopts)
        e1.record(stream)
        e1.synchronize()
        bms = e0.elapsed_time(e1) / nb
        progress("batched 1024 x 2^20", round(bms, 4), "ms")
        batched = {"rows": B, "row_len": 1 << 20, "k": 64, "ms": round(bms, 4),
                   "gelem_s": round((B << 20) / bms / 1e6, 2),
                   "frac_of_roofline": round(4.0 * (B << 20) / bms / 1e6 / HBM_PEAK_GBPS, 4),
                   "S_per_row": stf.solve(1 << 20, 64, EPS / B, options=bopts)["S"]}

    batched_long = None
    if "batched" in want and N >= (1 << 26):
        # rows longer than 2^20 (the page's N = 2^22, B = 16), next to one flat call over
        # the same 2^26 values
        xl = xds[0][: 1 << 26]
        xb = xl.view(16, 1 << 22)
        bopts = stf.make_options(s_rule=args.s_rule)
        batched_long = {"rows": 16, "row_len": 1 << 22}
        for k in (64, 1024):
            for _ in range(max(1, args.warmup)):
                stf.topk_batched(xb, k, eps=EPS, seed=0, options=bopts)
            torch.cuda.synchronize()
            e0, e1 = _events(torch)
            e0.record(stream)
            for c in range(args.steps):
                stf.topk_batched(xb, k, eps=EPS, seed=c, options=bopts)
            e1.record(stream)
            e1.synchronize()
            bms = e0.elapsed_time(e1) / args.steps
            fms = time_calls(stf, torch, [xl], k, EPS, bopts, args.steps, args.warmup, stream, out_pair(torch, dev, k))
            batched_long[str(k)] = {"ms": round(bms, 4), "gelem_s": round((1 << 26) / bms / 1e6, 2),
                                    "flat_call_same_values_ms": round(fms, 4),
                                    "S_per_row": stf.solve(1 << 22, k, EPS / 16, options=bopts)["S"]}
        progress("batched long rows", batched_long)

    configs = bench_configs(stf, torch, dev, stream, args, opts, want, keep) if want & {"c1", "c2", "c3", "c5", "t7"} else None

    large = bench_large(stf, torch, dev, stream, args, opts) if "large" in want else None
    progress("large done")

    # device workspace each configuration holds (sized for it alone: the cache is
    # released first, so this is its need plus the library's 25% growth margin)
    workspace = {}
    for name, xd, k, eps, o in keep:
        stf.release()
        _, _, st = stf.topk(xd, k, eps=eps, seed=0, options=o, stats=True)
        workspace[name] = st["workspace_bytes"]
    stf.release()
    del keep, xds
    torch.cuda.synchronize()

    progress("workspace pass done")
    cpu = cpu_baseline(x0) if "cpu" in want and x0 is not None else None

    line = {
        "metric": "Gelem/s + % of HBM peak, exact top-k N=2^30 fp32, k=2^5..2^19, 1 GPU",
        "value": round(value, 2) if value else None,
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms, 4) if total_ms else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"Pareto(1.5) fp32 flat tensor N=2^{args.log2n} ({args.inputs} input tensors, seeds "
                               f"0..{args.inputs - 1}), exact top-k k sweep {list(KS)}, eps=1e-3",
                   "N": N, "ks": list(KS), "eps": EPS, "inputs": args.inputs, "s_rule": S_RULE_NAMES[args.s_rule],
                   "S": {str(k): stf.solve(N, k, EPS, options=opts)["S"] for k in KS}},
        "hbm_frac_alg": round(4.0 * N * len(KS) / (total_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4) if total_ms else None,
        "per_k": per_k,
        "per_k_cube_root_rule": other_rule,
        "retries": retries,
        "roofline": roofline,
        "read_ceiling": ceiling,
        "configs": configs,
        "batched": batched,
        "batched_long_rows": batched_long,
        "large": large,
        "workspace_bytes": workspace,
        "cpu_baseline": cpu,
        "host_gen_s": round(gen_s, 2),
        "inputs": {"generator": "numpy PCG64, workloads.generate / sae_pool, 2^24-value chunks on child seeds",
                   "numpy": np.__version__, "digest": "sha256 over the chunks' sha256 digests (2^24 values each)",
                   "sha256_16": INPUT_DIGESTS},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
