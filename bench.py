#!/usr/bin/env python3
"""Benchmark of the isotonic-regression hot path on one MI355X.

A step fits the two 10^7-element single rows the headline metric is quoted on,
one after the other on one stream: the noisy row (ramp 0..3 plus N(0,1) noise)
and the dense-hull row (strictly increasing, every point a hull vertex), f32 in
and out, unit weights, inputs resident in device memory.  Before every step an
untimed kernel reads and writes a 1 GiB buffer, so neither row is served from
the 256 MB Infinity Cache; each step is timed with HIP events on the fitting
stream.  ``value`` is elements fitted per second over the timed steps.

Also reported: per-row times, per-kernel durations (HIP events around each
launch, from the library's timing hook), the roofline of the dominant kernel,
the same steps without the cache flush, and the CPU oracle (f64 PAVA in C, one
thread) timed on a bounded sample of the same rows.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload row1e7]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "elements/s and % HBM roofline, 1e7 single row (dense & noisy), 1 MI355X"
HBM_PEAK_GBS = 8000.0

WORKLOADS = {
    # name: list of (label, inputs config name, rows, n)
    "row1e7": [("noisy", "c3_row1e7_noisy", None, None), ("dense", "c4_row1e7_dense", None, None)],
    "c1": [("c1", "c1_row4096_noisy", None, None)],
    "c2": [("c2", "c2_batch1024x1024_noisy", None, None)],
    "c5": [("c5", "c5_calib256x2p20", None, None)],
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="row1e7", choices=sorted(WORKLOADS))
    ap.add_argument("--copy-control", action="store_true",
                    help="merge long rows by copying vertices (the measurement control)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU oracle baseline (0 skips it)")
    ap.add_argument("--profile-only", action="store_true",
                    help="warm up and run the timed steps only (for rocprofv3)")
    return ap.parse_args()


def kernel_source_sha():
    h = hashlib.sha256()
    src = os.path.join(ROOT, "lower_convex_hull_amd", "csrc")
    for f in sorted(os.listdir(src)):
        with open(os.path.join(src, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str, sha: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 --pmc summary,
    or None when there is none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
    if kv.get("source_sha") != sha:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (rows shard across "
              "GPUs with no communication; see DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lower_convex_hull_amd import inputs, iso

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    iso.lib()
    flags = iso.ISO_F_NOCHECK | (iso.ISO_F_COPY_CONTROL if args.copy_control else 0)

    # ---- inputs (generated on the host, copied once; not timed)
    jobs = []
    host = {}
    for label, cfg, rows, n in WORKLOADS[args.workload]:
        y, w = inputs.config(cfg, rows=rows, n=n)
        host[label] = (y, w)
        yt = torch.from_numpy(y).to(dev)
        wt = None if w is None else torch.from_numpy(w).to(dev)
        R, N = yt.shape
        out = torch.empty_like(yt)
        ws = iso.workspace(R, N, wt is not None, flags, device=dev)
        jobs.append(dict(label=label, cfg=cfg, y=yt, w=wt, out=out, ws=ws, rows=R, n=N))
    stream = torch.cuda.Stream(device=dev)
    sh = iso._stream_handle(stream)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB

    def fit(j):
        st = iso.iso_fit_ex(j["y"].data_ptr(), None if j["w"] is None else j["w"].data_ptr(),
                            j["rows"], j["n"], j["out"].data_ptr(), None, j["ws"].data_ptr(),
                            j["ws"].numel(), sh, flags)
        if st < 0:
            raise iso.IsoError(st)

    def run_steps(k, flush_cache, per_job=False):
        """Times k steps with events on the fitting stream; returns (total ms, per-job ms)."""
        tot = 0.0
        pj = {j["label"]: 0.0 for j in jobs}
        for _ in range(k):
            if flush_cache:
                with torch.cuda.stream(stream):
                    flush.add_(1.0)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(jobs) + 1)]
            evs[0].record(stream)
            for i, j in enumerate(jobs):
                fit(j)
                if per_job:
                    evs[i + 1].record(stream)
            if not per_job:
                evs[-1].record(stream)
            stream.synchronize()
            tot += evs[0].elapsed_time(evs[-1])
            if per_job:
                for i, j in enumerate(jobs):
                    pj[j["label"]] += evs[i].elapsed_time(evs[i + 1])
        return tot, pj

    # ---- warm-up, including a busy second to raise the clocks
    for _ in range(max(args.warmup, 1)):
        for j in jobs:
            fit(j)
    with torch.cuda.stream(stream):
        for _ in range(20):
            flush.add_(1.0)
    stream.synchronize()

    if args.profile_only:
        run_steps(args.steps, True)
        torch.cuda.synchronize()
        print(json.dumps({"profile_only": True, "steps": args.steps}), flush=True)
        return

    # ---- the timed steps (cache flushed before each)
    torch.cuda.synchronize()
    ms_total, _ = run_steps(args.steps, True)
    ms_step = ms_total / args.steps
    elems = sum(j["rows"] * j["n"] for j in jobs)
    value = elems / (ms_step * 1e-3)

    # ---- per-row times and per-kernel durations (separate passes, same steps)
    _, per_job = run_steps(args.steps, True, per_job=True)
    iso.iso_timing_enable(True)
    run_steps(args.steps, True)
    phases = iso.iso_timing_read()
    # the same, one row at a time, for a per-row breakdown
    job_phases = {}
    for j in jobs:
        for _ in range(args.steps):
            with torch.cuda.stream(stream):
                flush.add_(1.0)
            fit(j)
        stream.synchronize()
        jp = iso.iso_timing_read()
        job_phases[j["label"]] = {k: round(v[0] / v[1], 5) for k, v in jp.items() if v[1] > 0}
    iso.iso_timing_enable(False)
    warm_total, _ = run_steps(args.steps, False)

    rows_rep = {}
    for j in jobs:
        t = per_job[j["label"]] / args.steps
        e = j["rows"] * j["n"]
        byt = e * (12 if j["w"] is not None else 8)
        rows_rep[j["label"]] = {
            "elements": e, "ms": round(t, 5), "elements_per_s": e / (t * 1e-3),
            "kernel_ms": job_phases[j["label"]],
            "compulsory_gb_s": byt / (t * 1e-3) / 1e9,
            "hbm_frac": byt / (t * 1e-3) / 1e9 / HBM_PEAK_GBS,
        }

    # ---- roofline of the dominant kernel
    per_elem_bytes = {"chunk_hulls": 4, "expand": 4, "short_rows": 8, "merge": 0, "merge_top": 0,
                      "copy_bridge": 0, "copy_move": 0, "chunk_redo": 0}
    weighted = any(j["w"] is not None for j in jobs)
    if weighted:
        per_elem_bytes.update(chunk_hulls=8, short_rows=12)
    live = {k: v for k, v in phases.items() if v[1] > 0}
    dom = max(live, key=lambda k: live[k][0])
    dom_ms = live[dom][0] / live[dom][1]
    launches_per_step = live[dom][1] / args.steps
    elems_per_launch = elems / launches_per_step
    alg = per_elem_bytes[dom] * elems_per_launch
    achieved = alg / (dom_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    traffic = committed_traffic(dom, args.workload, sha)
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic,
                "kernel": dom, "kernel_ms": round(dom_ms, 5),
                "algorithmic_bytes_per_launch": alg, "source_sha": sha}

    # ---- CPU oracle baseline (bounded sample of the same rows)
    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        done, t_cpu, k = 0, 0.0, 0
        labels = list(host)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds or k < len(labels):
            y, w = host[labels[k % len(labels)]]
            rows = min(y.shape[0], max(1, int(2e6 // y.shape[1])))
            a = time.perf_counter()
            oracle.fit_rows_f32(y[:rows], None if w is None else w[:rows])
            t_cpu += time.perf_counter() - a
            done += rows * y.shape[1]
            k += 1
        cpu = {"value": done / t_cpu, "unit": "elements/s", "cores": 1, "kind": "oracle",
               "sample": f"{k} oracle calls (f64 PAVA in C, f32 in/out, one thread) over "
                         f"{', '.join(labels)} rows of the same workload, {t_cpu:.1f} s"}

    rep = {
        "metric": METRIC, "value": value, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": {"row1e7": "row1e7_noisy+dense"}.get(args.workload, args.workload),
                   "rows": [f"{j['label']}:{j['rows']}x{j['n']}" for j in jobs],
                   "weights": "counts" if weighted else "unit", "io": "f32",
                   "merge": "copy_control" if args.copy_control else "segment_lists",
                   "cache": "1 GiB flush before each step (untimed)"},
        "hbm_frac_whole_call": (elems * (12 if weighted else 8)) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows_rep,
        "phases_ms_per_launch": {k: round(v[0] / v[1], 5) for k, v in live.items()},
        "phase_launches_per_step": {k: v[1] / args.steps for k, v in live.items()},
        "warm_ms_per_step": warm_total / args.steps,
    }
    print(json.dumps(rep), flush=True)


if __name__ == "__main__":
    main()
