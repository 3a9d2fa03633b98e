#!/usr/bin/env python3
"""Benchmark of the isotonic-regression hot path on one MI355X.

A step fits the two 10^7-element single rows the headline metric is quoted on,
one after the other on one stream: the noisy row (ramp 0..3 plus N(0,1) noise)
and the dense-hull row (strictly increasing, every point a hull vertex), f32 in
and out, unit weights, inputs resident in device memory.  Before every step an
untimed kernel reads and writes a 1 GiB buffer, so neither row is served from
the 256 MB Infinity Cache; each step is timed with HIP events on the fitting
stream.  ``value`` is elements fitted per second over the timed steps.

Also reported on the same line:
  * step-time median and interquartile range, per-row times and HBM fractions,
    per-kernel durations (HIP events around each launch, the library's timing
    hook) and the roofline of the dominant kernel;
  * the copy ceiling: the library's plain streaming copy kernel on the same
    bytes;
  * the merge control: the same rows merged by copying vertices (the paper's
    grid-copy control) against segment lists, merge phase and whole call;
  * other workloads under "workloads": the short-row configurations (1x4096,
    1024x1024), the weighted calibration batch (256x2^20), 10^8-element rows,
    f64 input and output, the backward pass, and the calibration front end;
  * the CPU oracle (f64 PAVA in C, one thread) on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--no-extras]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "elements/s and % HBM roofline, 1e7 single row (dense & noisy), 1 MI355X"
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--copy-control", action="store_true",
                    help="headline rows merged by copying vertices (the measurement control)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU oracle baseline (0 skips it)")
    ap.add_argument("--no-extras", action="store_true",
                    help="headline only (no other workloads, ceiling or control)")
    ap.add_argument("--profile-only", action="store_true",
                    help="warm up and run the timed headline steps only (for rocprofv3)")
    ap.add_argument("--profile-workload", default="",
                    help="with --profile-only: time this extra workload instead of the headline")
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


def stats(ms):
    import numpy as np

    a = np.asarray(ms, np.float64)
    q1, med, q3 = np.percentile(a, [25, 50, 75])
    return {"mean": float(a.mean()), "median": float(med), "iqr": [float(q1), float(q3)], "n": len(a)}


class Bench:
    def __init__(self, torch, iso, dev, stream):
        self.torch = torch
        self.iso = iso
        self.dev = dev
        self.stream = stream
        self.sh = iso._stream_handle(stream)
        self.flush_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB

    def flush(self):
        with self.torch.cuda.stream(self.stream):
            self.flush_buf.add_(1.0)

    def timed(self, fns, k, flush=True):
        """k steps; each step runs every fn in order between two events on the
        fitting stream (a cache flush before each step, outside the events).
        Returns the per-step ms and the per-fn ms lists."""
        torch = self.torch
        steps, per = [], [[] for _ in fns]
        for _ in range(k):
            if flush:
                self.flush()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)]
            ev[0].record(self.stream)
            for i, f in enumerate(fns):
                f()
                ev[i + 1].record(self.stream)
            self.stream.synchronize()
            steps.append(ev[0].elapsed_time(ev[-1]))
            for i in range(len(fns)):
                per[i].append(ev[i].elapsed_time(ev[i + 1]))
        return steps, per

    def warm(self, fns, w):
        for _ in range(max(w, 1)):
            for f in fns:
                f()
        self.stream.synchronize()

    def phases(self, fns, k):
        """Per-launch ms and launches per call of each phase (timing hook)."""
        iso = self.iso
        iso.iso_timing_enable(True)
        try:
            for _ in range(k):
                self.flush()
                for f in fns:
                    f()
            self.stream.synchronize()
            ph = iso.iso_timing_read()
        finally:
            iso.iso_timing_enable(False)
        return {name: {"ms_per_launch": v[0] / v[1], "launches_per_step": v[1] / k}
                for name, v in ph.items() if v[1] > 0}


def fit_job(b, y, w, flags, f64=False):
    torch, iso = b.torch, b.iso
    R, N = y.shape
    out = torch.empty_like(y)
    ws = iso.workspace(R, N, w is not None, flags, device=b.dev)
    fn = iso.iso_fit_ex_f64 if f64 else iso.iso_fit_ex
    args = (y.data_ptr(), None if w is None else w.data_ptr(), R, N, out.data_ptr(), None, ws.data_ptr(),
            ws.numel(), b.sh, flags | iso.ISO_F_NOCHECK)

    def run():
        st = fn(*args)
        if st < 0:
            raise iso.IsoError(st)

    run.keep = (y, w, out, ws)
    return run


def workload_entry(name, elems, byts, steps, note, extra=None):
    s = stats(steps)
    t = s["median"] * 1e-3
    e = {"elements": elems, "ms_median": round(s["median"], 5),
         "ms_iqr": [round(v, 5) for v in s["iqr"]], "elements_per_s": elems / t,
         "compulsory_bytes": byts, "compulsory_gb_s": byts / t / 1e9,
         "hbm_frac": byts / t / 1e9 / HBM_PEAK_GBS, "note": note}
    if extra:
        e.update(extra)
    return e


def extras(b, args, np):
    """The other workloads, the copy ceiling and the merge control."""
    from lower_convex_hull_amd import inputs

    torch, iso = b.torch, b.iso
    K = max(5, args.steps)
    out = {}
    dev = b.dev

    def run_fit(label, y, w, note, f64=False, byt_per=None, flags=0):
        job = fit_job(b, y, w, flags, f64)
        b.warm([job], 2)
        steps, _ = b.timed([job], K)
        ph = b.phases([job], min(K, 10))
        R, N = y.shape
        es = y.element_size()
        per = byt_per if byt_per is not None else es * (3 if w is not None else 2)
        out[label] = workload_entry(label, R * N, R * N * per, steps, note,
                                    {"kernel_ms": {k: round(v["ms_per_launch"], 5) for k, v in ph.items()}})
        say(f"[bench] {label}: {out[label]['ms_median']:.4f} ms, hbm_frac {out[label]['hbm_frac']:.3f}")
        del job

    def dev_t(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # short rows and the calibration batch
    y, _ = inputs.config("c1_row4096_noisy")
    run_fit("c1_row4096_noisy", dev_t(y), None, "1 x 4096, f32, unit weights (launch-bound)")
    y, _ = inputs.config("c2_batch1024x1024_noisy")
    run_fit("c2_batch1024x1024_noisy", dev_t(y), None, "1024 x 1024, f32, unit weights")
    y, w = inputs.config("c5_calib256x2p20")
    yt, wt = dev_t(y), dev_t(w)
    run_fit("c5_calib256x2p20", yt, wt, "256 x 2^20, f32, integer-count weights")
    if args.cpu_seconds > 0:
        out["c5_calib256x2p20"]["cpu_oracle_all_cores"] = cpu_rows_all_cores(y, w, args.cpu_seconds)

    # backward pass on the calibration batch: d/dy and d/dw
    st, bid = None, torch.empty(yt.shape, dtype=torch.int32, device=dev)
    o = torch.empty_like(yt)
    ws = iso.workspace(yt.shape[0], yt.shape[1], True, 0, device=dev)
    st = iso.iso_fit_ex(yt.data_ptr(), wt.data_ptr(), yt.shape[0], yt.shape[1], o.data_ptr(), bid.data_ptr(),
                        ws.data_ptr(), ws.numel(), b.sh, 0)
    assert st == 0
    del ws, o
    g = torch.randn(yt.shape, dtype=torch.float32, device=dev)
    gy, gw = torch.empty_like(g), torch.empty_like(g)
    R, N = yt.shape
    nb = iso.iso_vjp_workspace_bytes(R, N)
    vws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)

    def vjp_c5():
        s_ = iso.iso_vjp(g.data_ptr(), yt.data_ptr(), wt.data_ptr(), bid.data_ptr(), R, N, gy.data_ptr(),
                         gw.data_ptr(), vws.data_ptr(), nb, b.sh)
        assert s_ == 0

    b.warm([vjp_c5], 2)
    steps, _ = b.timed([vjp_c5], K)
    out["vjp_c5_calib256x2p20"] = workload_entry("vjp_c5", R * N, R * N * 24, steps,
                                                 "d/dy and d/dw over the forward's blocks, weighted; "
                                                 "bytes: g, ids, w, y read, two gradients written")
    say(f"[bench] vjp c5: {out['vjp_c5_calib256x2p20']['ms_median']:.4f} ms")
    del g, gy, gw, vws, bid, yt, wt, y, w

    # 10^8-element rows (noisy; consecutive floats, every point a vertex)
    y, _ = inputs.noisy(1, 100_000_000, 8)
    run_fit("row1e8_noisy", dev_t(y), None, "1 x 1e8, f32, unit weights (merge beyond two stages)")
    y = inputs.consecutive_floats(100_000_000)[None, :]
    run_fit("row1e8_consecutive", dev_t(y), None, "1 x 1e8 consecutive floats, every point a vertex")
    del y

    # f64 input and output on the noisy 10^7 row
    y, _ = inputs.config("c3_row1e7_noisy")
    y64 = dev_t(y.astype(np.float64))
    run_fit("f64_row1e7_noisy", y64, None, "1 x 1e7, f64 in and out", f64=True)
    del y64

    # backward pass on the noisy 10^7 row, d/dy only, unit weights
    yt = dev_t(y)
    bid = torch.empty(yt.shape, dtype=torch.int32, device=dev)
    o = torch.empty_like(yt)
    ws = iso.workspace(1, yt.shape[1], False, 0, device=dev)
    assert iso.iso_fit_ex(yt.data_ptr(), None, 1, yt.shape[1], o.data_ptr(), bid.data_ptr(), ws.data_ptr(),
                          ws.numel(), b.sh, 0) == 0
    del ws, o
    g = torch.randn(yt.shape, dtype=torch.float32, device=dev)
    gy = torch.empty_like(g)
    N = yt.shape[1]
    nb = iso.iso_vjp_workspace_bytes(1, N)
    vws = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)

    def vjp_row():
        assert iso.iso_vjp(g.data_ptr(), None, None, bid.data_ptr(), 1, N, gy.data_ptr(), None, vws.data_ptr(),
                           nb, b.sh) == 0

    b.warm([vjp_row], 2)
    steps, _ = b.timed([vjp_row], K)
    out["vjp_row1e7_noisy"] = workload_entry("vjp_row1e7", N, N * 12, steps,
                                             "d/dy over the forward's blocks, unit weights; bytes: g and "
                                             "ids read, d/dy written")
    say(f"[bench] vjp row1e7: {out['vjp_row1e7_noisy']['ms_median']:.4f} ms")
    del g, gy, vws, bid, yt

    # calibration front end: one curve, and 280 segment curves
    for label, n, nseg in (("calib_curve_6p5e6", 6_500_000, 0), ("calib_curve_45p8e6", 45_800_000, 0),
                           ("calib_280_segments_6p5e6", 6_500_000, 280)):
        s, c, seg = inputs.click_scores(n, 90 + nseg, segments=nseg)
        st_, ct, gt = dev_t(s), dev_t(c), dev_t(seg)
        xp = torch.empty(n, dtype=torch.float64, device=dev)
        fp = torch.empty_like(xp)
        nb = iso.iso_calib_workspace_bytes(n)
        cws = torch.empty(nb, dtype=torch.uint8, device=dev)
        kk = ctypes.c_int64(0)

        def cal():
            assert iso.iso_calib_fit(st_.data_ptr(), ct.data_ptr(), None if gt is None else gt.data_ptr(), n,
                                     xp.data_ptr(), fp.data_ptr(), kk, cws.data_ptr(), nb, b.sh) == 0

        b.warm([cal], 1)
        steps, _ = b.timed([cal], max(5, K // 2))
        out[label] = workload_entry(label, n, n * 16, steps,
                                    "keys, sort, pooling of equal scores, fit, lift; f64 (one host wait "
                                    "for the number of distinct keys)", {"distinct_keys": kk.value})
        say(f"[bench] {label}: {out[label]['ms_median']:.4f} ms, {kk.value} distinct keys")
        del st_, ct, gt, xp, fp, cws
    torch.cuda.empty_cache()
    return out


STAMP_PHASES = {
    "chunk_hulls": ((0, 1, "loads, sums, scan"), (1, 5, "first quickhull level"), (5, 2, "later levels"),
                    (2, 4, "slot and window writes"), (0, 4, "whole workgroup")),
    "group_merge": ((0, 1, "prelude (window reads, starts)"), (1, 2, "merge tree"),
                    (1, 5, "tree level 0 (node 0)"), (5, 6, "tree level 1"), (6, 7, "tree level 2"),
                    (7, 8, "tree level 3"), (8, 9, "tree level 4"), (9, 10, "tree level 5"),
                    (2, 3, "group list and window"), (3, 4, "descriptors out"), (0, 4, "whole workgroup")),
    "top_merge": ((0, 1, "prelude (group windows, starts)"), (1, 2, "merge tree"),
                  (1, 5, "tree level 0 (node 0)"), (5, 6, "tree level 1"), (6, 7, "tree level 2"),
                  (7, 8, "tree level 3"), (8, 9, "tree level 4"), (9, 10, "tree level 5"),
                  (2, 3, "root list and prefix"), (3, 4, "chunk starts, first segments"),
                  (0, 4, "whole workgroup")),
    "expand": ((0, 1, "record"), (1, 4, "stores"), (0, 4, "whole workgroup")),
}


def phase_stamps(b, y, calls=5):
    """Per-phase durations inside the kernels of one long row (the library's
    phase stamps: a 100 MHz counter read by thread 0 of each workgroup)."""
    import numpy as np

    torch, iso = b.torch, b.iso
    R, N = y.shape
    flags = iso.ISO_F_PHASE_STAMPS
    nb0 = iso.iso_workspace_bytes(R, N, 0)
    nb = iso.iso_workspace_bytes(R, N, flags)
    m = -(-N // iso.iso_chunk_size(N))
    ng = -(-m // 64)
    ws = torch.empty(nb, dtype=torch.uint8, device=b.dev)
    out = torch.empty_like(y)
    acc = {}
    for _ in range(calls):
        b.flush()
        ws[nb0:].zero_()
        assert iso.iso_fit_ex(y.data_ptr(), None, R, N, out.data_ptr(), None, ws.data_ptr(), nb, b.sh,
                              flags | iso.ISO_F_NOCHECK) == 0
        b.stream.synchronize()
        st = ws[nb0:nb0 + (2 * R * m + R * ng + R) * 128].view(torch.int64).cpu().numpy().reshape(-1, 16)
        parts = {"chunk_hulls": st[:R * m], "group_merge": st[R * m:R * m + R * ng],
                 "top_merge": st[R * m + R * ng:R * m + R * ng + R],
                 "expand": st[R * m + R * ng + R:]}
        for kname, arr in parts.items():
            arr = arr[arr[:, 0] > 0]
            if not len(arr):
                continue
            d = acc.setdefault(kname, {"span_us": [], "wg": len(arr)})
            d["span_us"].append((arr[:, 4].max() - arr[:, 0].min()) / 100.0)
            for a, z, name in STAMP_PHASES[kname]:
                ok = (arr[:, a] > 0) & (arr[:, z] > 0)
                if ok.any():
                    d.setdefault(name, []).append(float(np.median(arr[ok, z] - arr[ok, a])) / 100.0)
    res = {}
    for kname, d in acc.items():
        res[kname] = {"workgroups": d["wg"], "launch_span_us": round(float(np.median(d["span_us"])), 2),
                      "median_per_workgroup_us": {k: round(float(np.median(v)), 2) for k, v in d.items()
                                                  if k not in ("span_us", "wg")}}
    return res


def cpu_rows_all_cores(y, w, seconds):
    """The oracle on the host cores, rows spread over a thread pool (the C
    oracle runs with the interpreter lock released), over a bounded sample of
    the batch's rows: elements per second and the threads used."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    rows = y.shape[0]
    t0 = time.perf_counter()
    oracle.fit_rows_f32(y[:1], None if w is None else w[:1])
    per_row = max(time.perf_counter() - t0, 1e-6)
    take = int(min(rows, max(cores, seconds * cores / per_row / 4)))
    take -= take % cores if take >= cores else 0

    def one(r):
        oracle.fit_rows_f32(y[r:r + 1], None if w is None else w[r:r + 1])

    t0 = time.perf_counter()
    with ThreadPoolExecutor(cores) as ex:
        list(ex.map(one, range(take)))
    t = time.perf_counter() - t0
    return {"value": take * y.shape[1] / t, "unit": "elements/s", "cores": cores, "kind": "oracle",
            "sample": f"{take} of the batch's {rows} rows, one row per task on {cores} threads, {t:.2f} s"}


def copy_ceiling(b, K):
    """The library's streaming copy kernel, cache flushed before each call."""
    torch, iso = b.torch, b.iso
    res = {}
    for label, nbytes in (("40MB", 40_000_000), ("1GiB", 1 << 30)):
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=b.dev)
        dst = torch.empty_like(src)

        def cp():
            assert iso.iso_copy_probe(src.data_ptr(), dst.data_ptr(), nbytes, b.sh) == 0

        b.warm([cp], 2)
        steps, _ = b.timed([cp], K)
        s = stats(steps)
        res[label] = {"bytes_moved": 2 * nbytes, "ms_median": round(s["median"], 5),
                      "gb_s": 2 * nbytes / (s["median"] * 1e-3) / 1e9}
        del src, dst
    return res


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (rows shard across "
              "GPUs with no communication). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lower_convex_hull_amd import inputs, iso

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    iso.lib()
    stream = torch.cuda.Stream(device=dev)
    b = Bench(torch, iso, dev, stream)
    flags = iso.ISO_F_COPY_CONTROL if args.copy_control else 0

    # ---- inputs of the headline (generated on the host, copied once; not timed)
    host = {}
    jobs = []
    for label, cfg in (("noisy", "c3_row1e7_noisy"), ("dense", "c4_row1e7_dense")):
        y, w = inputs.config(cfg)
        host[label] = (y, w)
        yt = torch.from_numpy(y).to(dev)
        job = fit_job(b, yt, None, flags)
        job.label = label
        jobs.append(job)
    elems = sum(j.keep[0].numel() for j in jobs)

    # ---- warm-up, including a busy stretch to raise the clocks
    b.warm(jobs, args.warmup)
    with torch.cuda.stream(stream):
        for _ in range(20):
            b.flush_buf.add_(1.0)
    stream.synchronize()

    if args.profile_only:
        b.timed(jobs, args.steps)
        torch.cuda.synchronize()
        print(json.dumps({"profile_only": True, "steps": args.steps}), flush=True)
        return

    # ---- the timed steps (cache flushed before each)
    torch.cuda.synchronize()
    steps, per = b.timed(jobs, args.steps)
    ms_total = sum(steps)
    ms_step = ms_total / args.steps
    value = elems / (ms_step * 1e-3)
    st = stats(steps)

    # ---- per-row times and per-kernel durations (separate passes, same steps)
    phases = b.phases(jobs, args.steps)
    rows_rep = {}
    for j, pj in zip(jobs, per):
        jp = b.phases([j], args.steps)
        s = stats(pj)
        t = s["median"] * 1e-3
        e = j.keep[0].numel()
        byt = 8 * e
        rows_rep[j.label] = {
            "elements": e, "ms_median": round(s["median"], 5), "ms_iqr": [round(v, 5) for v in s["iqr"]],
            "elements_per_s": e / t, "compulsory_gb_s": byt / t / 1e9, "hbm_frac": byt / t / 1e9 / HBM_PEAK_GBS,
            "kernel_ms": {k: round(v["ms_per_launch"], 5) for k, v in jp.items()},
            "kernel_hbm_frac": {k: round(a * e / (v["ms_per_launch"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 5)
                                for k, v in jp.items() for a in ([4] if k in ("chunk_hulls", "expand") else [])},
        }
    warm_steps, _ = b.timed(jobs, args.steps, flush=False)

    # ---- roofline of the dominant kernel (largest summed duration per step)
    per_elem_bytes = {"chunk_hulls": 4, "expand": 4, "short_rows": 8}
    dom = max(phases, key=lambda k: phases[k]["ms_per_launch"] * phases[k]["launches_per_step"])
    dom_ms = phases[dom]["ms_per_launch"]
    elems_per_launch = elems / phases[dom]["launches_per_step"]
    alg = per_elem_bytes.get(dom, 0) * elems_per_launch
    achieved = alg / (dom_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    traffic = committed_traffic(dom, "row1e7", sha)
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 5), "traffic": traffic, "kernel": dom,
                "kernel_ms": round(dom_ms, 5), "algorithmic_bytes_per_launch": alg, "source_sha": sha,
                "per_row_frac": {r: v["kernel_hbm_frac"].get(dom) for r, v in rows_rep.items()}}

    rep_extra = {}
    if not args.no_extras:
        # ---- copy ceiling and the merge control
        rep_extra["copy_ceiling"] = copy_ceiling(b, max(5, args.steps))
        ctl = {}
        for label, (y, _) in host.items():
            yt = torch.from_numpy(y).to(dev)
            seg_job = fit_job(b, yt, None, 0)
            cpy_job = fit_job(b, yt, None, iso.ISO_F_COPY_CONTROL)
            b.warm([seg_job, cpy_job], 2)
            s_seg, _ = b.timed([seg_job], max(5, args.steps // 2))
            s_cpy, _ = b.timed([cpy_job], max(5, args.steps // 2))
            p_seg = b.phases([seg_job], 5)
            p_cpy = b.phases([cpy_job], 5)
            merge = lambda p, ks: sum(p[k]["ms_per_launch"] * p[k]["launches_per_step"] for k in ks if k in p)
            ctl[label] = {
                "segment_lists": {"call_ms": round(stats(s_seg)["median"], 5),
                                  "merge_ms": round(merge(p_seg, ("merge", "merge_top")), 5)},
                "copy_control": {"call_ms": round(stats(s_cpy)["median"], 5),
                                 "merge_ms": round(merge(p_cpy, ("merge", "copy_bridge", "copy_move")), 5),
                                 "levels": p_cpy.get("copy_move", {}).get("launches_per_step")},
            }
            del seg_job, cpy_job, yt
        rep_extra["merge_control"] = ctl
        rep_extra["phase_stamps"] = {j.label: phase_stamps(b, j.keep[0]) for j in jobs}
        rep_extra["workloads"] = extras(b, args, np)

    # ---- CPU oracle baseline (bounded sample of the same rows)
    cpu = None
    if args.cpu_seconds > 0:
        import oracle

        done, t_cpu, k = 0, 0.0, 0
        labels = list(host)
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds or k < len(labels):
            y, w = host[labels[k % len(labels)]]
            a = time.perf_counter()
            oracle.fit_rows_f32(y, w)
            t_cpu += time.perf_counter() - a
            done += y.size
            k += 1
        cpu = {"value": done / t_cpu, "unit": "elements/s", "cores": 1, "kind": "oracle",
               "sample": f"{k} oracle calls (f64 PAVA in C, f32 in/out, one thread) over the noisy and "
                         f"dense 1e7 rows, {t_cpu:.1f} s; PAVA is sequential within a row, so one "
                         f"thread is also the all-core rate of a single row"}
        # the whole step's two rows at once, one per thread (the C oracle
        # releases the interpreter lock): the most cores this workload can use
        from concurrent.futures import ThreadPoolExecutor

        pair = [host[lb] for lb in labels]
        t0 = time.perf_counter()
        reps = 0
        with ThreadPoolExecutor(len(pair)) as ex:
            while reps == 0 or time.perf_counter() - t0 < args.cpu_seconds / 2:
                list(ex.map(lambda yw: oracle.fit_rows_f32(yw[0], yw[1]), pair))
                reps += 1
        t_all = time.perf_counter() - t0
        rep_extra["cpu_baseline_all_cores"] = {
            "value": reps * sum(y.size for y, _ in pair) / t_all, "unit": "elements/s", "cores": len(pair),
            "kind": "oracle",
            "sample": f"{reps} rounds of the step's {len(pair)} rows fitted concurrently, one row per "
                      f"thread, {t_all:.1f} s"}

    rep = {
        "metric": METRIC, "value": value, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
        "data": "synthetic",
        "config": {"workload": "row1e7_noisy+dense",
                   "rows": [f"{j.label}:1x{j.keep[0].numel()}" for j in jobs],
                   "weights": "unit", "io": "f32",
                   "merge": "copy_control" if args.copy_control else "segment_lists",
                   "cache": "1 GiB flush before each step (untimed)"},
        "step_ms_median": round(st["median"], 5), "step_ms_iqr": [round(v, 5) for v in st["iqr"]],
        "hbm_frac_whole_call": (elems * 8) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows_rep,
        "phases_ms_per_launch": {k: round(v["ms_per_launch"], 5) for k, v in phases.items()},
        "phase_launches_per_step": {k: v["launches_per_step"] for k, v in phases.items()},
        "warm_ms_per_step": sum(warm_steps) / args.steps,
    }
    rep.update(rep_extra)
    print(json.dumps(rep), flush=True)


if __name__ == "__main__":
    main()
