"""Benchmark of the batched weighted isotonic fit on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload batch|cfg1|cfg3|cfg4|dense|all_vertices|soft_rank|calibration|fits|all]
                    [--no-cpu] [--copy-probe] [--cpu-seconds S]

A step is one whole fit (every kernel of the path) over one batch of
synthetic input already resident in HBM.  Every leg reports elements/s, the
fraction of HBM peak its algorithmic bytes reach, and the CPU oracle on the
host's cores on a bounded sample of the same input:

  batch (the headline line; `value` is its elements/s):
         1000 rows x 5000 float32, y ~ N(0,1), w ~ U(0.1, 1.1), non-increasing,
         clipped to [0, 1]; one launch of k_row_fit; both backward products
         are timed as well ("backward");
  cfg1:  1 row x 4096 float64, y ~ N(0,1), unit weights, increasing;
  cfg3:  4096 x 512 float32, y_i = s_i - i/512 (s sorted descending N(0,1)),
         unit weights, increasing: the fit with its blocks and the product in y
         of an N(0,1) upstream gradient, one step = both;
  cfg4:  1 row x 6.5e6 float64, calibration-shaped (sorted scores, counts as
         weights, rational labels), increasing, clipped to [0, 1]; both
         backward products timed as well (the three launches of long rows);
  dense: 32 rows x 2^22 float64, y_i = i/n with 1% of positions pushed down by
         |N(0, 0.01)|, w ~ U(0.5, 1.5), increasing (k_chunk_hull, k_merge_sub,
         k_merge_top, k_fixup); both backward products timed as well;
  all_vertices: 32 rows x 2^22 float64 increasing data (every point a hull
         vertex, the first page's Sec. 7.5 regime), w ~ U(0.1, 1.1);
  soft rank: 4096 x 512 float32 standard normal scores, forward and backward
         of the first page's Sec. 7.9 composition at eps = 1 and 1/n;
  calibration: one curve over 6.5e6 float64 scores (the first page's Sec. 7.7
         day), sort, pooling and fit, then 100001 queries.

Prints ONE JSON line.  Algorithmic bytes are y and w read once and the fit
written once (12 B/element for the batch, 16 for cfg1, 16 for cfg3's fit and
product, 24 for the float64 weighted rows); "% of HBM peak" divides them by
the measured time and 8 TB/s.  The roofline object times the batch's kernel
with HIP events on the stream it is launched on.  Its `traffic` is the HBM
bytes per launch that rocprofv3 counted (FETCH_SIZE and WRITE_SIZE, scaled
against a plain copy of known size), read from the committed summary under
profiles/ and reported only while the kernel sources are the ones that summary
was taken from.  The CPU baseline is the float64 oracle on the host cores, on
a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "fit elements/s and % of HBM peak, 1000×5000 f32 and 32×2^22 f64 dense"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "k_row_fit_1000x5000_f32.md")
DENSE_SUMMARY = os.path.join(ROOT, "profiles", "dense_32x4194304_f64.md")
CSRC = os.path.join(ROOT, "weighted_isotonic_regression_row_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed (a comment
    edit does not change the kernels the counters describe)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


# the sources k_row_fit and its launcher are built from
FIT_SOURCES = ("iso_device.hpp", "iso_fit.hip", "iso_internal.hpp", "iso_tile.hpp")


def source_hash() -> str:
    """Hash of the sources the batch kernel is built from, comments and
    whitespace aside (what its counters depend on)."""
    h = hashlib.sha256()
    for f in FIT_SOURCES:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(path=TRAFFIC_SUMMARY):
    """HBM bytes per fit call from a committed counter summary (the batch's one
    launch of k_row_fit, or the dense fit's four kernels summed), if it was
    taken from the current sources; else None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m_hash = re.search(r"source hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic bytes per launch:\s*([0-9]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash():
        return None
    return int(m_bytes.group(1))


def make_inputs(which):
    import workloads
    if which == "batch":
        return workloads.cfg2_batch_noise()
    if which == "cfg1":
        return workloads.cfg1_single_row()
    if which == "cfg3":
        return workloads.cfg3_soft_rank()
    if which == "cfg4":
        return workloads.cfg4_calibration()
    if which in ("packed48", "packed65", "packed512"):
        rows, n = {"packed48": (1_000_000, 48), "packed65": (1_000_000, 65), "packed512": (10_000, 512)}[which]
        wl = workloads.family("noise", rows, n, seed=65, dtype=np.float32, weights="uniform")
        wl.name = f"packed_{rows}x{n}_f32"
        return wl
    if which == "all_vertices":
        wl = workloads.family("increasing", 32, 1 << 22, seed=55, dtype=np.float64, weights="uniform")
        wl.name = "all_vertices_32x2^22_f64"
        return wl
    return workloads.cfg5_dense()


def host_cores() -> int:
    """Threads the oracle may use: the CPUs this process may run on (at most 16,
    a GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_gpu(wl, steps, warmup):
    """Returns (ms_per_step from the wall clock, mean and median per-step ms from
    a pair of HIP events around each call, ms per step from one pair of HIP
    events around the K timed calls), all events on the launch stream."""
    import torch
    import weighted_isotonic_regression_row_amd as iso
    dev = torch.device("cuda:0")
    y = torch.from_numpy(wl.y).to(dev)
    w = None if wl.w is None else torch.from_numpy(wl.w).to(dev)
    out = torch.empty_like(y)
    ws = iso.workspace(wl.rows, wl.n, y.dtype, dev)
    # one call with the status check (raises on bad weights)
    iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, out=out, ws=ws, blocks=False, check=True)
    for _ in range(warmup):
        iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, out=out, ws=ws, blocks=False, check=False)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the library launches on this stream
    # the K timed steps: plain fit calls between two synchronisations, with one
    # pair of HIP events around all of them (the launches back to back)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    r0.record(stream)
    for _ in range(steps):
        iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, out=out, ws=ws, blocks=False, check=False)
    r1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    region = r0.elapsed_time(r1) / steps
    # then K more with a pair of HIP events around each call (recording events
    # costs host time, so they stay out of the loop above)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(stream)
        iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, out=out, ws=ws, blocks=False, check=False)
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return (t1 - t0) * 1e3 / steps, float(np.mean(per)), float(np.median(per)), float(region)


def time_backward(wl, steps):
    """Event-timed products of the fit (inputs and blocks resident): grad_y
    alone, and grad_y with grad_w.  Returns a dict."""
    import torch
    import weighted_isotonic_regression_row_amd as iso
    dev = torch.device("cuda:0")
    y = torch.from_numpy(wl.y).to(dev)
    w = None if wl.w is None else torch.from_numpy(wl.w).to(dev)
    ws = iso.workspace(wl.rows, wl.n, y.dtype, dev)
    _, blocks = iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, ws=ws, blocks=True, check=True)
    g = torch.randn_like(y)
    gy = torch.empty_like(y)
    stream = torch.cuda.current_stream(dev)

    def run(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    ms_y = run(lambda: iso.iso_vjp(g, blocks, out=gy, ws=ws))
    ms_yw = run(lambda: iso.iso_vjp_yw(g, blocks, y, ws=ws))
    elems = wl.rows * wl.n
    es = wl.y.dtype.itemsize
    wb = 0 if wl.w is None else es
    by = elems * (2 * es + wb)          # g read, w read, grad_y written
    byw = elems * (4 * es + wb)         # g, y, w read, grad_y and grad_w written
    return {"vjp_ms": ms_y, "vjp_algorithmic_bytes": by, "vjp_hbm_frac": by / (ms_y * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "vjp_yw_ms": ms_yw, "vjp_yw_algorithmic_bytes": byw,
            "vjp_yw_hbm_frac": byw / (ms_yw * 1e-3) / 1e9 / HBM_PEAK_GBS}


def time_fit_and_vjp(wl, steps, warmup):
    """One step = the fit with its blocks and the product in y of the upstream
    gradient wl.g over them.  Returns (ms per step from the wall clock, mean
    event-timed ms of the fit call, of the product call)."""
    import torch
    import weighted_isotonic_regression_row_amd as iso
    dev = torch.device("cuda:0")
    y = torch.from_numpy(wl.y).to(dev)
    w = None if wl.w is None else torch.from_numpy(wl.w).to(dev)
    g = torch.from_numpy(wl.g).to(dev)
    out = torch.empty_like(y)
    gy = torch.empty_like(y)
    ws = iso.workspace(wl.rows, wl.n, y.dtype, dev)
    _, blocks = iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, out=out, ws=ws, check=True)

    def step():
        _, b = iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, out=out, ws=ws, check=False)
        iso.iso_vjp(g, b, out=gy, ws=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stream = torch.cuda.current_stream(dev)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    for k in range(steps):
        e[3 * k].record(stream)
        _, b = iso.iso_fit(y, w, wl.increasing, wl.y_min, wl.y_max, out=out, ws=ws, check=False)
        e[3 * k + 1].record(stream)
        iso.iso_vjp(g, b, out=gy, ws=ws)
        e[3 * k + 2].record(stream)
    torch.cuda.synchronize()
    fit_ms = float(np.mean([e[3 * k].elapsed_time(e[3 * k + 1]) for k in range(steps)]))
    vjp_ms = float(np.mean([e[3 * k + 1].elapsed_time(e[3 * k + 2]) for k in range(steps)]))
    return (t1 - t0) * 1e3 / steps, fit_ms, vjp_ms


FIT_LEGS = {
    # name: (description, bytes per element, steps cap, cpu rows cap)
    "cfg1": ("1 row x 4096 float64, y~N(0,1), unit weights, increasing, no clipping", 16, None, None),
    "cfg4": ("1 row x 6.5e6 float64, sorted N(0,1) scores, counts 1+Poisson(2) as weights, "
             "y = Binomial(count, sigmoid(1.5 s - 3))/count, increasing, clipped to [0,1]", 24, 20, None),
    "dense": ("32 rows x 2^22 float64, y_i = i/n with 1% pushed down by |N(0,0.01)|, w~U(0.5,1.5), increasing",
              24, 10, None),
    "all_vertices": ("32 rows x 2^22 float64, y_i = i/n (every point a hull vertex), w~U(0.1,1.1), increasing",
                     24, 10, None),
    # rows of 33 to 128 packed several to a wave (first page, Sec. 3.5); 512: one wave a row
    "packed48": ("10^6 rows x 48 float32, y~N(0,1), w~U(0.1,1.1), increasing", 12, 20, 200_000),
    "packed65": ("10^6 rows x 65 float32, y~N(0,1), w~U(0.1,1.1), increasing", 12, 20, 200_000),
    "packed512": ("10^4 rows x 512 float32, y~N(0,1), w~U(0.1,1.1), increasing", 12, None, None),
}


def fit_leg(name, steps, warmup, cpu_seconds, no_cpu, backward=False):
    """A fit leg: wall-clock ms per step, event-timed fit calls, elements/s,
    the fraction of HBM peak, and the oracle on the host on the same input;
    with `backward`, both products of the fit event-timed as well."""
    desc, bpe, cap, cpu_rows = FIT_LEGS[name]
    wl = make_inputs(name)
    log(f"{name}: {wl.name} {wl.y.shape}")
    k = steps if cap is None else max(1, min(steps, cap))
    ms, kmean, kmed, kreg = time_gpu(wl, k, min(warmup, 3) if cap else warmup)
    elems = wl.rows * wl.n
    algo = elems * bpe
    leg = {"workload": desc, "rows": wl.rows, "n": wl.n, "steps": k, "ms_per_step": ms,
           "fit_ms_events_mean": kmean, "fit_ms_events_median": kmed, "fit_ms_events_region": kreg,
           "elements_per_s": elems / (ms * 1e-3), "algorithmic_bytes": algo, "bytes_per_element": bpe,
           "hbm_frac_end_to_end": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "hbm_frac_events": algo / (kmean * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if backward:
        leg["backward"] = time_backward(wl, k)
    if not no_cpu:
        log(f"cpu baseline ({name}) ...")
        leg["cpu_baseline"] = cpu_baseline(wl, seconds=cpu_seconds, max_rows=cpu_rows)
    return leg


def time_soft_rank(steps, rows=4096, n=512):
    """Event-timed soft rank (first page, Sec. 7.9) of standard normal scores, forward and backward, at
    eps = 1 and eps = 1/n.  Algorithmic bytes: x read, ranks and the permutation written (12 B/element)
    forward; the gradient and the permutation read, the gradient in x written (12 B/element) backward."""
    import torch
    import weighted_isotonic_regression_row_amd as iso
    import workloads
    dev = torch.device("cuda:0")
    x, g = workloads.soft_rank_input(rows, n)
    x, g = torch.from_numpy(x).to(dev), torch.from_numpy(g).to(dev)
    ws = iso.soft_rank_workspace(rows, n, x.dtype, dev)
    r = torch.empty_like(x)
    d = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)

    def run(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    out = {"workload": f"{rows} rows x {n} float32, x~N(0,1), g~N(0,1)"}
    elems = rows * n
    for name, eps in (("eps_1", 1.0), ("eps_1_over_n", 1.0 / n)):
        _, st = iso.soft_rank(x, eps, out=r, ws=ws)
        fwd = run(lambda: iso.soft_rank(x, eps, out=r, ws=ws))
        bwd = run(lambda: iso.soft_rank_vjp(g, st, out=d, ws=ws))
        out[name] = {"forward_ms": fwd, "backward_ms": bwd, "elements_per_s_fwd_bwd": elems / ((fwd + bwd) * 1e-3),
                     "forward_hbm_frac": 12 * elems / (fwd * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "backward_hbm_frac": 12 * elems / (bwd * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def time_calibration(steps):
    """Event-timed calibration curve (first page, Sec. 7.7; PyPI usage) of 6.5 million float64 scores on a 1e-5
    grid with click labels: sort, pooling of equal scores, weighted fit; then 100001 queries on the curve.
    Algorithmic bytes: scores and labels read, distinct scores and the curve written (at most 32 B/element)."""
    import torch
    import weighted_isotonic_regression_row_amd as iso
    import workloads
    dev = torch.device("cuda:0")
    s, y, q = workloads.calibration_input()
    s, y, q = torch.from_numpy(s).to(dev), torch.from_numpy(y).to(dev), torch.from_numpy(q).to(dev)
    rows, n = s.shape
    ws = iso.calibration_workspace(rows, n, s.dtype, dev)
    xs, fit, m = iso.calibration_fit(s, y, ws=ws)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)

    def run(fn, k):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(k):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / k

    k = max(1, min(steps, 10))
    fit_ms = run(lambda: iso.calibration_fit(s, y, ws=ws), k)
    pred_ms = run(lambda: iso.calibrate(q, xs, fit, m, out=out), k)
    distinct = int(m[0].item())
    algo = n * 16 + distinct * 16
    return {"workload": "1 curve over 6.5e6 float64 scores (N(0,1) on a 1e-5 grid), Bernoulli(sigmoid(1.5 s - 3)) "
                        "labels; 100001 queries",
            "distinct_scores": distinct, "fit_ms": fit_ms, "scores_per_s": n / (fit_ms * 1e-3),
            "fit_hbm_frac": algo / (fit_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "predict_ms": pred_ms,
            "queries_per_s": q.numel() / (pred_ms * 1e-3)}


def copy_probe(nbytes=256 << 20, reps=20):
    """Device-to-device copy bandwidth of a plain copy of known size (read + write)."""
    import torch
    dev = torch.device("cuda:0")
    a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).uniform_()
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / reps
    return 2 * nbytes / (ms * 1e-3) / 1e9, nbytes


def cpu_baseline(wl, seconds=10.0, max_rows=None):
    """The oracle as it stands, timed on the host cores on a bounded sample (rows
    split over the threads; one row is sequential in pool adjacent violators)."""
    import oracle
    threads = host_cores()
    rows = wl.rows if max_rows is None else min(wl.rows, max_rows)
    threads = min(threads, rows)
    y = wl.y[:rows].astype(np.float64)
    w = None if wl.w is None else wl.w[:rows].astype(np.float64)
    elems = 0
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.fit(y, w, wl.increasing, wl.y_min, wl.y_max, threads=threads)
        elems += rows * wl.n
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": elems / dt, "unit": "elements/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{rows} of {wl.rows} rows x {wl.n}, float64 pool adjacent violators, "
                      f"{threads} threads, {reps} repetitions in {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=["batch", "cfg1", "cfg3", "cfg4", "dense", "all_vertices", "packed", "soft_rank",
                                           "calibration", "fits", "all", "both"], default="all")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg (profiling runs)")
    ap.add_argument("--copy-probe", action="store_true", help="time a plain device copy (also done by default runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time for the batch; the other legs take half of it")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only (--gpus 1); rows are independent and would "
                                   "shard across GPUs with no exchange"}), flush=True)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    import weighted_isotonic_regression_row_amd as iso
    iso.load_library()

    rec = {"metric": METRIC, "value": None, "unit": "elements/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f64", "data": "synthetic"}

    if args.workload in ("batch", "all", "both", "fits"):
        wl = make_inputs("batch")
        log(f"batch: {wl.name} {wl.y.shape}")
        ms, kmean, kmed, kreg = time_gpu(wl, args.steps, args.warmup)
        elems = wl.rows * wl.n
        algo = elems * (4 + 4 + 4)
        rec["value"] = elems / (ms * 1e-3)
        rec["ms_per_step"] = ms
        rec["config"] = {"workload": "1000 rows x 5000 float32, y~N(0,1), w~U(0.1,1.1), non-increasing, "
                                     "clipped to [0,1]",
                         "rows": wl.rows, "n": wl.n, "input_dtype": "f32", "accumulation": "f64",
                         "algorithmic_bytes": algo,
                         "hbm_frac_end_to_end": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        ach = algo / (kreg * 1e-3) / 1e9
        rec["roofline"] = {"bound": "hbm", "kernel": "k_row_fit<float,20>",
                           "timed": "the whole fit call (one launch of k_row_fit<float,20>): HIP events on the "
                                    "launch stream around the K timed calls, divided by K (kernel_ms_region); "
                                    "kernel_ms_mean and _median come from a pair of events around each call, "
                                    "which adds the events' own cost",
                           "achieved": ach,
                           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                           "traffic": committed_traffic(), "kernel_ms_region": kreg, "kernel_ms_mean": kmean,
                           "kernel_ms_median": kmed,
                           "bytes_per_element": 12, "elements_per_launch": elems,
                           "source_hash": source_hash()}
        rec["backward"] = time_backward(wl, args.steps)
        if not args.no_cpu:
            log("cpu baseline (batch) ...")
            rec["cpu_baseline"] = cpu_baseline(wl, seconds=args.cpu_seconds)
        del wl

    fits = ("fits", "all")
    if args.workload in ("cfg1",) + fits:
        rec["cfg1"] = fit_leg("cfg1", args.steps, args.warmup, args.cpu_seconds / 2, args.no_cpu)

    if args.workload in ("cfg3",) + fits:
        wl = make_inputs("cfg3")
        log(f"cfg3: {wl.name} {wl.y.shape}")
        ms, fit_ms, vjp_ms = time_fit_and_vjp(wl, args.steps, args.warmup)
        elems = wl.rows * wl.n
        algo = elems * 16  # y read, fit written; g read, grad_y written
        leg = {"workload": "4096 rows x 512 float32, y_i = s_i - i/512 (s sorted descending N(0,1)), unit weights, "
                           "increasing; the fit with its blocks and the product in y of an N(0,1) gradient",
               "rows": wl.rows, "n": wl.n, "steps": args.steps, "ms_per_step": ms,
               "fit_ms_events_mean": fit_ms, "vjp_ms_events_mean": vjp_ms,
               "elements_per_s": elems / (ms * 1e-3), "algorithmic_bytes": algo, "bytes_per_element": 16,
               "hbm_frac_end_to_end": algo / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               "hbm_frac_events": algo / ((fit_ms + vjp_ms) * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if not args.no_cpu:
            log("cpu baseline (cfg3, fit only) ...")
            leg["cpu_baseline"] = cpu_baseline(wl, seconds=args.cpu_seconds / 2)
            leg["cpu_baseline"]["sample"] += " (the fit; the oracle's product is not timed)"
        rec["cfg3"] = leg
        del wl

    if args.workload in ("cfg4",) + fits:
        rec["cfg4"] = fit_leg("cfg4", args.steps, args.warmup, args.cpu_seconds / 2, args.no_cpu, backward=True)

    if args.workload in ("dense", "both") + fits:
        dense = fit_leg("dense", args.steps, args.warmup, args.cpu_seconds / 2, args.no_cpu, backward=True)
        ach = dense["algorithmic_bytes"] / (dense["fit_ms_events_region"] * 1e-3) / 1e9
        dense["roofline"] = {"bound": "hbm", "timed": "the whole fit call (k_chunk_hull, k_chunk_cover, "
                                                      "k_merge_sub, k_merge_top, k_fixup): events on the launch "
                                                      "stream around the K timed calls, divided by K",
                             "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                             "traffic": committed_traffic(DENSE_SUMMARY), "bytes_per_element": 24,
                             "elements_per_launch": dense["rows"] * dense["n"]}
        rec["dense"] = dense
        if rec["value"] is None:
            rec["value"] = dense["elements_per_s"]
            rec["ms_per_step"] = dense["ms_per_step"]
            rec["config"] = {"workload": dense["workload"]}

    if args.workload in ("all_vertices",) + fits:
        rec["all_vertices"] = fit_leg("all_vertices", args.steps, args.warmup, args.cpu_seconds / 2, args.no_cpu)

    if args.workload in ("packed",) + fits:
        for name in ("packed48", "packed65", "packed512"):
            rec[name] = fit_leg(name, args.steps, args.warmup, args.cpu_seconds / 2, args.no_cpu)

    if args.workload in ("soft_rank", "all"):
        log("soft rank 4096 x 512 ...")
        rec["soft_rank"] = time_soft_rank(args.steps)
        # the long shapes of the first page's Table 6, sorted by tiles and merge passes
        log("soft rank 64 x 10^4 and 1 x 10^6 ...")
        rec["soft_rank_64x10000"] = time_soft_rank(max(2, args.steps // 5), 64, 10_000)
        rec["soft_rank_1x1000000"] = time_soft_rank(max(2, args.steps // 5), 1, 1_000_000)

    if args.workload in ("calibration", "all"):
        log("calibration 6.5e6 ...")
        rec["calibration"] = time_calibration(args.steps)

    if args.copy_probe or args.workload == "all":
        gbs, nb = copy_probe()
        rec["copy_probe"] = {"bytes_moved_per_copy": 2 * nb, "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS}

    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
