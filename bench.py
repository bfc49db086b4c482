"""Benchmark: exact Lloyd K-Means iterations on one MI355X.

Default run (what `python bench.py --gpus 1 --steps K --warmup W` prints): the
largest workload, c5 (bf16, N = 10^9 rows, D = 64, K = 4,096, 3 Lloyd
iterations per fit; X in host memory, streamed in 64 Mi-row chunks).  A step
is one Lloyd iteration over all 10^9 rows (every chunk uploaded, assigned and
reduced, then the means formed): the W warm-up and K timed iterations run as
consecutive fits of the workload's 3 iterations, each starting again from
C^0, so every iteration of the workload is timed in its proportion.  After
the headline, the device-resident workloads c2, c3 and c4 are timed the same
way (a step = one kmeans_fit of all their iterations on X already in HBM) and
reported under "extra_configs", each with its own FlashAssign roofline,
whole-update roofline and CPU baseline.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload c1..c5] [--extra c2,c3,c4|none] [--no-cpu-baseline]
  python bench.py --workload c1 --batch 256      (256 independent c1-shaped problems per call)
  python bench.py --ablation                     (the designs FlashAssign and Sort-Inverse Update replace)
  python bench.py --planner-study                (the static plan against every alternative, five shapes)
  python bench.py --segment-tile-study           (update time, short vs long segment tiles, N = 2^13..2^22)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {  # MI355X published dense peaks
    "bf16": 2.5e15, "f16": 2.5e15, "f32": 157.3e12,  # matrix FLOP/s
    "hbm": 8.0e12,                                   # bytes/s
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


ASSIGN_SOURCES = [os.path.join(ROOT, "means_clustering_amd", "csrc", f) for f in ("flash_assign.hip", "km_internal.hpp")]


def _src_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_srcs, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the kernel is unchanged since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        r = rec[workload]
        if r["source_sha"] != _src_hash(kernel_srcs):
            return None
        return r["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def measured_peaks(dev, dtype):
    """Same-run peaks: sustained MFMA rate (random operands), device copy, pinned host-to-device copy."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "means_clustering_amd", "libkm_peaks.so"))
    lib.km_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double)]
    lib.km_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_double)]
    lib.km_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_double)]
    lib.km_peak_lds.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double)]
    out = {}
    blocks = 512  # two workgroups (two wavefronts per SIMD) per CU
    scratch = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    tf = ctypes.c_double()
    if dtype in ("bf16", "f16"):
        rc = lib.km_peak_mfma(1 if dtype == "bf16" else 0, blocks, 20000, ctypes.c_void_p(scratch.data_ptr()),
                              ctypes.byref(tf))
        if rc == 0:
            out["mfma_TFLOPs"] = round(tf.value, 1)
    nbytes = 1 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    gb = ctypes.c_double()
    if lib.km_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, 5,
                        ctypes.byref(gb)) == 0:
        out["hbm_copy_GBps"] = round(gb.value, 1)
    rs = torch.empty(256 * 4096, dtype=torch.int32, device=dev)
    if lib.km_peak_read(ctypes.c_void_p(src.data_ptr()), nbytes, 5, ctypes.c_void_p(rs.data_ptr()),
                        ctypes.byref(gb)) == 0:
        out["hbm_read_GBps"] = round(gb.value, 1)
    del src, dst, rs
    # LDS reads per compute unit (FlashAssign at D = 64 issues one 1 KiB LDS read per MFMA)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    lds_scratch = torch.empty(2 * cus * (4 * 8 + 256 * 16), dtype=torch.uint8, device=dev)
    bpc, tb = ctypes.c_double(), ctypes.c_double()
    if lib.km_peak_lds(40000, ctypes.c_void_p(lds_scratch.data_ptr()), lds_scratch.numel(), ctypes.byref(bpc),
                       ctypes.byref(tb)) == 0:
        out["lds_read_bytes_per_clock_per_cu"] = round(bpc.value, 1)
        out["lds_read_TBps"] = round(tb.value, 1)
    del lds_scratch
    # pinned host -> device: 1 GiB copies after two untimed ones (first-touch and mapping costs), best of 5
    h = torch.ones(1 << 30, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    for _ in range(2):
        d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        d.copy_(h, non_blocking=True)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    out["h2d_pinned_GBps"] = round(best, 1)
    del h, d
    return out


def cpu_baseline(w, C0, rows_of, budget_s=10.0):
    """The oracle (never tuned) on a bounded sample of the same workload, scaled to the full N.

    ``rows_of(r)`` returns the first r rows of X as stored.  A first run on a
    small sample calibrates the rate; the measured run then takes enough
    leading rows for about ``budget_s`` seconds of one Lloyd iteration.
    """
    import oracle

    def timed(rows, iters=1):
        Xs = rows_of(rows)
        t0 = time.perf_counter()
        oracle.fit(Xs, C0, iters, contract=True, xdtype=w.dtype)
        return time.perf_counter() - t0

    rows = max(256, min(w.N, w.N // 256, 1 << 20))
    dt = timed(rows)
    rows = int(min(w.N, max(rows, rows * budget_s / max(dt, 1e-3))))
    dt = timed(rows)
    iters = 1
    if rows == w.N and dt < 0.5 * budget_s:  # the whole workload is cheap: time several iterations
        iters = max(2, min(10000, int(budget_s / max(dt, 1e-4))))
        dt = timed(rows, iters)
    sec_per_iter_full = dt / iters * (w.N / rows)
    what = (f"all {w.N} points, {iters} Lloyd iterations" if rows == w.N
            else f"first {rows} of {w.N} points, 1 Lloyd iteration")
    return {"value": round(1.0 / sec_per_iter_full, 6), "unit": "iterations/s", "cores": oracle.num_threads(),
            "kind": "oracle", "sample": f"{what} (assign + update) in {dt:.1f} s"
                                         + ("" if rows == w.N else "; time scaled linearly to all points"),
            "distances_per_s": round(w.K * w.N / sec_per_iter_full, 1)}


def ablation(dev):
    """The designs Flash-KMeans replaces, timed next to the library's kernels on the same inputs."""
    import numpy as np
    import torch

    import means_clustering_amd as km
    import synth
    from means_clustering_amd import ablation as abl

    def timeit(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3  # us

    out = {"ablation": "designs replaced by FlashAssign and Sort-Inverse Update, same GPU, same inputs"}
    for name, rows in (("c2", None), ("c4", 1 << 21)):
        w = synth.WORKLOADS[name]
        n = w.N if rows is None else rows
        Xn = synth.points(w, 0, n)
        C = torch.from_numpy(synth.init_centroids(w.scaled(N=n), Xn)).to(dev)
        X = torch.from_numpy(Xn.view(np.int16)).view(torch.bfloat16).to(dev)
        del Xn
        print(f"[bench] ablation assign {name} N={n}", file=sys.stderr, flush=True)
        ws = km.Workspace(dev)
        a_out = torch.empty(n, dtype=torch.int32, device=dev)
        scratch = torch.empty(abl.lib().kmeans_abl_materialized_bytes(n, w.D, w.K), dtype=torch.uint8, device=dev)
        t_fa = timeit(lambda: km.assign(X, C, out=a_out, ws=ws), 5)
        t_mat = timeit(lambda: abl.assign_materialized(X, C, scratch), 3)
        same = torch.equal(a_out, abl.assign_materialized(X, C, scratch))
        out[f"assign_{name}"] = {"N": n, "D": w.D, "K": w.K, "flash_assign_us": round(t_fa, 1),
                                 "materialized_us": round(t_mat, 1), "speedup": round(t_mat / t_fa, 2),
                                 "score_matrix_bytes": n * w.K * 4, "same_assignment": bool(same)}
        del scratch, X
        torch.cuda.empty_cache()
    w = synth.WORKLOADS["c4"]
    Xn = synth.points(w)
    C = torch.from_numpy(synth.init_centroids(w, Xn)).to(dev)
    X = torch.from_numpy(Xn.view(np.int16)).view(torch.bfloat16).to(dev)
    del Xn
    a_real, _ = km.assign(X, C)
    rng = np.random.default_rng(11)
    zw = 1.0 / np.arange(1, w.K + 1) ** 1.2
    cases = {"c4_assignments": a_real,
             "zipf_ids": torch.from_numpy(rng.choice(w.K, size=w.N, p=zw / zw.sum()).astype(np.int32)).to(dev),
             "one_cluster": torch.zeros(w.N, dtype=torch.int32, device=dev)}
    ws = km.Workspace(dev)
    C_out = torch.empty_like(C)
    cnt = torch.empty(w.K, dtype=torch.int32, device=dev)
    scratch = torch.empty(abl.lib().kmeans_abl_atomic_bytes(w.D, w.K), dtype=torch.uint8, device=dev)
    bmin = w.N * w.D * 2 + w.N * 4 + w.K * w.D * 4
    for cname, a in cases.items():
        print(f"[bench] ablation update {cname}", file=sys.stderr, flush=True)
        t_si = timeit(lambda: km.update(X, a, C, out=C_out, counts_out=cnt, ws=ws), 5)
        t_at = timeit(lambda: abl.update_atomic(X, a, C, scratch), 3)
        out[f"update_{cname}"] = {"N": w.N, "D": w.D, "K": w.K, "sort_inverse_us": round(t_si, 1),
                                  "atomic_scatter_us": round(t_at, 1), "speedup": round(t_at / t_si, 2),
                                  "sort_inverse_GBps_Bmin": round(bmin / (t_si * 1e-6) / 1e9, 1),
                                  "atomic_GBps_Bmin": round(bmin / (t_at * 1e-6) / 1e9, 1)}
    print(json.dumps(out), flush=True)



# Timed steps when --steps is not given (the driver always gives them).
DEFAULT_STEPS = {"c1": 200, "c2": 10, "c5": 6}
EXTRA_DEFAULT = "c2,c3,c4"
UPDATE_PHASES = ("sort", "segments", "reduce", "finalize")


def timed_step(i: int, steps: int) -> bool:
    """Whether timed step i carries the FlashAssign events.  A timing event costs a
    marker packet and a few microseconds of host time per launch, which is ~12%
    of a c1 iteration, so with many steps only every s-th step is bracketed
    (s = ceil(steps / 8)); the launches of those steps give the average."""
    return i % -(-steps // 8) == 0


def read_phases(km):
    out = {}
    for ph in km.PHASES:
        ms, n = km.timing_read(ph)
        if n:
            out[ph] = {"total_ms": round(ms, 4), "launches": n, "avg_us": round(1e3 * ms / n, 3)}
    km.timing_reset()
    return out


def assign_roofline(w, phases, total_iters, peaks):
    """FlashAssign: algorithmic flops 2*N*K*D per iteration over the launches' average duration."""
    if "assign" not in phases:
        return None
    n = phases["assign"]["launches"]
    flops = 2.0 * w.N * w.K * w.D * total_iters / n  # per launch (streamed: chunks differ, ragged last one)
    avg_s = phases["assign"]["avg_us"] * 1e-6
    achieved = flops / avg_s
    peak = PEAK[w.dtype]
    roof = {"bound": "mfma", "kernel": "flash_assign", "achieved": round(achieved / 1e12, 2),
            "peak": round(peak / 1e12, 1), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": _traffic(ASSIGN_SOURCES, w.name), "flops_per_launch": flops,
            "avg_launch_us": phases["assign"]["avg_us"], "timed_launches": n}
    if peaks and "mfma_TFLOPs" in peaks and w.dtype != "f32":
        roof["peak_measured"] = peaks["mfma_TFLOPs"]
        roof["frac_of_measured"] = round(roof["achieved"] / peaks["mfma_TFLOPs"], 4)
    return roof


def update_roofline(w, breakdown, iters, peaks):
    """The whole Sort-Inverse Update (argsort + boundaries + segmented reduction + fix-up/finalise) of one
    iteration against HBM, on the algorithmic minimum B_min = N*D*s + 4N + 4KD (read X and the assignment
    once, write the centroids), from the per-phase step; the segmented-reduction kernel alone is given
    separately (its own bytes: the gathered rows plus 8 B of sorted key and index per point)."""
    if not any(p in breakdown for p in UPDATE_PHASES):
        return None
    es = 4 if w.dtype == "f32" else 2
    bmin = w.N * w.D * es + 4 * w.N + 4 * w.K * w.D
    t_iter = sum(breakdown[p]["total_ms"] for p in UPDATE_PHASES if p in breakdown) * 1e-3 / iters
    gbps = bmin / t_iter / 1e9
    out = {"bound": "hbm", "kernel": "whole update: " + " + ".join(p for p in UPDATE_PHASES if p in breakdown),
           "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(gbps / 8000.0, 4),
           "bytes_min_per_iteration": bmin, "us_per_iteration": round(t_iter * 1e6, 2),
           "phase_us_per_iteration": {p: round(breakdown[p]["total_ms"] * 1e3 / iters, 2)
                                      for p in UPDATE_PHASES if p in breakdown}}
    if peaks and "hbm_read_GBps" in peaks:
        out["peak_measured_read"] = peaks["hbm_read_GBps"]
        out["frac_of_measured_read"] = round(gbps / peaks["hbm_read_GBps"], 4)
    if "reduce" in breakdown:
        small = w.K <= 64
        per_point = w.D * es + (4 if small else 8)
        per_launch = w.N * per_point * iters / breakdown["reduce"]["launches"]
        kg = per_launch / (breakdown["reduce"]["avg_us"] * 1e-6) / 1e9
        out["reduce_kernel"] = {"kernel": "small_update" if small else "segment_reduce",
                                "bytes_per_launch": round(per_launch), "avg_launch_us": breakdown["reduce"]["avg_us"],
                                "achieved": round(kg, 1), "frac": round(kg / 8000.0, 4)}
    return out


def run_resident(w, args, dev, peaks, steps, warmup, tag):
    """One workload with X resident in HBM: a step is one kmeans_fit of all its iterations."""
    import numpy as np
    import torch

    import means_clustering_amd as km
    import synth

    print(f"[bench] {tag} {w.name}: {w.description}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    Xn = synth.points(w)
    C0 = torch.from_numpy(synth.init_centroids(w, Xn)).to(dev)
    X = (torch.from_numpy(Xn.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16"
         else torch.from_numpy(Xn)).to(dev)
    print(f"[bench] {w.name}: inputs in HBM after {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    C = C0.clone()
    a = torch.empty(w.N, dtype=torch.int32, device=dev)
    counts = torch.empty(w.K, dtype=torch.int32, device=dev)
    ws = km.Workspace(dev)

    def one_step():
        C.copy_(C0)
        km.fit(X, C, w.iters, inplace=True, ws=ws, assign_out=a, counts_out=counts)

    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    timing = not args.no_timing
    if timing:
        km.timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if timing:
            km.timing_enable(2 if timed_step(i, steps) else 0)
        one_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    phases, breakdown = {}, {}
    if timing:
        km.timing_enable(False)
        phases = read_phases(km)
        # per-phase breakdown from one more step with every phase timed (not part of `value`)
        km.timing_enable(1)
        one_step()
        torch.cuda.synchronize()
        km.timing_enable(False)
        breakdown = read_phases(km)
    timed_steps = sum(timed_step(i, steps) for i in range(steps))
    roof = assign_roofline(w, phases, timed_steps * w.iters, peaks)
    if roof is not None:
        roof["timed_steps"] = timed_steps
    res = {"value": round(steps * w.iters / elapsed, 3), "unit": "iterations/s", "steps": steps, "warmup": warmup,
           "step": f"one kmeans_fit of all {w.iters} iterations from C^0, X resident in HBM",
           "ms_per_step": round(1e3 * elapsed / steps, 3), "dtype": w.dtype,
           "config": {"workload": w.description, "name": w.name, "N": w.N, "D": w.D, "K": w.K,
                      "iters_per_step": w.iters},
           "distances_per_s": round(steps * w.iters / elapsed * w.N * w.K, 1),
           "roofline": roof, "update_roofline": update_roofline(w, breakdown, w.iters, peaks),
           "phases_timed_region": phases, "phase_breakdown_extra_step": breakdown}
    del X
    torch.cuda.empty_cache()
    res["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        print(f"[bench] {w.name}: cpu baseline (the oracle on a sample)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, C0.cpu().numpy(), lambda r: Xn[:r], budget_s=args.cpu_budget)
    return res


def resident_copy_fit(w, dev, Xh, C0, stage, copy_stream):
    """Not part of `value`: the same streamed fit with a device copy of X in the workspace (X fits in one GPU's
    HBM), so only the first iteration crosses the host link.  Times one fit of 1 and one of the workload's
    iteration count; the difference gives the cost of an iteration that reads X from HBM."""
    import torch

    import means_clustering_amd as km

    torch.cuda.empty_cache()
    need = km.workspace_bytes(km.KM_OP_FIT_STREAMED_RESIDENT, w.N, w.D, w.K, Xh.dtype, w.chunk_rows)
    free, _ = torch.cuda.mem_get_info(dev)
    if need + (4 << 30) > free:
        return {"skipped": f"needs {need / 2**30:.1f} GiB of workspace, {free / 2**30:.1f} GiB free"}
    rws = km.Workspace(dev)
    times = {}
    for it in (1, w.iters):
        print(f"[bench] {w.name} with a resident copy of X: fit of {it} iteration(s)", file=sys.stderr, flush=True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        km.fit_streamed(Xh, C0, it, w.chunk_rows, copy_stream=copy_stream, want_assign=False, ws=rws, stage=stage,
                        resident=True)
        torch.cuda.synchronize()
        times[it] = time.perf_counter() - t1
    later = (times[w.iters] - times[1]) / max(w.iters - 1, 1)
    del rws
    torch.cuda.empty_cache()
    return {"what": "kmeans_fit_streamed with a device copy of all of X in the workspace: X crosses the host link "
                    "in the first iteration only (same results bit for bit)",
            "workspace_GB": round(need / 1e9, 2), "fit_iterations": w.iters,
            "fit_s": round(times[w.iters], 3), "fit_iterations_per_s": round(w.iters / times[w.iters], 4),
            "first_iteration_s": round(times[1], 3), "later_iteration_s": round(later, 4),
            "later_iterations_per_s": round(1.0 / later, 3) if later > 0 else None}


def run_streamed(w, args, dev, peaks, steps, warmup):
    """The out-of-core workload: X in host memory, a step is one Lloyd iteration over every chunk."""
    import torch

    import means_clustering_amd as km
    import synth

    print(f"[bench] workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    t0 = time.perf_counter()

    def progress(done):
        if done % (1 << 28) < (1 << 24) or done == w.N:
            print(f"[bench] generated {done} / {w.N} rows", file=sys.stderr, flush=True)

    # pageable: 10^9 x 64 bf16 is more than the host lets one process pin; uploaded through a staging ring
    Xh = synth.host_points(w, dev, pinned=False, progress=progress)
    stage = km.staging_buffer()
    Xrows = synth.as_numpy_rows(Xh)
    C0 = torch.from_numpy(synth.init_centroids(w, Xrows)).to(dev)
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)
    ws = km.Workspace(dev)
    copy_stream = torch.cuda.Stream(dev)

    def run_iterations(n, label):
        """n Lloyd iterations as consecutive fits of the workload's iteration count, each from C^0."""
        done = 0
        while done < n:
            it = min(w.iters, n - done)
            km.fit_streamed(Xh, C0, it, w.chunk_rows, copy_stream=copy_stream, want_assign=False, ws=ws, stage=stage)
            torch.cuda.synchronize()
            done += it
            print(f"[bench] {label}: {done} / {n} iterations", file=sys.stderr, flush=True)

    run_iterations(warmup, "warm-up")
    timing = not args.no_timing
    if timing:
        km.timing_reset()
        km.timing_enable(2)  # FlashAssign launches only: two events per 64 Mi-row chunk
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_iterations(steps, "timed")
    elapsed = time.perf_counter() - t0
    phases, breakdown = {}, {}
    if timing:
        km.timing_enable(False)
        phases = read_phases(km)
        km.timing_enable(1)
        run_iterations(w.iters, "per-phase step")
        km.timing_enable(False)
        breakdown = read_phases(km)
    resident = None
    if not args.no_resident:
        del ws  # the streamed run's workspace goes back to the allocator first
        resident = resident_copy_fit(w, dev, Xh, C0, stage, copy_stream)
    es = 2 if w.dtype == "bf16" else 4
    e2e = w.N * w.D * es * steps / elapsed / 1e9
    stream = {"h2d_bytes_per_iteration": w.N * w.D * es, "end_to_end_GBps": round(e2e, 2),
              "peak": 64.0, "unit": "GB/s", "frac_of_pcie5_x16": round(e2e / 64.0, 4)}
    if "h2d" in breakdown:  # each chunk's upload bracketed on the copy stream
        stream["h2d_GBps_while_copying"] = round(w.N * w.D * es * w.iters / (breakdown["h2d"]["total_ms"] * 1e-3) / 1e9,
                                                 2)
    if peaks and "h2d_pinned_GBps" in peaks:
        stream["peak_measured_h2d"] = peaks["h2d_pinned_GBps"]
        stream["frac_of_measured_h2d"] = round(e2e / peaks["h2d_pinned_GBps"], 4)
    res = {"value": round(steps / elapsed, 4), "unit": "iterations/s", "steps": steps, "warmup": warmup,
           "step": (f"one Lloyd iteration over all {w.N} rows (upload, FlashAssign, Sort-Inverse Update of every "
                    f"{w.chunk_rows}-row chunk, then the means); steps run as consecutive {w.iters}-iteration fits "
                    "from C^0"),
           "ms_per_step": round(1e3 * elapsed / steps, 3), "dtype": w.dtype,
           "config": {"workload": w.description, "name": w.name, "N": w.N, "D": w.D, "K": w.K,
                      "iters_per_fit": w.iters, "chunk_rows": w.chunk_rows},
           "distances_per_s": round(steps / elapsed * w.N * w.K, 1),
           "roofline": assign_roofline(w, phases, steps, peaks),
           "update_roofline": update_roofline(w, breakdown, w.iters, peaks), "streaming": stream,
           "phases_timed_region": phases, "phase_breakdown_extra_step": breakdown, "resident_copy": resident}
    res["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        print(f"[bench] {w.name}: cpu baseline (the oracle on a sample)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, C0.cpu().numpy(), lambda r: Xrows[:r], budget_s=args.cpu_budget)
    del Xh, Xrows, stage
    return res


def batched(args, dev):
    """B independent problems of one workload's shape per call (kmeans_fit_batched); one JSON line.

    Problem b draws its own mixture and points with seed (workload seed + 1000 b), so problem 0 is the
    workload itself.  ``value`` is Lloyd iterations per second summed over the batch.
    """
    import numpy as np
    import torch

    import means_clustering_amd as km
    import synth

    base = synth.WORKLOADS[args.workload]
    if base.chunk_rows:
        raise SystemExit("--batch applies to device-resident workloads")
    B = args.batch
    print(f"[bench] batch of {B} x {base.name}: {base.description}", file=sys.stderr, flush=True)
    Xs, Cs = [], []
    for b in range(B):
        w = base.scaled(seed=base.seed + 1000 * b)
        Xn = synth.points(w)
        Cs.append(synth.init_centroids(w, Xn))
        Xs.append(Xn)
    Xn = np.stack(Xs)
    del Xs
    X = (torch.from_numpy(Xn.view(np.int16)).view(torch.bfloat16) if base.dtype == "bf16"
         else torch.from_numpy(Xn)).to(dev)
    C0 = torch.from_numpy(np.stack(Cs)).to(dev)
    C = C0.clone()
    a = torch.empty((B, base.N), dtype=torch.int32, device=dev)
    counts = torch.empty((B, base.K), dtype=torch.int32, device=dev)
    ws = km.Workspace(dev)

    def one_step():
        C.copy_(C0)
        km.fit_batched(X, C, base.iters, inplace=True, ws=ws, assign_out=a, counts_out=counts)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i} done", file=sys.stderr, flush=True)
    timing = not args.no_timing
    if timing:
        km.timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if timing:
            km.timing_enable(2 if timed_step(i, args.steps) else 0)
        one_step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if timing:
        km.timing_enable(False)
    value = args.steps * base.iters * B / elapsed
    roof, breakdown = None, {}
    if timing:
        ms, n = km.timing_read("assign")
        km.timing_reset()
        if n:
            flops = 2.0 * B * base.N * base.K * base.D
            avg_s = ms * 1e-3 / n
            peak = PEAK[base.dtype]
            roof = {"bound": "mfma", "kernel": "flash_assign (batched)", "achieved": round(flops / avg_s / 1e12, 2),
                    "peak": round(peak / 1e12, 1), "unit": "TFLOP/s", "frac": round(flops / avg_s / peak, 4),
                    "traffic": None, "flops_per_launch": flops, "avg_launch_us": round(avg_s * 1e6, 3),
                    "timed_launches": n, "timed_steps": sum(timed_step(i, args.steps) for i in range(args.steps))}
        km.timing_enable(1)
        one_step()
        torch.cuda.synchronize()
        km.timing_enable(False)
        for ph in km.PHASES:
            ms, n = km.timing_read(ph)
            if n:
                breakdown[ph] = {"total_ms": round(ms, 4), "launches": n, "avg_us": round(1e3 * ms / n, 3)}
        km.timing_reset()
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: timing the oracle on problem 0", file=sys.stderr, flush=True)
        cpu = cpu_baseline(base, Cs[0], lambda r: Xn[0][:r], budget_s=args.cpu_budget)
        cpu["sample"] += " (one problem of the batch; iterations/s of one problem)"
    line = {
        "metric": "Lloyd iterations/sec and point-centroid distances/sec (fused assign+update)",
        "value": round(value, 3), "unit": "iterations/s (summed over the batch)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(1e3 * elapsed / args.steps, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": base.dtype, "data": "synthetic",
        "config": {"workload": f"{B} independent problems of {base.description}", "name": base.name, "batch": B,
                   "N": base.N, "D": base.D, "K": base.K, "iters_per_step": base.iters},
        "distances_per_s": round(value * base.N * base.K, 1),
        "roofline": roof, "cpu_baseline": cpu, "phase_breakdown_extra_step": breakdown,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)


# Alternatives timed by --planner-study per workload (planner keys of kmeans_plan_override); variants whose plan
# description equals one already timed are skipped.
STUDY_KEYS = {
    "c1": [("small_update", 1), ("assign_split", 1), ("assign_split", 4), ("reduce_tile", 1), ("reduce_tile", 2)],
    "default": [("assign_kernel", 1), ("assign_kernel", 2), ("assign_fold", 1), ("assign_fold", 2),
                ("radix_items", 8), ("radix_items", 16), ("radix_items", 32), ("reduce_tile", 1), ("reduce_tile", 2),
                ("sort_scan", 1), ("sort_scan", 2), ("sort_rank", 1), ("sort_rank", 2), ("radix_bits", 6),
                ("radix_bits", 8)],
}


def planner_study(args, dev):
    """The static planner against every alternative it could have chosen, on the five workload shapes.

    For each shape: kmeans_fit of the workload's iterations with the planner's own choice, then with each single
    override that changes the plan (kmeans_plan_override), median of several fits timed in rounds that take every
    plan once, in rotated order; the gap is the static choice's time over the fastest plan's.  Time to first run: the host-side planning cost (kmeans_plan_describe +
    kmeans_workspace_bytes, no compilation anywhere) and the first fit of each shape in the process against the
    steady state.  The c5 shape is timed resident, one 2^26-row chunk of it (the kernels its streamed fit runs).
    """
    import numpy as np
    import torch

    import means_clustering_amd as km
    import synth

    L = km.lib()
    shapes = [("c1", synth.WORKLOADS["c1"]), ("c2", synth.WORKLOADS["c2"]), ("c3", synth.WORKLOADS["c3"]),
              ("c4", synth.WORKLOADS["c4"]), ("c5", synth.WORKLOADS["c5"].scaled(N=1 << 26, chunk_rows=0))]
    out = {"planner_study": "static plan vs every single-choice alternative, one GPU", "shapes": {}}
    reps = 7
    for name, w in shapes:
        print(f"[bench] planner study {name}: {w.description}", file=sys.stderr, flush=True)
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        X = torch.empty((w.N, w.D), dtype=tdt, device=dev)
        synth.DeviceGenerator(w, dev).fill(X, 0)
        C0 = torch.from_numpy(synth.init_centroids(w)).to(dev)
        a = torch.empty(w.N, dtype=torch.int32, device=dev)
        cnt = torch.empty(w.K, dtype=torch.int32, device=dev)
        C = C0.clone()
        # host planning cost: plan + workspace size, per call (the device query, once per process, done before)
        km.plan_describe(w.N, w.D, w.K, tdt)
        t0 = time.perf_counter()
        for _ in range(200):
            km.plan_describe(w.N, w.D, w.K, tdt)
            L.kmeans_workspace_bytes(km.KM_OP_FIT, w.N, w.D, w.K, km._DT[tdt], 0)
        plan_us = (time.perf_counter() - t0) / 200 * 1e6

        def run(ws):
            C.copy_(C0)
            km.fit(X, C, w.iters, inplace=True, ws=ws, assign_out=a, counts_out=cnt)

        def kernels_of(plan):  # the plan without its workspace size (carved for every path)
            return plan.split("; workspace")[0]

        # the plans: the static one, then every single override that changes the kernels
        plans = [(None, km.plan_describe(w.N, w.D, w.K, tdt))]
        seen = {kernels_of(plans[0][1])}
        for key, val in STUDY_KEYS.get(name, STUDY_KEYS["default"]):
            km.plan_override(key, val)
            try:
                plan = km.plan_describe(w.N, w.D, w.K, tdt)
            finally:
                km.plan_override(key, 0)
            if kernels_of(plan) not in seen:
                seen.add(kernels_of(plan))
                plans.append(((key, val), plan))

        def with_plan(ov, fn):
            if ov:
                km.plan_override(*ov)
            try:
                return fn()
            finally:
                if ov:
                    km.plan_override(ov[0], 0)

        def timed(ws):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            run(ws)
            torch.cuda.synchronize()
            return time.perf_counter() - t0

        # first fit of each plan (the static one first: the shape's first fit in the process), then rounds that
        # time every plan once each, in an order rotated from round to round, so that the GPU's clock drift
        # over the study falls on all plans alike
        wss = [km.Workspace(dev) for _ in plans]
        first = [with_plan(ov, lambda i=i: timed(wss[i])) for i, (ov, _) in enumerate(plans)]
        times = [[] for _ in plans]
        finals = [None] * len(plans)
        for r in range(reps):
            for j in range(len(plans)):
                i = (j + r) % len(plans)
                times[i].append(with_plan(plans[i][0], lambda i=i: timed(wss[i])))
                finals[i] = a.clone()
        res = [{"plan": plan, "first_fit_ms": round(first[i] * 1e3, 3),
                "fit_ms": round(float(np.median(times[i])) * 1e3, 3)} for i, (_, plan) in enumerate(plans)]
        static, variants = res[0], res[1:]
        for i, r in enumerate(variants, 1):
            # every plan reaches the same final assignment (sums may round differently, so only agreement is
            # reported: the trajectories may part after a near tie)
            r["override"] = {plans[i][0][0]: plans[i][0][1]}
            r["same_final_assignment"] = bool(torch.equal(finals[i], finals[0]))
        best = min([static] + variants, key=lambda r: r["fit_ms"])
        out["shapes"][name] = {
            "workload": w.description if name != "c5" else "one 2^26-row chunk of " + w.description,
            "static": static, "alternatives": variants, "best_fit_ms": best["fit_ms"],
            "gap_static_vs_best": round(static["fit_ms"] / best["fit_ms"] - 1.0, 4),
            "best_override": best.get("override", "static"), "host_plan_us": round(plan_us, 2),
            "first_fit_over_steady": round(static["first_fit_ms"] / static["fit_ms"], 3)}
        del X
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


SORT_STUDY_SHAPES = [("c2", 1 << 20, 1024), ("c3", 1 << 20, 65536), ("c4", 1 << 23, 4096),
                     ("c5 chunk", 1 << 26, 4096), ("2^22 keys, 16-bit ids", 1 << 22, 65536),
                     ("2^20 keys, 8-bit ids", 1 << 20, 200), ("2^20 keys, 19-bit ids", 1 << 20, 300_000)]
SORT_STUDY_VARIANTS = [("static", []), ("whole-table count scans", [("sort_scan", 1)]),
                       ("per-digit count scans", [("sort_scan", 2)]), ("thread-counter ranks", [("sort_rank", 1)]),
                       ("wavefront ranks", [("sort_rank", 2)]), ("digits <= 6 bits", [("radix_bits", 6)]),
                       ("digits <= 8 bits", [("radix_bits", 8)])]


def sort_study(dev):
    """The argsort of the update (kmeans_sort_by_cluster) under each of its planner choices: how the (digit,
    block) count table is scanned, how a block's keys are ranked, and the widest digit.  Uniform random ids; each
    variant's time is the best over 3 rotated rounds of the average of 50 calls (10 for 2^26 keys).  Variants
    whose plan equals the static one are still timed (they show the spread)."""
    import torch

    import means_clustering_amd as km

    out = {"sort_study": "kmeans_sort_by_cluster per planner choice, uniform ids, one GPU", "shapes": []}
    for name, N, K in SORT_STUDY_SHAPES:
        print(f"[bench] sort study {name}: N={N} K={K}", file=sys.stderr, flush=True)
        g = torch.Generator(device="cpu").manual_seed(1)
        a = torch.randint(0, K, (N,), generator=g, dtype=torch.int32).to(dev)
        ws = km.Workspace(dev)
        reps = 50 if N <= (1 << 23) else 10
        times = {v: [] for v, _ in SORT_STUDY_VARIANTS}
        plans = {}
        for rnd in range(3):
            order = SORT_STUDY_VARIANTS[rnd % len(SORT_STUDY_VARIANTS):] + SORT_STUDY_VARIANTS[:rnd % len(SORT_STUDY_VARIANTS)]
            for vname, ovs in order:
                for k, v in ovs:
                    km.plan_override(k, v)
                try:
                    plans[vname] = km.plan_describe(N, 64, K, torch.bfloat16).split("update: ")[1].split(", segment")[0]
                    for _ in range(3):
                        km.sort_by_cluster(a, K, ws=ws)
                    torch.cuda.synchronize()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(reps):
                        km.sort_by_cluster(a, K, ws=ws)
                    e1.record()
                    torch.cuda.synchronize()
                    times[vname].append(1e3 * e0.elapsed_time(e1) / reps)
                finally:
                    for k, _ in ovs:
                        km.plan_override(k, 0)
        out["shapes"].append({"name": name, "N": N, "K": K,
                              "us": {v: round(min(t), 2) for v, t in times.items()}, "plan": plans})
        del a, ws
        torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def segment_tile_study(dev):
    """Sort-Inverse Update time with short (16-position) against long (128-position) segment tiles, over N.

    The planner takes short tiles while N rows of G 16-byte lanes fit in half the last-level cache; this sweep
    places that threshold.  Three row shapes (bf16 D = 128 and D = 64, fp32 D = 32) against a sorted-path
    codebook, N = 2^13 .. 2^22, uniform random assignment; each point is the best of three runs of many updates.
    """
    import torch

    import means_clustering_amd as km

    out = {"segment_tile_study": "kmeans_update, short vs long segment tiles, one GPU", "rows": []}
    for dt, D, K in [(torch.bfloat16, 128, 1024), (torch.bfloat16, 64, 4096), (torch.float32, 32, 1024)]:
        lane_bytes = 16 * (1 << max(0, ((D * (4 if dt == torch.float32 else 2) + 15) // 16 - 1).bit_length()))
        for logn in range(13, 23):
            N = 1 << logn
            g = torch.Generator(device=dev).manual_seed(logn)
            X = torch.randn(N, D, device=dev, generator=g).to(dt)
            C = torch.randn(K, D, device=dev, generator=g)
            a = torch.randint(0, K, (N,), device=dev, generator=g, dtype=torch.int32)
            row = {"dtype": str(dt).split(".")[1], "D": D, "K": K, "N": N, "rows_bytes": N * lane_bytes}
            km.plan_override("small_update", 1)
            try:
                for tile in (1, 2):
                    km.plan_override("reduce_tile", tile)
                    C_new, counts = km.update(X, a, C)
                    torch.cuda.synchronize()
                    reps = max(20, min(2000, (1 << 24) // N))
                    best = float("inf")
                    for _ in range(3):
                        t0 = time.perf_counter()
                        for _ in range(reps):
                            km.update(X, a, C, out=C_new, counts_out=counts)
                        torch.cuda.synchronize()
                        best = min(best, (time.perf_counter() - t0) / reps * 1e6)
                    row["long_us" if tile == 1 else "short_us"] = round(best, 2)
            finally:
                km.plan_override("reduce_tile", 0)
                km.plan_override("small_update", 0)
            plan = km.plan_describe(N, D, K, dt)
            row["planner_tile"] = int(plan.split("segment tile ")[1].split(",")[0]) if "segment tile " in plan else None
            row["device"] = plan.split("device: ")[1]
            print(f"[bench] segment tiles {json.dumps(row)}", file=sys.stderr, flush=True)
            out["rows"].append(row)
            del X, C, a
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 6 for c5, 200 for c1, 10 for c2, 5 otherwise)")
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c5", help="headline workload (default c5, the largest)")
    ap.add_argument("--extra", default=None,
                    help="comma-separated resident workloads timed after the headline (default c2,c3,c4 when the "
                         "headline is c5; 'none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for each CPU baseline")
    ap.add_argument("--no-timing", action="store_true", help="no per-kernel events (for profiler runs)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the same-run peak probes")
    ap.add_argument("--no-resident", action="store_true",
                    help="streamed workload: skip the extra fits with a device copy of X")
    ap.add_argument("--batch", type=int, default=1,
                    help="B > 1: time B independent problems of the workload's shape per call (batched fit)")
    ap.add_argument("--ablation", action="store_true",
                    help="only time the materialised-distance assignment and the atomic scatter update "
                         "against FlashAssign and Sort-Inverse Update (one JSON line)")
    ap.add_argument("--planner-study", action="store_true",
                    help="only time the static plan against every single-choice alternative on the five shapes "
                         "(one JSON line)")
    ap.add_argument("--segment-tile-study", action="store_true",
                    help="only time the update with short and long segment tiles over N (one JSON line)")
    ap.add_argument("--sort-study", action="store_true",
                    help="only time the update's argsort under each of its planner choices (one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this "
              "path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    steps_given = args.steps is not None
    if not steps_given:
        args.steps = DEFAULT_STEPS.get(args.workload, 5)
    if args.calibrate_copy:
        import torch
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read_per_launch": 1 << 30, "bytes_written_per_launch": 1 << 30}))
        return
    if args.ablation:
        import torch
        ablation(torch.device("cuda:0"))
        return
    if args.planner_study:
        import torch
        planner_study(args, torch.device("cuda:0"))
        return
    if args.segment_tile_study:
        import torch
        segment_tile_study(torch.device("cuda:0"))
        return
    if args.sort_study:
        import torch
        sort_study(torch.device("cuda:0"))
        return
    if args.batch > 1:
        import torch
        batched(args, torch.device("cuda:0"))
        return

    import torch

    import synth

    dev = torch.device("cuda:0")
    w = synth.WORKLOADS[args.workload]
    extra = args.extra if args.extra is not None else (EXTRA_DEFAULT if w.chunk_rows else "none")
    extra = [] if extra in ("", "none") else [e.strip() for e in extra.split(",")]
    for e in extra:
        if e not in synth.WORKLOADS or synth.WORKLOADS[e].chunk_rows:
            raise SystemExit(f"--extra takes device-resident workloads, not {e!r}")
    peaks = None if args.no_peaks else measured_peaks(dev, w.dtype)
    if w.chunk_rows:
        res = run_streamed(w, args, dev, peaks, args.steps, args.warmup)
    else:
        res = run_resident(w, args, dev, peaks, args.steps, args.warmup, "workload")
    extras = {}
    for e in extra:
        we = synth.WORKLOADS[e]
        # the extras are short (milliseconds a step): the given counts, or enough steps for tens of milliseconds
        st = args.steps if steps_given else DEFAULT_STEPS.get(e, 5)
        extras[e] = run_resident(we, args, dev, peaks, st, max(args.warmup, 1), "extra workload")
        extras[e]["vs_baseline"] = None
    line = {
        "metric": "Lloyd iterations/sec and point-centroid distances/sec (fused assign+update)",
        "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": res["steps"], "warmup": res["warmup"],
        "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": res["dtype"], "data": "synthetic (seeded Gaussian mixtures of the workload's shape)",
        "config": res["config"], "step": res["step"], "distances_per_s": res["distances_per_s"],
        "roofline": res["roofline"], "update_roofline": res["update_roofline"],
        "streaming": res.get("streaming"), "resident_copy": res.get("resident_copy"),
        "cpu_baseline": res["cpu_baseline"],
        "phases_timed_region": res["phases_timed_region"],
        "phase_breakdown_extra_step": res["phase_breakdown_extra_step"],
        "extra_configs": extras, "peaks_measured": peaks, "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
