"""Benchmark: exact Lloyd K-Means iterations on one MI355X.

One step = one kmeans_fit call running the workload's full iteration count
(every iteration: centroid prep, FlashAssign, radix argsort, boundaries,
segmented reduction, fix-up/finalise) on synthetic data already resident in
HBM.  The default workload is c2 (bf16 N=1,048,576 D=128 K=1,024, 20
iterations).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload c1|c2|c3|c4|c5] [--no-cpu-baseline]
  python bench.py --workload c1 --batch 256      (256 independent c1-shaped problems per call)

--workload c5 runs the host-streamed path (X in pinned host memory).
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
    h = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(8):
        d.copy_(h, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    out["h2d_pinned_GBps"] = round(8 * (256 << 20) / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
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


# Timed steps by default: enough that the timed region is tens of milliseconds.
DEFAULT_STEPS = {"c1": 200, "c2": 10}


def timed_step(i: int, steps: int) -> bool:
    """Whether timed step i carries the FlashAssign events.  A timing event costs a
    marker packet and a few microseconds of host time per launch, which is ~12%
    of a c1 iteration, so with many steps only every s-th step is bracketed
    (s = ceil(steps / 8)); the launches of those steps give the average."""
    return i % -(-steps // 8) == 0


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 200 for c1, 10 for c2, 5 otherwise)")
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-timing", action="store_true", help="no per-kernel events (for profiler runs)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the same-run peak probes")
    ap.add_argument("--batch", type=int, default=1,
                    help="B > 1: time B independent problems of the workload's shape per call (batched fit)")
    ap.add_argument("--ablation", action="store_true",
                    help="only time the materialised-distance assignment and the atomic scatter update "
                         "against FlashAssign and Sort-Inverse Update (one JSON line)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.steps is None:
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
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU sharding of this "
              "path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)

    if args.batch > 1:
        import torch
        batched(args, torch.device("cuda:0"))
        return

    import numpy as np
    import torch

    import means_clustering_amd as km
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] workload {w.name}: {w.description}", file=sys.stderr, flush=True)
    torch_dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    streamed = w.chunk_rows > 0

    # ---- inputs (synthetic, seeded), resident in HBM before timing ------------
    t0 = time.perf_counter()
    if streamed:
        def progress(done):
            if done % (1 << 28) < (1 << 24) or done == w.N:
                print(f"[bench] generated {done} / {w.N} rows", file=sys.stderr, flush=True)

        # pageable: 10^9 x 64 bf16 is more than the host lets one process pin; uploaded through a staging ring
        Xh = synth.host_points(w, dev, pinned=False, progress=progress)
        stage = km.staging_buffer()
        Xrows = synth.as_numpy_rows(Xh)
        C0 = torch.from_numpy(synth.init_centroids(w, Xrows)).to(dev)
        rows_of = lambda r: Xrows[:r]  # noqa: E731
    else:
        Xn = synth.points(w)
        C0 = torch.from_numpy(synth.init_centroids(w, Xn)).to(dev)
        X = (torch.from_numpy(Xn.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16"
             else torch.from_numpy(Xn)).to(dev)
        rows_of = lambda r: Xn[:r]  # noqa: E731
    print(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s", file=sys.stderr, flush=True)

    C = C0.clone()
    a = torch.empty(w.N, dtype=torch.int32, device=dev) if not streamed else None
    counts = torch.empty(w.K, dtype=torch.int32, device=dev)
    ws = km.Workspace(dev)
    if streamed:
        copy_stream = torch.cuda.Stream(dev)

    def one_step():
        C.copy_(C0)
        if streamed:
            km.fit_streamed(Xh, C, w.iters, w.chunk_rows, copy_stream=copy_stream, want_assign=False, ws=ws,
                            stage=stage)
        else:
            km.fit(X, C, w.iters, inplace=True, ws=ws, assign_out=a, counts_out=counts)

    for i in range(args.warmup):
        one_step()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {i} done", file=sys.stderr, flush=True)

    # Timed region: HIP events bracket only the FlashAssign launches (mode 2) of a
    # sample of the steps, so the measured throughput carries almost none of their cost.
    timing = not args.no_timing
    if timing:
        km.timing_reset()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if timing:
            km.timing_enable(2 if timed_step(i, args.steps) else 0)
        one_step()
        if streamed:
            torch.cuda.synchronize()
            print(f"[bench] step {i} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if timing:
        km.timing_enable(False)

    its = args.steps * w.iters
    value = its / elapsed
    phases = {}

    def read_phases():
        out = {}
        for ph in km.PHASES:
            ms, n = km.timing_read(ph)
            if n:
                out[ph] = {"total_ms": round(ms, 4), "launches": n, "avg_us": round(1e3 * ms / n, 3)}
        km.timing_reset()
        return out

    if timing:
        phases = read_phases()
        # per-phase breakdown from one more step with every phase timed (not part of `value`)
        km.timing_enable(1)
        one_step()
        torch.cuda.synchronize()
        km.timing_enable(False)
        breakdown = read_phases()
    else:
        breakdown = {}

    # ---- roofline of the dominant kernel (FlashAssign): algorithmic flops per launch
    roof = None
    if "assign" in phases:
        rows_per_launch = w.chunk_rows if streamed else w.N
        flops = 2.0 * rows_per_launch * w.K * w.D
        avg_s = phases["assign"]["avg_us"] * 1e-6
        if streamed:  # launches differ in size (ragged last chunk): use the total
            flops = 2.0 * w.N * w.K * w.D * its / phases["assign"]["launches"]
        achieved = flops / avg_s
        peak = PEAK[w.dtype]
        traffic = _traffic(ASSIGN_SOURCES, w.name)
        roof = {"bound": "mfma", "kernel": "flash_assign", "achieved": round(achieved / 1e12, 2),
                "peak": round(peak / 1e12, 1), "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "flops_per_launch": flops, "avg_launch_us": phases["assign"]["avg_us"],
                "timed_launches": phases["assign"]["launches"],
                "timed_steps": sum(timed_step(i, args.steps) for i in range(args.steps))}

    peaks = None if args.no_peaks else measured_peaks(dev, w.dtype)
    if roof is not None and peaks and "mfma_TFLOPs" in peaks:
        roof["peak_measured"] = peaks["mfma_TFLOPs"]
        roof["frac_of_measured"] = round(roof["achieved"] / peaks["mfma_TFLOPs"], 4)

    # ---- the update's bandwidth: the reduction kernel(s) of the per-phase step against HBM.  Algorithmic
    # bytes per launch: the rows of X it reads once (gathered in cluster order) plus the sorted keys and
    # point indices (8 B a point; the small-codebook path reads the 4-byte ids instead).
    upd = None
    if "reduce" in breakdown:
        es = 2 if w.dtype in ("bf16", "f16") else 4
        rows = w.chunk_rows if streamed else w.N
        small = w.K <= 64
        per_launch = rows * (w.D * es + (4 if small else 8))
        if streamed:  # ragged last chunk: use the total
            per_launch = w.N * (w.D * es + (4 if small else 8)) * w.iters / breakdown["reduce"]["launches"]
        gbps = per_launch / (breakdown["reduce"]["avg_us"] * 1e-6) / 1e9
        upd = {"bound": "hbm", "kernel": "small_update + small_combine" if small else "segment_reduce",
               "achieved": round(gbps, 1), "peak": 8000.0, "unit": "GB/s", "frac": round(gbps / 8000.0, 4),
               "bytes_per_launch": round(per_launch), "avg_launch_us": breakdown["reduce"]["avg_us"]}
        if peaks and "hbm_read_GBps" in peaks:
            upd["peak_measured_read"] = peaks["hbm_read_GBps"]
            upd["frac_of_measured_read"] = round(gbps / peaks["hbm_read_GBps"], 4)

    stream = None
    if streamed:
        es = 2 if w.dtype == "bf16" else 4
        h2d_bytes = w.N * w.D * es * its
        e2e = h2d_bytes / elapsed / 1e9
        copying = None
        if "h2d" in breakdown:  # the extra step: w.iters iterations, each chunk's upload bracketed
            copying = round(w.N * w.D * es * w.iters / (breakdown["h2d"]["total_ms"] * 1e-3) / 1e9, 2)
        stream = {"h2d_bytes_per_iteration": w.N * w.D * es,
                  "h2d_GBps_while_copying": copying,
                  "end_to_end_GBps": round(e2e, 2),
                  "frac_of_pcie5_x16": round(e2e / 64.0, 4)}
        if peaks and "h2d_pinned_GBps" in peaks:
            stream["frac_of_measured_h2d"] = round(e2e / peaks["h2d_pinned_GBps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline: timing the oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, C0.cpu().numpy(), rows_of, budget_s=args.cpu_budget)

    line = {
        "metric": "Lloyd iterations/sec and point-centroid distances/sec (fused assign+update)",
        "value": round(value, 3), "unit": "iterations/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * elapsed / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.description, "name": w.name, "N": w.N, "D": w.D, "K": w.K,
                   "iters_per_step": w.iters, "chunk_rows": w.chunk_rows or None},
        "distances_per_s": round(value * w.N * w.K, 1),
        "roofline": roof, "update_roofline": upd, "cpu_baseline": cpu, "phases_timed_region": phases,
        "phase_breakdown_extra_step": breakdown,
        "streaming": stream, "peaks_measured": peaks,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
