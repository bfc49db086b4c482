"""The five workloads at full size, in the launch configuration the benchmark times, checked at every iteration.

Teacher-forced comparison (the page's claim is exact Lloyd at every step,
tech §3): iteration t of the GPU run is checked against the fp64 oracle fed
the GPU's own centroids C^t, for every t.

c1-c4: the benchmark's call is one kmeans_fit of all T iterations.  The same
T iterations are also run one call at a time, each call starting from the
previous call's C^t; the chain must end bit for bit where the one call ends
(centroids, last assignment, counts), so the per-iteration results checked
here are the timed run's.  Every iteration: assignments against the oracle on
every point (c1, c2) or on a fixed seeded sample (c3: 16,384 points against
65,536 centroids; c4: 65,536 points: the oracle's direct fp64 distances are
too slow for all of them), counts against the histogram, and the update on
every point against the oracle's update from the GPU's own assignment.

c5: 10^9 rows in pageable host memory, streamed in 2^26-row chunks through a
pinned staging ring.  One kmeans_fit_streamed call of all 3 iterations (the
benchmark's call) against 3 calls of one iteration (bit for bit), then each
iteration: 65,536 sampled assignments against the oracle, counts against the
histogram of all 10^9 assignments, and every one of the 4,096 centroids
against the oracle's fp64 update over all 10^9 points.
"""
import time

import numpy as np
import pytest
import torch

import means_clustering_amd as km
import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _fit(X, C_start, iters, ws, a, counts):
    C = C_start.clone()
    km.fit(X, C, iters, inplace=True, ws=ws, assign_out=a, counts_out=counts)
    torch.cuda.synchronize()
    return C, a.clone(), counts.clone()


@pytest.mark.parametrize("name,sample", [("c1", None), ("c2", None), ("c3", 16_384), ("c4", 65_536)])
def test_config_every_iteration(name, sample):
    w = synth.WORKLOADS[name]
    t0 = time.time()
    print(f"[config] {name}: {w.description}", flush=True)
    Xn = synth.points(w)
    C0 = synth.init_centroids(w, Xn)
    X = parity.x_from_numpy(Xn, w.dtype, DEV)
    C0t = torch.from_numpy(C0).to(DEV)
    ws = km.Workspace(DEV)
    a = torch.empty(w.N, dtype=torch.int32, device=DEV)
    counts = torch.empty(w.K, dtype=torch.int32, device=DEV)
    CT, aT, nT = _fit(X, C0t, w.iters, ws, a, counts)  # the benchmark's call
    rows = None
    if sample is not None:
        rows = np.sort(np.random.default_rng(1234).choice(w.N, sample, replace=False))
    C = C0t
    flips = []
    for t in range(w.iters):
        C_prev = C
        C, at, nt = _fit(X, C_prev, 1, ws, a, counts)
        Cp_n, at_n = C_prev.cpu().numpy(), at.cpu().numpy()
        nm, _ = parity.check_assign(Xn, w.dtype, Cp_n, at_n, rows=rows, label=f"{name} it{t}")
        parity.check_update(Xn, w.dtype, at_n, Cp_n, C.cpu().numpy(), nt.cpu().numpy(), label=f"{name} it{t}")
        flips.append(nm)
        print(f"[config] {name} it{t}: near-tie flips {nm}, empty clusters {int((nt == 0).sum())} "
              f"({time.time() - t0:.1f} s)", flush=True)
    assert torch.equal(C, CT) and torch.equal(at, aT) and torch.equal(nt, nT), \
        f"{name}: {w.iters} one-iteration calls differ from one call of {w.iters} iterations"
    print(f"[config] {name}: every iteration checked, flips per iteration {flips}, "
          f"{time.time() - t0:.1f} s", flush=True)


def test_config_c1_free_running():
    """c1 is small enough to compare the free-running trajectory too (equal whenever no near-tie flipped)."""
    w = synth.WORKLOADS["c1"]
    Xn = synth.points(w)
    C0 = synth.init_centroids(w, Xn)
    X = parity.x_from_numpy(Xn, "f32", DEV)
    C, a, n, _ = km.fit(X, torch.from_numpy(C0).to(DEV), w.iters)
    torch.cuda.synchronize()
    C_ref, a_ref, n_ref, J = oracle.fit(Xn, C0, w.iters, contract=True, xdtype="f32")
    same = np.array_equal(a.cpu().numpy(), a_ref)
    if same:
        assert np.array_equal(n.cpu().numpy(), n_ref)
        assert parity.centroid_error(C.cpu().numpy(), C_ref) <= parity.CENTROID_TOL["f32"]
    print(f"[config] c1 free-running: same final assignment {same}, J = {J[-1]:.6g}", flush=True)


# ---------------------------------------------------------------- c5 ----

_C5 = {}


def _c5():
    """c5's host X (generated on the GPU, 119 GiB pageable) and C^0, shared by the c5 tests of this module."""
    if "X" not in _C5:
        w = synth.WORKLOADS["c5"]
        t0 = time.time()

        def progress(done):
            if done % (1 << 28) < (1 << 24) or done == w.N:
                print(f"[config] c5: generated {done} rows ({time.time() - t0:.1f} s)", flush=True)

        Xh = synth.host_points(w, DEV, pinned=False, progress=progress)  # more than the host lets one process pin
        _C5["Xh"] = Xh
        _C5["X"] = synth.as_numpy_rows(Xh)
        _C5["C0"] = synth.init_centroids(w, _C5["X"])
        _C5["stage"] = km.staging_buffer()
        _C5["cs"] = torch.cuda.Stream(DEV)
    return _C5


def _c5_fit(C_start, iters):
    d = _c5()
    w = synth.WORKLOADS["c5"]
    C, a, n, _ = km.fit_streamed(d["Xh"], C_start, iters, w.chunk_rows, copy_stream=d["cs"], want_assign=True,
                                 stage=d["stage"])
    torch.cuda.synchronize()
    return C, a, n


def test_config_c5_iterations_streamed():
    """One call of 3 streamed iterations equals 3 calls of one, bit for bit; keeps every iteration's state."""
    w = synth.WORKLOADS["c5"]
    t0 = time.time()
    print(f"[config] c5: {w.description}", flush=True)
    d = _c5()
    C0t = torch.from_numpy(d["C0"]).to(DEV)
    CT, aT, nT = _c5_fit(C0t, w.iters)
    print(f"[config] c5: one call of {w.iters} iterations done ({time.time() - t0:.1f} s)", flush=True)
    states = []
    C = C0t
    for t in range(w.iters):
        C_prev = C
        C, a, n = _c5_fit(C_prev, 1)
        states.append((C_prev.cpu().numpy(), a, C.cpu().numpy(), n.cpu().numpy()))
        print(f"[config] c5: iteration {t} as its own call done ({time.time() - t0:.1f} s)", flush=True)
    assert torch.equal(C, CT) and torch.equal(n, nT) and torch.equal(states[-1][1], aT), \
        "c5: 3 one-iteration calls differ from one call of 3 iterations"
    d["states"] = states


@pytest.mark.parametrize("t", [0, 1, 2])
def test_config_c5_iteration_vs_oracle(t):
    d = _c5()
    if "states" not in d:
        pytest.skip("needs test_config_c5_iterations_streamed (it records the per-iteration states)")
    w = synth.WORKLOADS["c5"]
    Xn = d["X"]
    C_prev, a_t, C_next, n = d["states"][t]
    a = a_t.numpy()
    t0 = time.time()
    assert a.min() >= 0 and a.max() < w.K
    assert np.array_equal(n, np.bincount(a, minlength=w.K)), "counts != histogram of the assignments"
    rows = np.sort(np.random.default_rng(55 + t).choice(w.N, 65_536, replace=False))
    nm, _ = parity.check_assign(Xn, "bf16", C_prev, a, rows=rows, label=f"c5 it{t} sampled points")
    print(f"[config] c5 it{t}: {nm} near-tie flips of {len(rows)} sampled points ({time.time() - t0:.1f} s)",
          flush=True)
    err = parity.check_update(Xn, "bf16", a, C_prev, C_next, n, label=f"c5 it{t}")
    print(f"[config] c5 it{t}: all {w.K} centroids within {err:.2e} of the oracle's update over all {w.N} points, "
          f"empty clusters {int((n == 0).sum())} ({time.time() - t0:.1f} s)", flush=True)
    if t == w.iters - 1:
        _C5.clear()  # frees the 119 GiB of host X
