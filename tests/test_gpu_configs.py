"""The five workloads at full size, in the launch configuration the benchmark times.

c1-c4: one kmeans_fit of all T iterations (as timed), which must equal the
same run split as T-1 iterations + 1 (no hidden state), and whose last
iteration is checked against the fp64 oracle fed the GPU's own C^{T-1}:
assignments on every point (c1, c2) or on a seeded sample of points (c3, c4:
the oracle's direct fp64 distances to 65,536 / 4,096 centroids are too slow
for every point), the update on every point.
c5: 10^9 rows in pageable host memory, streamed in 2^26-row chunks through
a pinned staging ring; one
iteration checked on sampled points, on every count and on the centroids of
sampled clusters (their points gathered from all chunks).
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
def test_config_full_size(name, sample):
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
    CT, aT, nT = _fit(X, C0t, w.iters, ws, a, counts)
    Cm, _, _ = _fit(X, C0t, w.iters - 1, ws, a, counts)
    C1, a1, n1 = _fit(X, Cm, 1, ws, a, counts)
    assert torch.equal(CT, C1) and torch.equal(aT, a1) and torch.equal(nT, n1), "T != (T-1) + 1"
    print(f"[config] {name}: GPU runs done in {time.time() - t0:.1f} s", flush=True)
    rows = None
    if sample is not None:
        rows = np.sort(np.random.default_rng(1234).choice(w.N, sample, replace=False))
    Cm_n, aT_n = Cm.cpu().numpy(), aT.cpu().numpy()
    nm, _ = parity.check_assign(Xn, w.dtype, Cm_n, aT_n, rows=rows, label=f"{name} last iteration")
    err = parity.check_update(Xn, w.dtype, aT_n, Cm_n, CT.cpu().numpy(), nT.cpu().numpy(),
                              label=f"{name} last iteration")
    empty = int((nT.cpu().numpy() == 0).sum())
    print(f"[config] {name}: near-tie flips {nm}, centroid error {err:.2e}, empty clusters {empty}, "
          f"checked in {time.time() - t0:.1f} s", flush=True)


def test_config_c1_every_iteration_and_free_running():
    """c1 is small enough to check every iteration, and the free-running trajectory too."""
    w = synth.WORKLOADS["c1"]
    Xn = synth.points(w)
    C0 = synth.init_centroids(w, Xn)
    X = parity.x_from_numpy(Xn, "f32", DEV)
    C = torch.from_numpy(C0).to(DEV)
    flips = 0
    for t in range(w.iters):
        C_prev = C.cpu().numpy()
        C, a, n, _ = km.fit(X, C, 1)
        torch.cuda.synchronize()
        an = a.cpu().numpy()
        nm, _ = parity.check_assign(Xn, "f32", C_prev, an, label=f"c1 it{t}")
        flips += nm
        parity.check_update(Xn, "f32", an, C_prev, C.cpu().numpy(), n.cpu().numpy(), label=f"c1 it{t}")
    C_ref, a_ref, n_ref, J = oracle.fit(Xn, C0, w.iters, contract=True, xdtype="f32")
    if flips == 0:  # without a near-tie flip both trajectories are the same one
        assert np.array_equal(a.cpu().numpy(), a_ref) and np.array_equal(n.cpu().numpy(), n_ref)
        assert parity.centroid_error(C.cpu().numpy(), C_ref) <= parity.CENTROID_TOL["f32"]
    print(f"[config] c1 free-running: flips {flips}, J = {J[-1]:.6g}", flush=True)


def test_config_c5_streamed_full_size():
    w = synth.WORKLOADS["c5"]
    t0 = time.time()
    print(f"[config] c5: {w.description}", flush=True)

    def progress(done):
        if done % (1 << 28) < (1 << 24) or done == w.N:
            print(f"[config] c5: generated {done} rows ({time.time() - t0:.1f} s)", flush=True)

    Xh = synth.host_points(w, DEV, pinned=False, progress=progress)  # 119 GiB: more than can be pinned
    Xn = synth.as_numpy_rows(Xh)
    C0 = synth.init_centroids(w, Xn)
    C0t = torch.from_numpy(C0).to(DEV)
    cs = torch.cuda.Stream(DEV)
    stage = km.staging_buffer()
    C1, a1, n1, _ = km.fit_streamed(Xh, C0t, 1, w.chunk_rows, copy_stream=cs, want_assign=True, stage=stage)
    torch.cuda.synchronize()
    print(f"[config] c5: one streamed iteration done ({time.time() - t0:.1f} s)", flush=True)
    a = a1.numpy()
    n = n1.cpu().numpy()
    C1n = C1.cpu().numpy()
    assert np.array_equal(n, np.bincount(a, minlength=w.K)), "counts != histogram of the assignments"
    assert a.min() >= 0 and a.max() < w.K
    rng = np.random.default_rng(55)
    rows = np.sort(rng.choice(w.N, 65_536, replace=False))
    nm, _ = parity.check_assign(Xn, "bf16", C0, a, rows=rows, label="c5 sampled points")
    # centroids: the largest, smallest and some random clusters, their points gathered in index order
    nonempty = np.nonzero(n)[0]
    order = nonempty[np.argsort(n[nonempty], kind="stable")]
    S = np.unique(np.concatenate([order[:4], order[-4:], rng.choice(nonempty, 16, replace=False)]))
    lab_of = np.full(w.K, -1, dtype=np.int32)
    lab_of[S] = np.arange(len(S), dtype=np.int32)
    parts, labs = [], []
    for r0 in range(0, w.N, w.chunk_rows):
        ach = a[r0:r0 + w.chunk_rows]
        sel = np.nonzero(np.isin(ach, S))[0]
        parts.append(Xn[r0 + sel])
        labs.append(lab_of[ach[sel]])
    Xs, ls = np.concatenate(parts), np.concatenate(labs)
    C_ref, n_ref = oracle.update(Xs, ls, len(S), C0[S].astype(np.float64), "bf16")
    assert np.array_equal(n_ref, n[S])
    err = parity.centroid_error(C1n[S], C_ref)
    assert err <= parity.CENTROID_TOL["bf16"], f"c5 centroid error {err:.3e}"
    empty = n == 0
    assert np.array_equal(C1n[empty], C0[empty])
    print(f"[config] c5: near-tie flips {nm} of {len(rows)} sampled, centroid error {err:.2e} over "
          f"{len(S)} clusters ({len(Xs)} points), empty {int(empty.sum())}, done in {time.time() - t0:.1f} s",
          flush=True)
