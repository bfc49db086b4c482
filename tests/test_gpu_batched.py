"""B independent problems per launch (kmeans_fit_batched) against the fp64 oracle, problem by problem."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _batch(name, B, seed0, **kw):
    """B workloads of one shape that differ only in their seed (own mixture, own points)."""
    Xs, Cs = [], []
    for b in range(B):
        w = synth.WORKLOADS[name].scaled(seed=seed0 + b, **kw)
        Xn = synth.points(w)
        Xs.append(Xn)
        Cs.append(synth.init_centroids(w, Xn))
    return w, np.stack(Xs), np.stack(Cs)


def _to_dev(Xn, xdtype):
    return parity.x_from_numpy(Xn.reshape(-1, Xn.shape[-1]), xdtype, DEV).reshape(Xn.shape)


def _teacher_forced(Xn, xdtype, C0, T, label, check=None):
    """T single batched iterations; every checked problem against the oracle fed the GPU's own state."""
    B = Xn.shape[0]
    check = range(B) if check is None else check
    X = _to_dev(Xn, xdtype)
    C = torch.from_numpy(C0).to(DEV)
    for t in range(T):
        print(f"[batched] {label} iteration {t}", flush=True)
        C_prev = C.cpu().numpy()
        C, a, counts, obj = km.fit_batched(X, C, 1, objective=True)
        torch.cuda.synchronize()
        an, cn, Cn, on = a.cpu().numpy(), counts.cpu().numpy(), C.cpu().numpy(), obj.cpu().numpy()
        for b in check:
            lab = f"{label} problem {b} it{t}"
            parity.check_assign(Xn[b], xdtype, C_prev[b], an[b], label=lab)
            parity.check_update(Xn[b], xdtype, an[b], C_prev[b], Cn[b], cn[b], label=lab)
            parity.check_objective(Xn[b], xdtype, C_prev[b], an[b], on[0, b], label=lab)
    return C


def test_batched_fp32_small_problems():
    w, Xn, C0 = _batch("c1", 6, 100, N=3000, K=40)
    _teacher_forced(Xn, "f32", C0, 4, "c1-like fp32 x6")


def test_batched_bf16_ragged():
    """N not a multiple of any block, K not a multiple of a centroid group, D not a multiple of 16."""
    w, Xn, C0 = _batch("c2", 5, 200, N=2001, K=77, D=72)
    _teacher_forced(Xn, "bf16", C0, 3, "bf16 ragged x5")


@pytest.mark.parametrize("B,K", [(3, 600), (2, 400), (3, 170)])
def test_batched_one_launch_update(B, K):
    """A few problems whose clusters take one workgroup per 4, 2 or 1 clusters (at most 512 workgroups): every
    problem and iteration against the oracle."""
    w, Xn, C0 = _batch("c1", B, 900, N=2000, K=K)
    _teacher_forced(Xn, "f32", C0, 2, f"one-launch update B={B} K={K}")


@pytest.mark.parametrize("xdtype,D", [("bf16", 64), ("f32", 24)])
def test_batched_split_sweep(xdtype, D):
    """Three problems of 3,000 points and 2,000 centroids: the centroid sweep is split over several workgroups
    per row block and merged; assignments, updates and the objective (from the merged distances) of every
    problem and iteration against the oracle, and T iterations in one call against T calls."""
    w, Xn, C0 = _batch("c2", 3, 500, N=3000, K=2000, D=D, dtype=xdtype)
    # one such problem splits its sweep (its assignment takes the split scratch); three have 3x the row
    # blocks, still far below the 512 where the split stops
    tdt = torch.bfloat16 if xdtype == "bf16" else torch.float32
    assert km.workspace_bytes(km.KM_OP_ASSIGN, 3 * 3000, D, 2000, tdt) > \
        km.workspace_bytes(km.KM_OP_ASSIGN, 600_000, D, 2000, tdt)
    C = _teacher_forced(Xn, xdtype, C0, 2, f"split sweep {xdtype} x3")
    X = _to_dev(Xn, xdtype)
    C2, a2, n2, _ = km.fit_batched(X, torch.from_numpy(C0).to(DEV), 2)
    torch.cuda.synchronize()
    assert torch.equal(C2, C)


@pytest.mark.parametrize("K", [300, 5000])
def test_batched_assignment_is_the_single_problem_assignment(K):
    """K = 5000: both calls split the centroid sweep, into different numbers of ranges."""
    w, Xn, C0 = _batch("c4", 4, 300, N=5000, K=K)
    X = _to_dev(Xn, "bf16")
    C0t = torch.from_numpy(C0).to(DEV)
    _, a, _, _ = km.fit_batched(X, C0t, 1)
    torch.cuda.synchronize()
    for b in range(4):
        a1, _ = km.assign(X[b], C0t[b])
        torch.cuda.synchronize()
        assert torch.equal(a[b], a1), b


def test_batch_of_one_is_fit():
    """With B = 1 the batched path runs the same kernels on the same data as kmeans_fit."""
    w = synth.WORKLOADS["c2"].scaled(N=30000, K=256)
    Xn = synth.points(w)
    C0 = torch.from_numpy(synth.init_centroids(w, Xn)).to(DEV)
    X = parity.x_from_numpy(Xn, "bf16", DEV)
    C1, a1, n1, o1 = km.fit(X, C0, 5, objective=True)
    Cb, ab, nb, ob = km.fit_batched(X[None], C0[None], 5, objective=True)
    torch.cuda.synchronize()
    assert torch.equal(C1, Cb[0]) and torch.equal(a1, ab[0]) and torch.equal(n1, nb[0])
    # the objective's fp64 sum runs in another (fixed) order
    np.testing.assert_allclose(ob[:, 0].cpu().numpy(), o1.cpu().numpy(), rtol=1e-12)


def test_batched_more_clusters_than_points_and_zero_iterations():
    g = torch.Generator().manual_seed(3)
    X = torch.randn(3, 5, 16, generator=g).to(DEV)
    C0 = torch.randn(3, 8, 16, generator=g).to(DEV)
    C, a, n, _ = km.fit_batched(X, C0, 0)
    torch.cuda.synchronize()
    assert torch.equal(C, C0)
    C, a, n, _ = km.fit_batched(X, C0, 2)
    torch.cuda.synchronize()
    Cn, an, nn, C0n = C.cpu().numpy(), a.cpu().numpy(), n.cpu().numpy(), C0.cpu().numpy()
    for b in range(3):
        assert an[b].min() >= 0 and an[b].max() < 8
        assert nn[b].sum() == 5
    # clusters left empty by the first iteration keep C0 bit for bit
    C1, a1, n1, _ = km.fit_batched(X, C0, 1)
    torch.cuda.synchronize()
    empty1 = n1.cpu().numpy() == 0
    assert np.array_equal(C1.cpu().numpy()[empty1], C0n[empty1])


def test_batched_empty_problem_points():
    X = torch.empty(4, 0, 8, device=DEV)
    C0 = torch.randn(4, 3, 8).to(DEV)
    C, a, n, obj = km.fit_batched(X, C0, 2, objective=True)
    torch.cuda.synchronize()
    assert torch.equal(C, C0) and int(n.abs().sum()) == 0 and float(obj.abs().sum()) == 0.0


def test_batched_c1_full_batch_sampled():
    """256 problems of c1's full shape (fp32, N=16384, D=32, K=64): the launch configuration the
    batched benchmark times.  Two teacher-forced iterations on sampled problems, then one 10-iteration
    call equals ten 1-iteration calls bit for bit."""
    B = 256
    w, Xn, C0 = _batch("c1", B, 1000)
    C = _teacher_forced(Xn, "f32", C0, 2, "c1 x256", check=[0, 1, 97, 254, 255])
    X = _to_dev(Xn, "f32")
    C0t = torch.from_numpy(C0).to(DEV)
    Ca, aa, na, oa = km.fit_batched(X, C0t, 10, objective=True)
    Cs, objs = C0t, []
    for t in range(10):
        Cs, a1, n1, o1 = km.fit_batched(X, Cs, 1, objective=True)
        objs.append(o1)
    torch.cuda.synchronize()
    assert torch.equal(Ca, Cs) and torch.equal(aa, a1) and torch.equal(na, n1)
    assert torch.equal(oa, torch.cat(objs))
