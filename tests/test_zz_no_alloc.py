"""kmeans_fit_noalloc (no workspace, fixed library scratch) against kmeans_fit, through the C ABI.

Two calls in a row on one GPU, the second with a smaller input (the scratch keeps the first call's
contents): each must equal kmeans_fit with a caller workspace on the same inputs bit for bit (same
kernels and order): centroids, last assignment, counts and objective.
"""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(name, **kw):
    w = synth.WORKLOADS[name].scaled(**kw)
    Xn = synth.points(w)
    return w, parity.x_from_numpy(Xn, w.dtype, DEV), torch.from_numpy(synth.init_centroids(w, Xn)).to(DEV)


def _both(X, C0, iters):
    N, K = X.shape[0], C0.shape[0]
    C_ref, a_ref, n_ref, J_ref = km.fit(X, C0, iters, objective=True)
    C = C0.clone()
    a = torch.full((N,), -7, dtype=torch.int32, device=DEV)
    n = torch.full((K,), -7, dtype=torch.int32, device=DEV)
    J = torch.full((iters,), -7.0, dtype=torch.float64, device=DEV)
    km.fit_noalloc(X, C, iters, assign_out=a, counts_out=n, objective_out=J)
    torch.cuda.synchronize()
    assert torch.equal(C, C_ref), "centroids differ from kmeans_fit"
    assert torch.equal(a, a_ref), "assignment differs from kmeans_fit"
    assert torch.equal(n, n_ref), "counts differ from kmeans_fit"
    assert torch.equal(J, J_ref), "objective differs from kmeans_fit"
    return C


def test_fit_noalloc_equals_fit_two_calls_second_smaller():
    # first: the 2^20-point bf16 workload shape at K = 1,024 (close to the scratch limit), 3 iterations
    w1, X1, C1 = _case("c2", N=1 << 20)
    assert km.workspace_bytes(km.KM_OP_FIT, w1.N, w1.D, w1.K, X1.dtype) <= km.NOALLOC_SCRATCH_BYTES
    print(f"[noalloc] call 1: bf16 N={w1.N} D={w1.D} K={w1.K}", flush=True)
    _both(X1, C1, 3)
    # second, smaller: fp32, ragged sizes, fewer clusters (the sorted path and the small-codebook path)
    for name, kw in (("c1", dict(N=5000, K=33, D=20)), ("c2", dict(N=70001, K=600, D=40))):
        w2, X2, C2 = _case(name, **kw)
        print(f"[noalloc] smaller call: {w2.dtype} N={w2.N} D={w2.D} K={w2.K}", flush=True)
        _both(X2, C2, 2)


def test_fit_noalloc_rejects_oversize():
    w, X, C = _case("c4", N=1 << 23)
    with pytest.raises(km.KMeansError) as e:
        km.fit_noalloc(X, C.clone(), 1)
    assert e.value.status == 2
