"""The size limit: kmeans_fit with N = 2^31 - 1 points, the largest N the ABI accepts (D = 2, bf16, K = 100;
X is 8 GiB, the fit's workspace about 55 GiB).  Every index of FlashAssign (cold and warm), the argsort and the
segmented reduction then runs up to the top of the int32 point range.  Checked on what the oracle can compute
at this size: the assignment of 65,536 random rows and of the last 4,096 rows, the counts against a histogram
of the assignment, and the new centroid of three clusters against the oracle's mean of their points."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _histogram(a, K):
    n = torch.zeros(K, dtype=torch.int64, device=DEV)
    step = 1 << 28
    for r0 in range(0, a.numel(), step):
        n += torch.bincount(a[r0:r0 + step].long(), minlength=K)
    return n


def _check_clusters(X, a, C_prev, C_new, counts, label):
    K = C_prev.shape[0]
    assert torch.equal(counts.long(), _histogram(a, K)), f"{label}: counts"
    n = counts.cpu().numpy()
    live = np.nonzero(n)[0]
    assert int(n.sum()) == a.numel()
    for k in (int(live[np.argmax(n[live])]), int(live[np.argmin(n[live])]), int(live[len(live) // 2])):
        step = 1 << 28  # indices of the cluster's points, in pieces (torch kernels stay below 2^31 elements)
        idx = torch.cat([torch.nonzero(a[r0:r0 + step] == k).squeeze(1) + r0 for r0 in range(0, a.numel(), step)])
        xs, name = parity.x_to_numpy(X[idx])
        C_ref, n_ref = oracle.update(xs, np.zeros(len(xs), dtype=np.int32), 1,
                                     C_prev[k:k + 1].astype(np.float64), name)
        assert int(n_ref[0]) == int(n[k]), f"{label}: cluster {k} count"
        err = parity.centroid_error(C_new[k:k + 1], C_ref)
        assert err <= parity.CENTROID_TOL[name], f"{label}: cluster {k} centroid error {err:.3e}"


def test_fit_at_max_n():
    N, D, K = 2**31 - 1, 2, 100
    free, _ = torch.cuda.mem_get_info()
    if free < 100 * 2**30:
        pytest.skip("needs about 100 GiB of free device memory")
    print(f"[limits] N={N} D={D} K={K}", flush=True)
    w = synth.WORKLOADS["c2"].scaled(N=N, D=D, K=K, M=K, seed=31)
    X = torch.empty((N, D), dtype=torch.bfloat16, device=DEV)
    gen = synth.DeviceGenerator(w, DEV)
    step = 1 << 28
    for r0 in range(0, N, step):
        gen.fill(X[r0:min(N, r0 + step)], r0)
    rng = np.random.default_rng(31)
    C0 = X[torch.from_numpy(rng.choice(N, K, replace=False)).to(DEV)].float().contiguous()
    rows = torch.from_numpy(np.concatenate([rng.choice(N - 4096, 65536, replace=False),
                                            np.arange(N - 4096, N)])).to(DEV)
    xs, name = parity.x_to_numpy(X[rows])

    C1, a1, n1, _ = km.fit(X, C0, 1)  # cold
    torch.cuda.synchronize()
    print("[limits] iteration 1 done", flush=True)
    parity.check_assign(xs, name, C0.cpu().numpy(), a1[rows].cpu().numpy(), label="it0", min_near_ties=1)
    _check_clusters(X, a1, C0.cpu().numpy(), C1.cpu().numpy(), n1, "it0")
    del a1

    C2, a2, n2, _ = km.fit(X, C0, 2)  # the second iteration warm-started
    torch.cuda.synchronize()
    print("[limits] two iterations done", flush=True)
    parity.check_assign(xs, name, C1.cpu().numpy(), a2[rows].cpu().numpy(), label="it1", min_near_ties=1)
    _check_clusters(X, a2, C1.cpu().numpy(), C2.cpu().numpy(), n2, "it1")
    C2b, a2b, n2b, _ = km.fit(X, C1, 1)  # the same iteration from a cold start
    torch.cuda.synchronize()
    assert torch.equal(C2b, C2) and torch.equal(n2b, n2) and torch.equal(a2b, a2)


def test_fit_large_codebook():
    """K = 2^21 + 3 clusters (65,537 groups of 32 on the single-accumulator kernel, a four-pass argsort, a
    fix-up over two million clusters), N = 2^22, D = 8 bf16; sampled rows against the oracle, counts against
    a histogram, three clusters against the oracle's means, warm against cold bit for bit."""
    N, D, K = 2**22, 8, 2**21 + 3
    print(f"[limits] N={N} D={D} K={K}", flush=True)
    w = synth.WORKLOADS["c3"].scaled(N=N, D=D, K=K, M=4096, seed=37)
    X = torch.empty((N, D), dtype=torch.bfloat16, device=DEV)
    synth.DeviceGenerator(w, DEV).fill(X, 0)
    rng = np.random.default_rng(37)
    C0 = X[torch.from_numpy(rng.choice(N, K, replace=False)).to(DEV)].float().contiguous()
    rows = torch.from_numpy(rng.choice(N, 1024, replace=False)).to(DEV)
    xs, name = parity.x_to_numpy(X[rows])

    C1, a1, n1, _ = km.fit(X, C0, 1)
    C2, a2, n2, _ = km.fit(X, C0, 2)
    C2b, a2b, n2b, _ = km.fit(X, C1, 1)
    torch.cuda.synchronize()
    parity.check_assign(xs, name, C0.cpu().numpy(), a1[rows].cpu().numpy(), label="it0", min_near_ties=1)
    parity.check_assign(xs, name, C1.cpu().numpy(), a2[rows].cpu().numpy(), label="it1", min_near_ties=1)
    _check_clusters(X, a1, C0.cpu().numpy(), C1.cpu().numpy(), n1, "it0")
    _check_clusters(X, a2, C1.cpu().numpy(), C2.cpu().numpy(), n2, "it1")
    assert torch.equal(C2b, C2) and torch.equal(n2b, n2) and torch.equal(a2b, a2)
