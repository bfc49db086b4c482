"""A whole fit captured in a HIP graph replays exactly (kmeans_fit with a caller workspace, kmeans_fit_noalloc).

The library clears its counters and carries with fill kernels (no memset nodes), plans on the host only, and
takes every buffer from the caller or its fixed scratch, so a fit can be captured once and replayed.  Each graph
is replayed three times with unrelated eager fits and synchronisations between the replays; every replay must
equal the eager fit on the same inputs bit for bit (centroids, last assignment, counts, objective).
"""
import pytest
import torch

import means_clustering_amd as km
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CASES = [("c2", dict(N=60_000, K=1024), 4), ("c4", dict(N=100_000, K=4096), 3), ("c1", dict(), 5)]


def _case(name, **kw):
    w = synth.WORKLOADS[name].scaled(**kw)
    Xn = synth.points(w)
    return parity.x_from_numpy(Xn, w.dtype, DEV), torch.from_numpy(synth.init_centroids(w, Xn)).to(DEV)


def _outputs(N, K, T):
    return (torch.empty(N, dtype=torch.int32, device=DEV), torch.empty(K, dtype=torch.int32, device=DEV),
            torch.empty(T, dtype=torch.float64, device=DEV))


def _eager_noise(X, C0):
    """Unrelated work between replays: another fit (through the default workspace and the fixed scratch)."""
    km.fit(X[: X.shape[0] // 2].contiguous(), C0, 2)
    C = C0.clone()
    km.fit_noalloc(X[: X.shape[0] // 3].contiguous(), C, 2)
    torch.cuda.synchronize()


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_fit_graph_replays(case, noalloc):
    name, kw, T = case
    X, C0 = _case(name, **kw)
    N, K = X.shape[0], C0.shape[0]
    print(f"[graph] {name} N={N} D={X.shape[1]} K={K} T={T} noalloc={noalloc}", flush=True)
    # eager reference
    C_ref = C0.clone()
    a_ref, n_ref, J_ref = _outputs(N, K, T)
    ws = km.Workspace(DEV)
    if noalloc:
        km.fit_noalloc(X, C_ref, T, assign_out=a_ref, counts_out=n_ref, objective_out=J_ref)
    else:
        km.fit(X, C_ref, T, inplace=True, ws=ws, assign_out=a_ref, counts_out=n_ref, objective_out=J_ref)
    torch.cuda.synchronize()

    C = torch.empty_like(C0)
    a, n, J = _outputs(N, K, T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream (workspace sized, device queried)
        C.copy_(C0)
        if noalloc:
            km.fit_noalloc(X, C, T, assign_out=a, counts_out=n, objective_out=J)
        else:
            km.fit(X, C, T, inplace=True, ws=ws, assign_out=a, counts_out=n, objective_out=J)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        C.copy_(C0)
        if noalloc:
            km.fit_noalloc(X, C, T, assign_out=a, counts_out=n, objective_out=J)
        else:
            km.fit(X, C, T, inplace=True, ws=ws, assign_out=a, counts_out=n, objective_out=J)
    for r in range(3):
        C.fill_(-1.0)
        a.fill_(-7)
        n.fill_(-7)
        J.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, C_ref), f"replay {r}: centroids differ from the eager fit"
        assert torch.equal(a, a_ref), f"replay {r}: assignment differs"
        assert torch.equal(n, n_ref), f"replay {r}: counts differ"
        assert torch.equal(J, J_ref), f"replay {r}: objective differs"
        _eager_noise(X, C0)
