"""Rows too long for the register-resident kernels: the depth-tiled FlashAssign and the column-strip update.

16-bit X with D > 512 and fp32 X with D > 256 take these paths.  Every entry
point is checked against the fp64 oracle on the same inputs, element by
element: assignments (near-tie rule), distances, counts, centroids, exact
ties, split sweeps (few points, many centroids), batched problems, the fit
(every iteration teacher-forced, T iterations in one call equal to T calls
bit for bit) and the streamed fit.
"""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
import oracle
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _data(N, D, K, xdtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    X = (torch.randn(N, D, generator=g) * scale).to(TORCH_DT[xdtype])
    C = (torch.randn(K, D, generator=g) * scale).float()
    return X.to(DEV), C.to(DEV)


def _mixture(N, D, K, xdtype, seed):
    """Points near the centroids (so the assignment is not dominated by near-ties in high dimension)."""
    w = synth.WORKLOADS["c2"].scaled(N=N, D=D, K=K, M=K, dtype="f32", seed=seed, sigma=0.5)
    Xn = synth.points(w)
    C0 = synth.init_centroids(w, Xn)
    X = torch.from_numpy(Xn).to(TORCH_DT[xdtype])
    return X.to(DEV), torch.from_numpy(C0).to(DEV)


def _check_assign(X, C, label):
    print(f"[deep] assign {label} N={X.shape[0]} D={X.shape[1]} K={C.shape[0]} {X.dtype}", flush=True)
    a, d = km.assign(X, C, min_dist=True)
    torch.cuda.synchronize()
    Xn, xdt = parity.x_to_numpy(X)
    Cn = C.cpu().numpy()
    an = a.cpu().numpy()
    nm, a_ref = parity.check_assign(Xn, xdt, Cn, an, label=label)
    Xd = oracle.decode(Xn, xdt)
    Cq = oracle.quantize(Cn.astype(np.float64), xdt)
    ref_d = ((Xd - Cq[an]) ** 2).sum(axis=1)
    scale = (Xd ** 2).sum(axis=1) + (Cq[an] ** 2).sum(axis=1) + 1.0
    D = X.shape[1]
    err = np.abs(d.cpu().numpy().astype(np.float64) - ref_d) / scale
    # fp32 accumulation of D products plus the norms: (D + 2) * 2^-22 relative to ||x||^2 + ||c||^2
    assert err.max() <= (D + 2) * 2.0**-22, f"{label}: distance error {err.max():.2e}"
    return an, a_ref


DEEP_SHAPES = [("bf16", 1000, 513, 100), ("bf16", 777, 1000, 129), ("f16", 2049, 640, 300),
               ("bf16", 300, 4096, 70), ("f32", 1000, 257, 64), ("f32", 513, 600, 33), ("f32", 300, 1024, 100),
               ("bf16", 1, 2000, 1), ("f32", 5, 300, 3), ("bf16", 4133, 520, 1000)]


@pytest.mark.parametrize("case", DEEP_SHAPES, ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}")
def test_deep_assign_random(case):
    xdtype, N, D, K = case
    X, C = _data(N, D, K, xdtype, seed=N + 7 * D + 13 * K)
    _check_assign(X, C, f"random {case}")


@pytest.mark.parametrize("case", [("bf16", 3000, 1024, 256), ("f32", 2000, 300, 128), ("f16", 1500, 700, 500)],
                         ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}")
def test_deep_assign_mixture(case):
    xdtype, N, D, K = case
    X, C = _mixture(N, D, K, xdtype, seed=D)
    an, a_ref = _check_assign(X, C, f"mixture {case}")
    assert (an == a_ref).mean() > 0.999


@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_deep_assign_exact_ties(xdtype):
    # integer grids: every distance is exact in fp32 on both sides, and duplicated centroids never win
    g = torch.Generator().manual_seed(11)
    D = 600
    X = (torch.randint(-2, 3, (1500, D), generator=g).float() / 2).to(TORCH_DT[xdtype]).to(DEV)
    C = torch.randint(-1, 2, (70, D), generator=g).float().to(DEV)
    C[40] = C[2]
    C[69] = C[0]
    C[10] = X[5].float()  # point 5 sits on centroid 10
    an, a_ref = _check_assign(X, C, "exact ties")
    assert np.array_equal(an, a_ref)
    assert not np.isin(an, [40, 69]).any()
    assert an[5] == 10


@pytest.mark.parametrize("case", [("bf16", 600, 1000, 20000), ("f32", 300, 400, 9000)],
                         ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}")
def test_deep_assign_split_sweep(case):
    """Few points against many centroids: the sweep is split over workgroups and merged in index order."""
    xdtype, N, D, K = case
    X, C = _data(N, D, K, xdtype, seed=K)
    _check_assign(X, C, f"split {case}")


UPDATE_SHAPES = [("bf16", 5000, 1000, 70), ("f16", 3001, 513, 300), ("bf16", 20000, 4096, 50),
                 ("f32", 7000, 257, 100), ("f32", 4000, 600, 9), ("f32", 100_000, 300, 2000), ("bf16", 1, 700, 3)]


@pytest.mark.parametrize("case", UPDATE_SHAPES, ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}")
def test_deep_update(case):
    xdtype, N, D, K = case
    X, C = _data(N, D, K, xdtype, seed=N + D)
    g = torch.Generator().manual_seed(D)
    a = torch.randint(0, K, (N,), generator=g, dtype=torch.int32)
    a[: N // 3] = K // 2  # a hot cluster spanning many tiles
    if K > 2:
        a[a == K - 1] = 0  # the last cluster empty
    a = a.to(DEV)
    print(f"[deep] update {case}", flush=True)
    C_new, counts = km.update(X, a, C)
    torch.cuda.synchronize()
    Xn, xdt = parity.x_to_numpy(X)
    parity.check_update(Xn, xdt, a.cpu().numpy(), C.cpu().numpy(), C_new.cpu().numpy(), counts.cpu().numpy(),
                        label=f"deep update {case}")


FIT_CASES = [("bf16", 6000, 1000, 64, 3), ("f32", 4000, 400, 100, 3), ("f16", 3000, 768, 700, 2),
             ("bf16", 16384, 600, 40, 2)]


@pytest.mark.parametrize("case", FIT_CASES, ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}-T{c[4]}")
def test_deep_fit_every_iteration(case):
    xdtype, N, D, K, T = case
    X, C0 = _mixture(N, D, K, xdtype, seed=N + D + K)
    Xn, xdt = parity.x_to_numpy(X)
    print(f"[deep] fit {case}", flush=True)
    C_all, a_all, n_all, J_all = km.fit(X, C0, T, objective=True)
    C = C0
    for t in range(T):
        C_prev = C
        C, a, n, J = km.fit(X, C_prev, 1, objective=True)
        torch.cuda.synchronize()
        Cp = C_prev.cpu().numpy()
        an = a.cpu().numpy()
        parity.check_assign(Xn, xdt, Cp, an, label=f"deep fit {case} it{t}")
        parity.check_update(Xn, xdt, an, Cp, C.cpu().numpy(), n.cpu().numpy(), label=f"deep fit {case} it{t}")
        parity.check_objective(Xn, xdt, Cp, an, J.cpu().numpy()[0], label=f"deep fit {case} it{t}")
        assert J.cpu().numpy()[0] == J_all.cpu().numpy()[t]
    assert torch.equal(C, C_all) and torch.equal(a, a_all) and torch.equal(n, n_all), "T calls != one call"


def test_deep_fit_batched():
    B, N, D, K, T = 3, 2000, 700, 50, 2
    Xs, Cs = [], []
    for b in range(B):
        X, C0 = _mixture(N, D, K, "bf16", seed=100 + b)
        Xs.append(X)
        Cs.append(C0)
    X = torch.stack(Xs)
    C0 = torch.stack(Cs)
    print(f"[deep] batched B={B} N={N} D={D} K={K}", flush=True)
    C, a, n, _ = km.fit_batched(X, C0, T)
    torch.cuda.synchronize()
    for b in range(B):
        Cb, ab, nb, _ = km.fit(Xs[b], Cs[b], T)
        torch.cuda.synchronize()
        assert torch.equal(a[b], ab), f"problem {b}: batched assignment differs"
        assert torch.equal(n[b], nb)
        assert parity.centroid_error(C[b].cpu().numpy(), Cb.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_deep_fit_streamed(xdtype):
    """Streamed in ragged chunks: each iteration against the oracle from its own C^t; one call of T iterations
    equals T calls of one, bit for bit; the first assignment equals the resident one."""
    N, D, K, T, rows = 20000, 600, 80, 2, 7000
    X, C0 = _mixture(N, D, K, xdtype, seed=D + 1)
    Xh = X.cpu().contiguous().pin_memory()
    Xn, xdt = parity.x_to_numpy(X)
    print(f"[deep] streamed {xdtype} N={N} D={D} K={K} chunk {rows}", flush=True)
    C_all, a_all, n_all, _ = km.fit_streamed(Xh, C0, T, rows)
    torch.cuda.synchronize()
    C = C0
    for t in range(T):
        C_prev = C
        C, a_host, n, _ = km.fit_streamed(Xh, C_prev, 1, rows)
        torch.cuda.synchronize()
        Cp = C_prev.cpu().numpy()
        an = a_host.numpy()
        if t == 0:
            assert np.array_equal(an, km.assign(X, C0)[0].cpu().numpy())
        parity.check_assign(Xn, xdt, Cp, an, label=f"deep streamed it{t}")
        parity.check_update(Xn, xdt, an, Cp, C.cpu().numpy(), n.cpu().numpy(), label=f"deep streamed it{t}")
    assert torch.equal(C, C_all) and torch.equal(n, n_all) and np.array_equal(a_host.numpy(), a_all.numpy())


@pytest.mark.parametrize("case", [("bf16", 300, 20_000, 9, 2), ("f32", 200, 5_000, 6, 2), ("f16", 700, 8_192, 40, 2)],
                         ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}")
def test_deep_fit_very_long_rows(case):
    """Rows of thousands of values: tens of depth chunks per tile and up to 40 column strips per update."""
    xdtype, N, D, K, T = case
    X, C0 = _mixture(N, D, K, xdtype, seed=D)
    Xn, xdt = parity.x_to_numpy(X)
    print(f"[deep] very long rows {case}: {km.plan_describe(N, D, K, X.dtype)}", flush=True)
    C = C0
    for t in range(T):
        C_prev = C
        C, a, n, J = km.fit(X, C_prev, 1, objective=True)
        torch.cuda.synchronize()
        Cp = C_prev.cpu().numpy()
        an = a.cpu().numpy()
        parity.check_assign(Xn, xdt, Cp, an, label=f"very long rows {case} it{t}")
        parity.check_update(Xn, xdt, an, Cp, C.cpu().numpy(), n.cpu().numpy(), label=f"very long rows {case} it{t}")
        parity.check_objective(Xn, xdt, Cp, an, J.cpu().numpy()[0], label=f"very long rows {case} it{t}")


@pytest.mark.parametrize("case", [("bf16", 7, 712, 2000), ("f32", 1, 966, 100), ("f16", 300, 2377, 700)],
                         ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}")
def test_deep_fit_more_clusters_than_points(case):
    """K above N on the deep paths: most clusters stay empty and keep their centroids bit for bit."""
    xdtype, N, D, K = case
    X, C0 = _data(N, D, K, xdtype, seed=K + D)
    Xn, xdt = parity.x_to_numpy(X)
    print(f"[deep] K > N {case}", flush=True)
    C = C0
    for t in range(2):
        C_prev = C
        C, a, n, J = km.fit(X, C_prev, 1, objective=True)
        torch.cuda.synchronize()
        Cp = C_prev.cpu().numpy()
        an = a.cpu().numpy()
        parity.check_assign(Xn, xdt, Cp, an, label=f"K > N {case} it{t}")
        parity.check_update(Xn, xdt, an, Cp, C.cpu().numpy(), n.cpu().numpy(), label=f"K > N {case} it{t}")
        parity.check_objective(Xn, xdt, Cp, an, J.cpu().numpy()[0], label=f"K > N {case} it{t}")
        assert int((n.cpu().numpy() == 0).sum()) >= K - N
