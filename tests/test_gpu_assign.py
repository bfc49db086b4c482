"""FlashAssign (kmeans_assign) against the fp64 oracle, element by element."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
import oracle
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _data(N, D, K, xdtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    X = (torch.randn(N, D, generator=g) * scale).to(TORCH_DT[xdtype])
    C = (torch.randn(K, D, generator=g) * scale).float()
    return X.to(DEV), C.to(DEV)


def _run(X, C, label):
    print(f"[assign] {label} N={X.shape[0]} D={X.shape[1]} K={C.shape[0]} {X.dtype}", flush=True)
    a, d = km.assign(X, C, min_dist=True)
    torch.cuda.synchronize()
    Xn, xdt = parity.x_to_numpy(X)
    Cn = C.cpu().numpy()
    nm, a_ref = parity.check_assign(Xn, xdt, Cn, a.cpu().numpy(), label=label)
    # distance output: ||x||^2 - 2 x.c + ||c||^2 in fp32 against the fp64 distance to the same centroid
    an = a.cpu().numpy()
    Xd = oracle.decode(Xn, xdt)
    Cq = oracle.quantize(Cn.astype(np.float64), xdt)
    ref_d = ((Xd - Cq[an]) ** 2).sum(axis=1)
    scale = (Xd ** 2).sum(axis=1) + (Cq[an] ** 2).sum(axis=1) + 1.0
    err = np.abs(d.cpu().numpy().astype(np.float64) - ref_d) / scale
    assert err.max() < 2e-5, f"{label}: distance error {err.max():.2e}"
    return an, a_ref


SHAPES = [(1, 1, 1), (37, 3, 2), (1000, 32, 64), (4133, 128, 1000), (2049, 64, 65), (777, 200, 129),
          (300, 512, 37), (5000, 96, 300), (129, 16, 257), (64, 7, 1), (3, 40, 500)]


@pytest.mark.parametrize("xdtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_assign_random(shape, xdtype):
    N, D, K = shape
    X, C = _data(N, D, K, xdtype, seed=N * 131 + D * 7 + K)
    _run(X, C, f"random {shape} {xdtype}")


# long centroid sweeps (>= 256 groups of 32) take the single-accumulator kernel for D <= 128
LONG_SHAPES = [(1500, 16, 8192), (1100, 40, 8200), (900, 64, 9000), (700, 100, 8300), (600, 128, 8192),
               (300, 200, 8192)]


@pytest.mark.parametrize("xdtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", LONG_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_assign_long_sweep(shape, xdtype):
    N, D, K = shape
    X, C = _data(N, D, K, xdtype, seed=N * 17 + D * 3 + K)
    _run(X, C, f"long sweep {shape} {xdtype}")


@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_assign_exact_ties(xdtype):
    # centroids on a coarse grid, points on a finer grid: many exactly equal distances,
    # all computed exactly in fp32 on both sides; the lowest index must win every tie
    g = torch.Generator().manual_seed(5)
    X = (torch.randint(-8, 9, (3000, 8), generator=g).float() / 2).to(TORCH_DT[xdtype]).to(DEV)
    C = (torch.randint(-2, 3, (40, 8), generator=g).float()).to(DEV)
    C[17] = C[3]
    C[39] = C[0]
    an, a_ref = _run(X, C, "exact ties")
    assert np.array_equal(an, a_ref)
    assert not np.isin(an, [17, 39]).any()


def test_assign_centroids_are_points():
    X, _ = _data(500, 64, 1, "bf16", seed=9)
    C = X.float()[:300].clone()
    an, _ = _run(X, C, "C = X[:300]")
    assert np.array_equal(an[:300], np.arange(300))


def test_assign_more_centroids_than_points_and_nan_row():
    X, C = _data(50, 32, 700, "bf16", seed=10)
    X[7] = float("nan")
    a, _ = km.assign(X, C)
    torch.cuda.synchronize()
    an = a.cpu().numpy()
    assert an[7] == 0
    Xn, xdt = parity.x_to_numpy(X)
    keep = np.arange(50) != 7
    ref, _, _ = oracle.assign(Xn[keep], C.cpu().numpy().astype(np.float64), xdt)
    assert np.array_equal(an[keep], ref)


def test_assign_large_offsets_precision():
    # points and centroids far from the origin: the expanded form must still pick the right centroid
    X, C = _data(4000, 128, 256, "bf16", seed=11)
    X = (X.float() + 20.0).to(torch.bfloat16)
    C = C * 0.3 + 20.0
    _run(X, C, "offset +20")


def test_assign_deterministic():
    X, C = _data(20000, 128, 1000, "bf16", seed=12)
    a1, d1 = km.assign(X, C, min_dist=True)
    a2, d2 = km.assign(X, C, min_dist=True)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(d1, d2)


@pytest.mark.parametrize("xdtype,D,K", [("bf16", 64, 4000), ("bf16", 32, 9000), ("f16", 300, 2000), ("f32", 32, 3000),
                                        ("f32", 5, 20000), ("bf16", 128, 70000), ("bf16", 512, 3000)],
                         ids=lambda v: str(v))
def test_assign_split_sweep_equals_unsplit(xdtype, D, K):
    """A small N with a long centroid sweep splits the sweep over several workgroups per row block and merges
    the ranges' best scores in index order.  The same rows inside a large N (one workgroup per row block sweeps
    every centroid) must get the same centroid and distance bit for bit, a row of NaN index 0, and the small
    call must match the oracle."""
    n = 3001
    # the small call takes the split sweep's scratch, the large one none
    assert km.workspace_bytes(km.KM_OP_ASSIGN, n, D, K, TORCH_DT[xdtype]) > \
        km.workspace_bytes(km.KM_OP_ASSIGN, 600_000, D, K, TORCH_DT[xdtype])
    X, C = _data(600_000, D, K, xdtype, seed=K + D)
    X[7] = float("nan")
    print(f"[assign split] {xdtype} D={D} K={K}", flush=True)
    a_big, d_big = km.assign(X, C, min_dist=True)
    a_s, d_s = km.assign(X[:n].contiguous(), C, min_dist=True)
    torch.cuda.synchronize()
    assert int(a_s[7]) == 0
    assert torch.equal(a_s, a_big[:n])
    assert torch.equal(d_s.view(torch.int32), d_big[:n].view(torch.int32))
    keep = np.arange(n) != 7
    Xn, xdt = parity.x_to_numpy(X[:n])
    parity.check_assign(Xn[keep], xdt, C.cpu().numpy(), a_s.cpu().numpy()[keep], label="split sweep")
