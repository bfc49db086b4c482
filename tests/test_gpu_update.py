"""Sort-Inverse Update (kmeans_update) against the fp64 oracle."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _run(X, a_np, C_prev, label, inplace=False):
    print(f"[update] {label} N={X.shape[0]} D={X.shape[1]} K={C_prev.shape[0]} {X.dtype}", flush=True)
    a = torch.from_numpy(a_np.astype(np.int32)).to(DEV)
    prev_np = C_prev.cpu().numpy().copy()
    if inplace:
        C_new, counts = km.update(X, a, C_prev, out=C_prev)
    else:
        C_new, counts = km.update(X, a, C_prev)
    torch.cuda.synchronize()
    Xn, xdt = parity.x_to_numpy(X)
    return parity.check_update(Xn, xdt, a_np, prev_np, C_new.cpu().numpy(), counts.cpu().numpy(), label=label)


def _x(N, D, xdtype, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(N, D, generator=g) * 2).to(TORCH_DT[xdtype]).to(DEV)


@pytest.mark.parametrize("xdtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(1, 1, 1), (100, 3, 7), (1000, 32, 64), (20000, 128, 1024), (5000, 64, 5000),
                                   (3001, 200, 50), (700, 512, 9), (12345, 96, 4096)],
                         ids=lambda s: "x".join(map(str, s)))
def test_update_random(shape, xdtype):
    N, D, K = shape
    X = _x(N, D, xdtype, seed=N + D + K)
    rng = np.random.default_rng(N * 3 + K)
    a = rng.integers(0, K, N)
    C_prev = torch.randn(K, D, generator=torch.Generator().manual_seed(K)).to(DEV)
    _run(X, a, C_prev, f"random {shape} {xdtype}")


def test_update_hot_cluster_spanning_many_tiles():
    X = _x(400_000, 64, "bf16", seed=1)
    rng = np.random.default_rng(2)
    a = np.where(rng.random(400_000) < 0.7, 5, rng.integers(0, 4096, 400_000))
    C_prev = torch.randn(4096, 64).to(DEV)
    _run(X, a, C_prev, "70% of points in cluster 5")


def test_update_all_points_one_cluster_and_empty_rest():
    X = _x(300_000, 128, "bf16", seed=3)
    a = np.full(300_000, 2)
    C_prev = torch.randn(17, 128).to(DEV)
    _run(X, a, C_prev, "single cluster")


def test_update_zipf_inplace():
    X = _x(250_000, 64, "bf16", seed=4)
    rng = np.random.default_rng(5)
    w = 1.0 / np.arange(1, 4097) ** 1.2
    a = rng.choice(4096, size=250_000, p=w / w.sum())
    C_prev = torch.randn(4096, 64).to(DEV)
    _run(X, a, C_prev, "zipf in place", inplace=True)


@pytest.mark.parametrize("cluster", [0, 16])
def test_update_only_first_or_last_cluster(cluster):
    """Cluster offsets written by the segmented reduction at both ends of the id range."""
    X = _x(5000, 40, "bf16", seed=8 + cluster)
    C_prev = torch.randn(17, 40).to(DEV)
    _run(X, np.full(5000, cluster), C_prev, f"only cluster {cluster}")


def _reduce_geometry(D, xdtype, fine):
    """(sorted positions one segmented-reduction workgroup covers, positions per tile, largest N with short
    tiles): 256 / G tiles of 128 positions, or, for N * G * 16 <= 2^27, of 16 positions (8 for G = 1, G for
    G > 16); G = lanes holding a row in 16-byte pieces (a power of two, at most 64)."""
    per = 4 if xdtype == "f32" else 8
    G = 1
    while G < -(-D // per) and G < 64:
        G *= 2
    tile = (8 if G == 1 else max(G, 16)) if fine else 128
    return (256 // G) * tile, tile, 2**27 // (16 * G)


@pytest.mark.parametrize("D,xdtype,fine", [(64, "bf16", True), (512, "bf16", True), (200, "f32", True),
                                           (128, "bf16", True), (8, "bf16", True), (16, "bf16", True),
                                           (32, "bf16", True), (4, "f32", True), (12, "f32", True),
                                           (512, "bf16", False), (200, "f32", False), (128, "bf16", False),
                                           (64, "bf16", False), (32, "bf16", False), (12, "f32", False),
                                           (8, "bf16", False)])
def test_update_segments_at_group_edges(D, xdtype, fine):
    """Long segments that start or end on, or one position off, the edges of the
    segmented reduction's workgroups, so that whole workgroup sums, head tiles and
    tail tiles are all added; with short tiles (small N) and long ones."""
    B, tile, fine_max_n = _reduce_geometry(D, xdtype, fine)
    sizes = [3 * B, 2 * B + 1, 2 * B - 2, 1, 5 * B + tile, 70 * B - 1, tile - 1, B + 77]
    if not fine:  # a last long segment takes N up to the long-tile range
        sizes.append(max(B, fine_max_n + 1 - sum(sizes)))
    assert (sum(sizes) <= fine_max_n) == fine
    # ids 0, 10, 20, ...: the clusters between stay empty, and K >= 80 takes the sorted path
    a = np.repeat(np.arange(len(sizes) * 10, step=10), sizes)
    np.random.default_rng(11).shuffle(a)
    X = _x(a.size, D, xdtype, seed=12 + D)
    C_prev = torch.randn(len(sizes) * 10, D).to(DEV)
    _run(X, a, C_prev, f"segments at group edges D={D} {xdtype}")


@pytest.mark.parametrize("xdtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(512, 32, 64), (513, 32, 64), (2048, 32, 64), (2049, 32, 64), (50000, 64, 64), (20000, 17, 33), (9000, 1, 2),
                                   (6000, 512, 5), (4100, 100, 1), (600_000, 16, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_update_small_codebook(shape, xdtype):
    """K <= 64: the on-chip path (one workgroup per cluster for N <= 16384, else one chunk of 512 or 2048
    points per workgroup with the chunk sums added in order)."""
    N, D, K = shape
    X = _x(N, D, xdtype, seed=N + 7 * D + K)
    rng = np.random.default_rng(N + K)
    w = rng.random(K) ** 3  # uneven cluster sizes, some clusters empty
    a = rng.choice(K, size=N, p=w / w.sum())
    if K > 3:
        a[a == K // 2] = K - 1  # one empty cluster for sure
    C_prev = torch.randn(K, D, generator=torch.Generator().manual_seed(K + D)).to(DEV)
    _run(X, a, C_prev, f"small codebook {shape} {xdtype}")


@pytest.mark.parametrize("xdtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("shape", [(1, 8, 65), (1000, 32, 512), (16384, 128, 512), (16384, 512, 100), (7777, 3, 257),
                                   (16385, 32, 100), (1000, 32, 513), (5000, 64, 1000), (3000, 16, 2047),
                                   (16384, 32, 2048), (9000, 200, 1999), (16384, 32, 2049)],
                         ids=lambda s: "x".join(map(str, s)))
def test_update_one_workgroup_per_cluster(shape, xdtype):
    """N <= 16384 and 64 < K <= 2048: one workgroup per 1, 2 or 4 clusters (at most 512 workgroups) lists
    each cluster's points and sums them (no sort); one point more (N = 16385) or one cluster more (K = 2049)
    than that takes the sorted path."""
    N, D, K = shape
    X = _x(N, D, xdtype, seed=N + 3 * D + K)
    rng = np.random.default_rng(N + 2 * K)
    w = rng.random(K) ** 4  # uneven cluster sizes, many clusters empty
    a = rng.choice(K, size=N, p=w / w.sum())
    a[a == K - 1] = 0  # the last cluster empty for sure
    C_prev = torch.randn(K, D, generator=torch.Generator().manual_seed(K + D)).to(DEV)
    _run(X, a, C_prev, f"one workgroup per cluster {shape} {xdtype}")


@pytest.mark.parametrize("shape,xdtype", [((7001, 37, 300), "bf16"), ((5000, 3, 129), "f32"), ((9000, 100, 200), "f16"),
                                          ((4000, 257, 70), "bf16")],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_update_rows_not_whole_16_byte_pieces(shape, xdtype):
    """Sorted path (K > 64) with rows whose byte length is not a multiple of 16 (element-wise row loads)."""
    N, D, K = shape
    X = _x(N, D, xdtype, seed=N + D)
    rng = np.random.default_rng(K + 5)
    a = rng.integers(0, K, N)
    a[: N // 3] = K // 2  # one long segment across many tiles
    C_prev = torch.randn(K, D, generator=torch.Generator().manual_seed(D)).to(DEV)
    _run(X, a, C_prev, f"unaligned rows {shape} {xdtype}")


def test_update_small_codebook_hot_cluster_and_invalid_ids():
    X = _x(120_000, 32, "f32", seed=21)
    rng = np.random.default_rng(22)
    a = np.where(rng.random(120_000) < 0.9, 3, rng.integers(0, 40, 120_000))
    a[::97] = -5
    a[1::89] = 40
    C_prev = torch.randn(40, 32).to(DEV)
    _run(X, a, C_prev, "small codebook, 90% in one cluster, invalid ids", inplace=True)


def test_update_five_million_points():
    """Radix blocks of 4096 keys (4 Mi <= N < 8 Mi)."""
    N = 5 * 2**20 + 7
    X = _x(N, 16, "bf16", seed=9)
    rng = np.random.default_rng(10)
    C_prev = torch.randn(3000, 16).to(DEV)
    _run(X, rng.integers(0, 3000, N), C_prev, "5 Mi points")


def test_update_invalid_ids_are_ignored():
    X = _x(10_000, 32, "f32", seed=6)
    rng = np.random.default_rng(7)
    a = rng.integers(0, 100, 10_000)
    a[::13] = -1
    a[1::17] = 100
    a[2::19] = 2**31 - 1
    C_prev = torch.randn(100, 32).to(DEV)
    _run(X, a, C_prev, "invalid ids")


def test_update_empty_input_keeps_centroids():
    X = torch.empty(0, 16, dtype=torch.bfloat16, device=DEV)
    C_prev = torch.randn(5, 16).to(DEV)
    C_new, counts = km.update(X, torch.empty(0, dtype=torch.int32, device=DEV), C_prev)
    torch.cuda.synchronize()
    assert torch.equal(C_new, C_prev) and counts.cpu().tolist() == [0] * 5


def test_update_deterministic():
    X = _x(300_000, 128, "bf16", seed=8)
    a = torch.from_numpy(np.random.default_rng(9).integers(0, 1024, 300_000).astype(np.int32)).to(DEV)
    C_prev = torch.randn(1024, 128).to(DEV)
    c1, n1 = km.update(X, a, C_prev)
    c2, n2 = km.update(X, a, C_prev)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(n1, n2)


MID_N = [("bf16", 300_000, 128, 1000), ("bf16", 1 << 20, 64, 4096), ("f32", 500_000, 32, 512),
         ("f16", 200_000, 100, 300), ("bf16", 400_000, 8, 2000)]


@pytest.mark.parametrize("case", MID_N, ids=lambda c: f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}")
def test_fit_mid_n_short_segment_tiles(case):
    """Default plans between 2 MiB and half the last-level cache of gathered rows take the short segment tiles:
    fits there, each iteration against the oracle (the update on every point, assignments on a sample), and two
    iterations in one call against two calls."""
    import synth
    xdtype, N, D, K = case
    w = synth.WORKLOADS["c2"].scaled(N=N, D=D, K=K, M=K, dtype="f32", seed=N + D)
    Xn = synth.points(w)
    X = torch.from_numpy(Xn).to(TORCH_DT[xdtype]).to(DEV)
    C0 = torch.from_numpy(synth.init_centroids(w, Xn)).to(DEV)
    plan = km.plan_describe(N, D, K, X.dtype)
    print(f"[update] mid N {case}: {plan}", flush=True)
    assert "segment tile 16" in plan or "segment tile 8" in plan, "expected the short segment tiles"
    Xs, name = parity.x_to_numpy(X)
    rows = np.random.default_rng(D).choice(N, 4096, replace=False)
    C = C0
    for t in range(2):
        C_prev = C.cpu().numpy()
        C, a, counts, _ = km.fit(X, C, 1)
        torch.cuda.synchronize()
        an = a.cpu().numpy()
        parity.check_assign(Xs, name, C_prev, an, rows=rows, label=f"mid N {case} it{t}", min_near_ties=1)
        parity.check_update(Xs, name, an, C_prev, C.cpu().numpy(), counts.cpu().numpy(), label=f"mid N {case} it{t}")
    C2, a2, n2, _ = km.fit(X, C0, 2)
    torch.cuda.synchronize()
    assert torch.equal(C2, C) and torch.equal(a2, a) and torch.equal(n2, counts)


@pytest.mark.parametrize("xdtype", ["bf16", "f32"])
def test_update_centroids_not_16_byte_aligned(xdtype):
    """Centroid buffers 4-byte but not 16-byte aligned (views one float into a larger buffer): the reduction's
    16-byte stores must step aside for them; results against the oracle and equal to the aligned call."""
    N, D, K = 200_000, 64, 5000  # short segments: most means are written by the segmented reduction itself
    g = torch.Generator().manual_seed(7)
    X = torch.randn(N, D, generator=g).to(TORCH_DT[xdtype]).to(DEV)
    C = torch.randn(K, D, generator=g).to(DEV)
    a = torch.randint(0, K - 2, (N,), generator=g, dtype=torch.int32).to(DEV)  # the last two clusters empty
    big_prev = torch.empty(K * D + 1, device=DEV)
    big_new = torch.empty(K * D + 3, device=DEV)
    C_prev = big_prev[1:].view(K, D)
    C_prev.copy_(C)
    C_new = big_new[3:].view(K, D)
    assert C_prev.data_ptr() % 16 and C_new.data_ptr() % 16
    C_ref, n_ref = km.update(X, a, C)
    _, n = km.update(X, a, C_prev, out=C_new)
    torch.cuda.synchronize()
    assert torch.equal(C_new, C_ref) and torch.equal(n, n_ref), "unaligned buffers differ from the aligned call"
    Xn, xdt = parity.x_to_numpy(X)
    parity.check_update(Xn, xdt, a.cpu().numpy(), C.cpu().numpy(), C_new.cpu().numpy(), n.cpu().numpy(),
                        label=f"unaligned {xdtype}")
