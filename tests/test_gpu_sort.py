"""The inverse map (kmeans_sort_by_cluster): bit-exact stable argsort and segment boundaries."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _expected(a: np.ndarray, K: int):
    key = a.astype(np.int64)
    invalid = (key < 0) | (key >= K)
    key = np.where(invalid, K - 1, key)
    perm = np.argsort(key, kind="stable").astype(np.int64)
    flagged = np.where(invalid[perm], perm | (1 << 31), perm)
    offsets = np.searchsorted(key[perm], np.arange(K + 1), side="left")
    return flagged.astype(np.uint32).view(np.int32), offsets.astype(np.int32)


def _check(a: np.ndarray, K: int, label: str):
    print(f"[sort] {label} N={len(a)} K={K}", flush=True)
    perm, off = km.sort_by_cluster(torch.from_numpy(a.astype(np.int32)).to(DEV), K)
    torch.cuda.synchronize()
    ep, eo = _expected(a, K)
    assert np.array_equal(perm.cpu().numpy(), ep), label
    assert np.array_equal(off.cpu().numpy(), eo), label


@pytest.mark.parametrize("K", [1, 2, 7, 255, 256, 257, 1024, 4096, 65536, 100_000])
@pytest.mark.parametrize("N", [1, 1000, 4096, 4097, 100_003])
def test_sort_uniform(N, K):
    rng = np.random.default_rng(N + K)
    _check(rng.integers(0, K, N), K, "uniform")


@pytest.mark.parametrize("K", [3, 4096, 65536])
def test_sort_all_one_cluster(K):
    _check(np.full(300_001, K - 1 if K > 1 else 0), K, "all in one cluster")
    _check(np.zeros(50_000, dtype=np.int64), K, "all in cluster 0")


def test_sort_zipf_and_invalid():
    rng = np.random.default_rng(3)
    K = 4096
    w = 1.0 / np.arange(1, K + 1) ** 1.2
    a = rng.choice(K, size=200_000, p=w / w.sum())
    _check(a, K, "zipf")
    a[::97] = -3
    a[5::101] = K + 10
    _check(a, K, "zipf + invalid ids")


@pytest.mark.parametrize("N", [4 * 2**20 - 1, 4 * 2**20 + 5, 8 * 2**20 + 3])
def test_sort_block_sizes(N):
    """Around the sizes where the block switches from 2048 to 4096 to 8192 keys."""
    rng = np.random.default_rng(N)
    K = 3000
    a = rng.integers(0, K, N)
    a[::1001] = K + 1  # a few invalid ids
    _check(a, K, "block sizes")


def test_sort_empty_input():
    perm, off = km.sort_by_cluster(torch.empty(0, dtype=torch.int32, device=DEV), 5)
    torch.cuda.synchronize()
    assert perm.numel() == 0 and off.cpu().tolist() == [0] * 6


@pytest.mark.parametrize("N", [2**20, 2**20 + 1])
def test_sort_scan_paths(N):
    """K = 4096 (two 6-bit passes) in blocks of 2048 keys: 64 x 512 digit counts (8 scan tiles, scanned by one
    workgroup) against 64 x 513 (9 tiles, scanned in three launches)."""
    rng = np.random.default_rng(N)
    _check(rng.integers(0, 4096, N), 4096, "scan paths")
