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


@pytest.mark.parametrize("scan", [1, 2])
@pytest.mark.parametrize("N,K", [(1, 1), (1000, 7), (4097, 257), (100_003, 4096), (300_001, 65536),
                                 (2**20 + 1, 4096), (8 * 2**20 + 3, 3000), (2**26 + 5, 100_000)])
def test_sort_count_scan_modes(N, K, scan):
    """Both ways of scanning the (digit, block) count table give the same stable argsort: the whole table (or, when
    small, summed by every scatter workgroup) and one scan per digit row with the digits' totals added by each
    scatter workgroup; from one block to 2^26 keys (rows of 8,192 blocks, two scan tiles a digit)."""
    rng = np.random.default_rng(N + 7 * K)
    a = rng.integers(0, K, N)
    a[::997] = K + 3  # a few invalid ids
    km.plan_override("sort_scan", scan)
    try:
        _check(a, K, f"count scan mode {scan}")
    finally:
        km.plan_override("sort_scan", 0)


@pytest.mark.parametrize("rank,bits", [(1, 0), (2, 0), (2, 7), (2, 8), (1, 5)])
@pytest.mark.parametrize("N,K", [(1, 1), (63, 5), (1000, 7), (4097, 257), (100_003, 4096), (300_001, 65536),
                                 (1_000_003, 100_000), (2**20 + 1, 1024), (8 * 2**20 + 3, 4096)])
def test_sort_rank_modes(N, K, rank, bits):
    """Every way of ranking a block's keys gives the same stable argsort: per-thread digit counters and
    wavefront ballots, at the planner's digit widths and at digits of 7 and 8 bits (ballots only; 2-3 passes fewer
    or more than the default), from one key to 2^23 keys (2,048- and 4,096-key blocks), with out-of-range ids."""
    rng = np.random.default_rng(N + 13 * K + rank)
    a = rng.integers(0, K, N)
    a[::991] = -1  # a few invalid ids
    km.plan_override("sort_rank", rank)
    if bits:
        km.plan_override("radix_bits", bits)
    try:
        _check(a, K, f"rank mode {rank}, digits of at most {bits or 'default'} bits")
    finally:
        km.plan_override("sort_rank", 0)
        km.plan_override("radix_bits", 0)


def test_sort_wave_rank_skewed():
    """Wavefront ballots with every lane of a step on one digit, alternating digits and a hot cluster."""
    K = 4096
    a = np.zeros(300_000, dtype=np.int64)
    a[1::2] = K - 1
    a[::7] = 1234
    km.plan_override("sort_rank", 2)
    try:
        _check(a, K, "alternating digits")
        _check(np.full(100_001, 77), K, "one cluster")
        rng = np.random.default_rng(5)
        w = 1.0 / np.arange(1, K + 1) ** 1.2
        _check(rng.choice(K, size=500_000, p=w / w.sum()), K, "zipf")
    finally:
        km.plan_override("sort_rank", 0)


def test_sort_wave_rank_8bit_largest_blocks():
    """8-bit digits ranked by ballots in 8,192-key blocks (2^26 keys: 8,193 blocks, per-digit scans of 3 tiles)."""
    rng = np.random.default_rng(11)
    a = rng.integers(0, 65536, 2**26 + 5)
    km.plan_override("radix_bits", 8)
    try:
        _check(a, 65536, "8-bit digits, 8192-key blocks")
    finally:
        km.plan_override("radix_bits", 0)
