"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments synchronously (before any HIP call), so no GPU is needed."""
import ctypes

import pytest

import means_clustering_amd as km


@pytest.fixture(scope="module")
def L():
    return km.lib()


def test_exports_every_declared_function(L):
    declared = km.header_functions()
    assert "kmeans_assign" in declared and "kmeans_fit_streamed" in declared
    for name in declared:
        assert hasattr(L, name), name
    assert len(declared) == 13


def test_status_strings(L):
    for code in range(5):
        assert L.kmeans_status_string(code)
    assert L.kmeans_status_string(99) == b"unknown status"


def test_workspace_bytes(L):
    f = L.kmeans_workspace_bytes
    assert f(km.KM_OP_ASSIGN, 1000, 128, 1024, km.KM_BF16, 0) > 0
    assert f(km.KM_OP_FIT, 1000, 128, 1024, km.KM_BF16, 0) >= f(km.KM_OP_UPDATE, 1000, 128, 1024, km.KM_BF16, 0)
    assert f(km.KM_OP_FIT, 1 << 20, 128, 1024, km.KM_BF16, 0) % 256 == 0
    # invalid sizes give 0
    assert f(km.KM_OP_ASSIGN, -1, 128, 64, km.KM_BF16, 0) == 0
    assert f(km.KM_OP_ASSIGN, 10, 0, 64, km.KM_BF16, 0) == 0
    assert f(km.KM_OP_ASSIGN, 10, 513, 64, km.KM_BF16, 0) == 0
    assert f(km.KM_OP_ASSIGN, 10, 257, 64, km.KM_F32, 0) == 0
    assert f(km.KM_OP_ASSIGN, 10, 8, 0, km.KM_F32, 0) == 0
    assert f(km.KM_OP_ASSIGN, 10, 8, 4, 7, 0) == 0
    assert f(km.KM_OP_FIT_STREAMED, 10, 8, 4, km.KM_F32, 0) == 0
    assert f(km.KM_OP_FIT_STREAMED, 10**9, 64, 4096, km.KM_BF16, 64 << 20) > 2 * (64 << 20) * 64 * 2
    assert f(km.KM_OP_SORT, 1 << 20, 0, 65536, km.KM_F32, 0) > 0


FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
WS = ctypes.c_void_p(0x100000)    # 256-byte aligned fake workspace address


def _last(L):
    return L.kmeans_last_error().decode()


def test_assign_validation(L):
    a = L.kmeans_assign
    codes = {
        "bad dtype": a(FAKE, 9, 10, 8, FAKE, 4, FAKE, None, WS, 1 << 30, None),
        "null X": a(None, km.KM_BF16, 10, 8, FAKE, 4, FAKE, None, WS, 1 << 30, None),
        "null C": a(FAKE, km.KM_BF16, 10, 8, None, 4, FAKE, None, WS, 1 << 30, None),
        "K=0": a(FAKE, km.KM_BF16, 10, 8, FAKE, 0, FAKE, None, WS, 1 << 30, None),
        "N<0": a(FAKE, km.KM_BF16, -5, 8, FAKE, 4, FAKE, None, WS, 1 << 30, None),
        "N=2^31": a(FAKE, km.KM_BF16, 1 << 31, 8, FAKE, 4, FAKE, None, WS, 1 << 30, None),
        "misaligned C": a(FAKE, km.KM_BF16, 10, 8, ctypes.c_void_p(0x10002), 4, FAKE, None, WS, 1 << 30, None),
    }
    for what, code in codes.items():
        assert code == 1, (what, code, _last(L))
    assert a(FAKE, km.KM_BF16, 10, 600, FAKE, 4, FAKE, None, WS, 1 << 30, None) == 2  # unsupported D
    assert "exceeds" in _last(L)
    assert a(FAKE, km.KM_BF16, 10, 8, FAKE, 4, FAKE, None, None, 0, None) == 3          # no workspace
    assert a(FAKE, km.KM_BF16, 10, 8, FAKE, 4, FAKE, None, WS, 16, None) == 3           # too small
    assert "too small" in _last(L)
    assert a(FAKE, km.KM_BF16, 10, 8, FAKE, 4, FAKE, None, ctypes.c_void_p(0x100010), 1 << 30, None) == 1


def test_update_and_fit_validation(L):
    u = L.kmeans_update
    assert u(FAKE, km.KM_F32, 10, 8, None, 4, FAKE, FAKE, None, WS, 1 << 30, None) == 1      # null assign
    assert u(FAKE, km.KM_F32, 10, 8, FAKE, 4, None, FAKE, None, WS, 1 << 30, None) == 1      # null C_prev
    assert u(FAKE, km.KM_F32, 10, 8, FAKE, 4, FAKE, FAKE, None, WS, 8, None) == 3
    f = L.kmeans_fit
    assert f(FAKE, km.KM_F32, 10, 8, 4, FAKE, -1, None, None, None, WS, 1 << 30, None) == 1  # iters < 0
    assert f(FAKE, km.KM_F32, 10, 8, 4, FAKE, 3, None, None, ctypes.c_void_p(0x10004), WS, 1 << 30, None) == 1
    s = L.kmeans_fit_streamed
    assert s(FAKE, km.KM_BF16, 10, 8, 4, FAKE, 1, 0, None, None, None, WS, 1 << 30, None, FAKE, None, 0) == 1  # chunk 0
    assert s(FAKE, km.KM_BF16, 10, 8, 4, FAKE, 1, 4, None, None, None, WS, 1 << 30, None, None, None, 0) == 1  # no copy stream
    assert s(FAKE, km.KM_BF16, 10, 8, 4, FAKE, 1, 4, None, None, None, WS, 1 << 30, FAKE, FAKE, None, 0) == 1  # same streams
    assert s(FAKE, km.KM_BF16, 10, 8, 4, FAKE, 1, 4, None, None, None, WS, 1 << 30, None, FAKE, FAKE, 63) == 1  # stage < 4 rows
    srt = L.kmeans_sort_by_cluster
    assert srt(None, 10, 4, FAKE, None, WS, 1 << 30, None) == 1
    assert srt(FAKE, 10, 0, FAKE, None, WS, 1 << 30, None) == 1


def test_batched_fit_validation(L):
    wb = L.kmeans_workspace_bytes_batched
    one = wb(1, 16384, 32, 64, km.KM_F32)
    assert one > 0 and one % 256 == 0
    assert wb(256, 16384, 32, 64, km.KM_F32) > 200 * one  # grows with the batch
    assert wb(0, 10, 8, 4, km.KM_F32) == 0
    assert wb(1 << 20, 1 << 12, 8, 4, km.KM_F32) == 0      # B*N = 2^32
    assert wb(1 << 16, 10, 8, 1 << 16, km.KM_F32) == 0     # B*K = 2^32
    assert wb(4, 10, 300, 4, km.KM_F32) == 0               # D > 256 for fp32
    f = L.kmeans_fit_batched
    assert f(FAKE, km.KM_F32, 0, 10, 8, 4, FAKE, 1, None, None, None, WS, 1 << 30, None) == 1        # B = 0
    assert f(FAKE, km.KM_F32, 1 << 20, 1 << 12, 8, 4, FAKE, 1, None, None, None, WS, 1 << 30, None) == 2
    assert "B*N" in _last(L)
    assert f(FAKE, km.KM_F32, 2, 10, 8, 4, FAKE, -1, None, None, None, WS, 1 << 30, None) == 1       # iters < 0
    assert f(FAKE, km.KM_F32, 2, 10, 8, 4, None, 1, None, None, None, WS, 1 << 30, None) == 1        # null C
    assert f(FAKE, km.KM_F32, 2, 10, 8, 4, FAKE, 1, None, None, None, WS, 64, None) == 3             # small ws
    assert f(FAKE, km.KM_F32, 2, 10, 8, 4, FAKE, 1, None, None, ctypes.c_void_p(0x10004), WS, 1 << 30, None) == 1


def test_timing_registry_without_gpu(L):
    assert L.kmeans_timing_enable(3) == 1 and L.kmeans_timing_enable(-1) == 1
    assert L.kmeans_timing_enable(2) == 0
    assert L.kmeans_timing_enable(1) == 0
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert L.kmeans_timing_read(b"assign", ctypes.byref(ms), ctypes.byref(n)) == 0 and n.value == 0
    assert L.kmeans_timing_read(None, ctypes.byref(ms), ctypes.byref(n)) == 1
    assert L.kmeans_timing_reset() == 0
    assert L.kmeans_timing_enable(0) == 0


def test_python_binding_rejects_host_tensors():
    import torch
    X = torch.zeros(4, 8, dtype=torch.bfloat16)
    C = torch.zeros(2, 8)
    with pytest.raises(ValueError):
        km.assign(X, C)


def test_ablation_library_exports_and_validates():
    from means_clustering_amd import ablation
    A = ablation.lib()
    declared = ablation.header_functions()
    assert len(declared) == 4
    for name in declared:
        assert hasattr(A, name), name
    assert A.kmeans_abl_materialized_bytes(10, 600, 4) == 0  # D > 512
    assert A.kmeans_abl_materialized_bytes(10, 64, 4) >= 10 * 4 * 4
    FAKE = ctypes.c_void_p(0x10000)
    assert A.kmeans_abl_assign_materialized(FAKE, 0, 10, 8, FAKE, 4, FAKE, FAKE, 1 << 30, None) == -1  # fp32 X
    assert A.kmeans_abl_assign_materialized(FAKE, 1, 10, 8, FAKE, 4, FAKE, FAKE, 8, None) == -1  # scratch too small
    assert A.kmeans_abl_update_atomic(FAKE, 1, 10, 8, FAKE, 4, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1  # alias

