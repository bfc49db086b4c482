"""Binding of libkm_ablation.so: the materialised-distance assignment and the
atomic scatter update that Flash-KMeans replaces (comparison baselines only;
see include/kmeans_ablation.h)."""
from __future__ import annotations

import ctypes
import os
import re

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkm_ablation.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kmeans_ablation.h")
_lib = None
_DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run means_clustering_amd.build.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.kmeans_abl_materialized_bytes.argtypes = [i64, i64, i64]
        L.kmeans_abl_materialized_bytes.restype = sz
        L.kmeans_abl_assign_materialized.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp, sz, vp]
        L.kmeans_abl_assign_materialized.restype = ctypes.c_int
        L.kmeans_abl_atomic_bytes.argtypes = [i64, i64]
        L.kmeans_abl_atomic_bytes.restype = sz
        L.kmeans_abl_update_atomic.argtypes = [vp, ctypes.c_int, i64, i64, vp, i64, vp, vp, vp, vp, sz, vp]
        L.kmeans_abl_update_atomic.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(kmeans_abl_\w+)\s*\(", text, re.M)))


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def assign_materialized(X: torch.Tensor, C: torch.Tensor, scratch: torch.Tensor | None = None) -> torch.Tensor:
    """Assignment through the full N x K score matrix (16-bit X)."""
    N, D = X.shape
    K = C.shape[0]
    nb = lib().kmeans_abl_materialized_bytes(N, D, K)
    if nb == 0 or X.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("unsupported arguments")
    if scratch is None or scratch.numel() < nb:
        scratch = torch.empty(nb, dtype=torch.uint8, device=X.device)
    a = torch.empty(N, dtype=torch.int32, device=X.device)
    rc = lib().kmeans_abl_assign_materialized(_p(X), _DT[X.dtype], N, D, _p(C), K, _p(a), _p(scratch),
                                              scratch.numel(), _stream(X.device))
    if rc != 0:
        raise RuntimeError(f"kmeans_abl_assign_materialized failed ({rc})")
    return a


def update_atomic(X: torch.Tensor, a: torch.Tensor, C_prev: torch.Tensor, scratch: torch.Tensor | None = None):
    """(C_new, counts) by point-parallel atomic scatter."""
    N, D = X.shape
    K = C_prev.shape[0]
    nb = lib().kmeans_abl_atomic_bytes(D, K)
    if scratch is None or scratch.numel() < nb:
        scratch = torch.empty(nb, dtype=torch.uint8, device=X.device)
    C_new = torch.empty_like(C_prev)
    counts = torch.empty(K, dtype=torch.int32, device=X.device)
    rc = lib().kmeans_abl_update_atomic(_p(X), _DT[X.dtype], N, D, _p(a), K, _p(C_prev), _p(C_new), _p(counts),
                                        _p(scratch), scratch.numel(), _stream(X.device))
    if rc != 0:
        raise RuntimeError(f"kmeans_abl_update_atomic failed ({rc})")
    return C_new, counts
