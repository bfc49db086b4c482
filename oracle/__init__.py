"""fp64 CPU oracle for exact Lloyd K-Means -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, loads or calls it, and the two share no
code: the oracle is plain C (``kmref.c``) built with gcc, plus an exact
rational brute force (``brute.py``) that pins it.

Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
of its technical summary.

Functions (all numpy in, numpy out):
  assign(X, C, xdtype)        -> a, d1, d2      nearest centroid, lowest index on ties
  update(X, a, K, C_prev)     -> C_new, counts  mean of assigned points, empty keeps
  fit(X, C0, T, contract)     -> C, a, counts, J  T Lloyd iterations
  quantize(C, xdtype)         -> Q(C)           centroids as the contraction sees them
  round_to(x, fmt)            -> RNE to binary32 / bfloat16 / binary16

Parity status: every function is pinned by ``tests/test_oracle_pins.py``
(exact rational brute force, enumeration, closed forms, library
cross-checks, invariants, planted-mistake checks).  At the full sizes of the
synthetic workloads the oracle is trusted through those pins plus the
per-iteration objective bound; nothing on the page pins a full-size result.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kmref.c")
_LIB_PATH = os.path.join(_HERE, "libkmref.so")

XF32, XBF16, XF16, XF64 = 0, 1, 2, 3
_DTYPE_CODES = {"f32": XF32, "bf16": XBF16, "f16": XF16, "f64": XF64}

_lock = threading.Lock()
_lib = None


def build(out_path: str = _LIB_PATH, src_path: str = _SRC, extra_flags=()) -> str:
    """Compile kmref.c with gcc (fp64, no fast-math, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", *extra_flags, "-o", out_path + ".tmp", src_path, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    return out_path


def _bind(lib):
    i64, i32p, f64p, vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double), ctypes.c_void_p
    lib.kmref_decode.argtypes = [vp, ctypes.c_int, i64, f64p]
    lib.kmref_decode.restype = ctypes.c_int
    lib.kmref_round.argtypes = [ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.kmref_round.restype = ctypes.c_double
    lib.kmref_quantize.argtypes = [f64p, i64, ctypes.c_int, f64p]
    lib.kmref_quantize.restype = None
    lib.kmref_assign.argtypes = [vp, ctypes.c_int, i64, i64, f64p, i64, i32p, f64p, f64p]
    lib.kmref_assign.restype = None
    lib.kmref_update.argtypes = [vp, ctypes.c_int, i64, i64, i32p, i64, f64p, f64p, ctypes.POINTER(ctypes.c_int64)]
    lib.kmref_update.restype = None
    lib.kmref_fit.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.POINTER(ctypes.c_float), ctypes.c_int,
                              ctypes.c_int, f64p, i32p, ctypes.POINTER(ctypes.c_int64), f64p]
    lib.kmref_fit.restype = ctypes.c_int
    lib.kmref_num_threads.argtypes = []
    lib.kmref_num_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
        return _lib


def _ptr(arr, ctype):
    return arr.ctypes.data_as(ctypes.POINTER(ctype))


def _xcode(X: np.ndarray, xdtype: str | None):
    """Map a numpy array of stored point values to (contiguous array, dtype code).

    bf16 / f16 data are passed as their raw uint16 bit patterns with xdtype set.
    """
    if xdtype is None:
        if X.dtype == np.float32:
            xdtype = "f32"
        elif X.dtype == np.float64:
            xdtype = "f64"
        elif X.dtype == np.float16:
            xdtype = "f16"
        else:
            raise ValueError("give xdtype for raw 16-bit storage")
    code = _DTYPE_CODES[xdtype]
    want = {XF32: (np.float32,), XF64: (np.float64,), XBF16: (np.uint16,), XF16: (np.uint16, np.float16)}[code]
    if X.dtype not in [np.dtype(w) for w in want]:
        raise TypeError(f"X dtype {X.dtype} does not match storage {xdtype}")
    return np.ascontiguousarray(X), code


_CODE_NAMES = {v: k for k, v in _DTYPE_CODES.items()}
_FORMATS = {"f32": (24, -126, 127), "bf16": (8, -126, 127), "f16": (11, -14, 15)}


class Oracle:
    """numpy-facing wrapper around one loaded copy of the C oracle."""

    def __init__(self, lib):
        self.lib = lib

    def decode(self, X: np.ndarray, xdtype: str | None = None) -> np.ndarray:
        X, code = _xcode(X, xdtype)
        out = np.empty(X.shape, dtype=np.float64)
        self.lib.kmref_decode(X.ctypes.data, code, X.size, _ptr(out, ctypes.c_double))
        return out

    def round_to(self, x, fmt: str):
        """Round fp64 values to the nearest binary32/bfloat16/binary16 value (ties to even)."""
        p, emin, emax = _FORMATS[fmt]
        flat = np.asarray(x, dtype=np.float64).ravel()
        out = np.array([self.lib.kmref_round(float(v), p, emin, emax) for v in flat], dtype=np.float64)
        return out.reshape(np.shape(x))

    def quantize(self, C: np.ndarray, xdtype: str) -> np.ndarray:
        C = np.ascontiguousarray(C, dtype=np.float64)
        out = np.empty_like(C)
        self.lib.kmref_quantize(_ptr(C, ctypes.c_double), C.size, _DTYPE_CODES[xdtype], _ptr(out, ctypes.c_double))
        return out

    def assign(self, X: np.ndarray, C: np.ndarray, xdtype: str | None = None, quantized: bool = False):
        """Nearest centroid of every row of X.

        C holds the centroid state (fp64 or fp32 values); unless ``quantized`` it is
        first rounded to X's storage type (identity for fp32/fp64 X).
        Returns (a int32 [N], d1 float64 [N], d2 float64 [N]).
        """
        X, code = _xcode(X, xdtype)
        N, D = X.shape
        C = np.ascontiguousarray(C, dtype=np.float64)
        K = C.shape[0]
        assert C.shape == (K, D)
        Cq = C if quantized else self.quantize(C, _CODE_NAMES[code])
        a = np.empty(N, dtype=np.int32)
        d1 = np.empty(N, dtype=np.float64)
        d2 = np.empty(N, dtype=np.float64)
        self.lib.kmref_assign(X.ctypes.data, code, N, D, _ptr(Cq, ctypes.c_double), K, _ptr(a, ctypes.c_int32),
                              _ptr(d1, ctypes.c_double), _ptr(d2, ctypes.c_double))
        return a, d1, d2

    def update(self, X: np.ndarray, a: np.ndarray, K: int, C_prev: np.ndarray, xdtype: str | None = None):
        """Means of the assigned points; an empty cluster keeps C_prev. Returns (C_new f64, counts i64)."""
        X, code = _xcode(X, xdtype)
        N, D = X.shape
        a = np.ascontiguousarray(a, dtype=np.int32)
        assert a.shape == (N,)
        Cp = np.ascontiguousarray(C_prev, dtype=np.float64).reshape(K, D)
        Cn = np.empty_like(Cp)
        counts = np.empty(K, dtype=np.int64)
        self.lib.kmref_update(X.ctypes.data, code, N, D, _ptr(a, ctypes.c_int32), K, _ptr(Cp, ctypes.c_double),
                              _ptr(Cn, ctypes.c_double), _ptr(counts, ctypes.c_int64))
        return Cn, counts

    def fit(self, X: np.ndarray, C0: np.ndarray, T: int, contract: bool = True, xdtype: str | None = None):
        """T Lloyd iterations from fp32 C0. Returns (C_T f64, a from the T-th assign, counts, J[T])."""
        X, code = _xcode(X, xdtype)
        N, D = X.shape
        C0 = np.ascontiguousarray(C0, dtype=np.float32)
        K = C0.shape[0]
        C = np.empty((K, D), dtype=np.float64)
        a = np.zeros(N, dtype=np.int32)
        counts = np.zeros(K, dtype=np.int64)
        J = np.zeros(max(T, 1), dtype=np.float64)
        rc = self.lib.kmref_fit(X.ctypes.data, code, N, D, K, _ptr(C0, ctypes.c_float), int(T), int(bool(contract)),
                                _ptr(C, ctypes.c_double), _ptr(a, ctypes.c_int32), _ptr(counts, ctypes.c_int64),
                                _ptr(J, ctypes.c_double))
        if rc != 0:
            raise MemoryError("oracle fit: allocation failed")
        return C, a, counts, J[:T]


def default() -> Oracle:
    return Oracle(load())


def decode(X, xdtype=None):
    return default().decode(X, xdtype)


def round_to(x, fmt):
    return default().round_to(x, fmt)


def quantize(C, xdtype):
    return default().quantize(C, xdtype)


def assign(X, C, xdtype=None, quantized=False):
    return default().assign(X, C, xdtype, quantized)


def update(X, a, K, C_prev, xdtype=None):
    return default().update(X, a, K, C_prev, xdtype)


def fit(X, C0, T, contract=True, xdtype=None):
    return default().fit(X, C0, T, contract, xdtype)


def num_threads() -> int:
    return int(load().kmref_num_threads())
