"""Exact Lloyd K-Means on MI355X (gfx950): Python binding of ``libkmeans_amd.so``.

A thin ctypes layer over the C ABI declared in ``include/kmeans.h``: it
checks tensor types, passes pointers, sizes and the current HIP stream, and
hands the library a device workspace.  Every step of the computation runs in
the library's HIP kernels; there is no CPU or PyTorch fallback, and using this
module without the built library raises an error.

Citations name the page "Flash-KMeans: Fast and Memory-Efficient Exact
K-Means" (gist.science summary of paper 2603.09229); "tech §n" is a section
of its technical summary.

Entry points (all tensors on one ROCm device unless stated):
  assign(X, C)                       nearest centroid per point   (tech §2.1 FlashAssign)
  sort_by_cluster(a, K)              stable argsort + boundaries  (tech §2.2 inverse map)
  update(X, a, C_prev)               means, empty keeps previous  (tech §2.2 Sort-Inverse Update)
  fit(X, C0, iters)                  Lloyd iterations, X resident
  fit_streamed(X_host, C0, iters, chunk_rows)   X in host memory (tech §2.3 chunked overlap)
  fit_batched(X, C0, iters)          B independent problems per launch (tech §1 online primitive)
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkmeans_amd.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kmeans.h")

KM_F32, KM_BF16, KM_F16 = 0, 1, 2
KM_OP_ASSIGN, KM_OP_UPDATE, KM_OP_FIT, KM_OP_FIT_STREAMED, KM_OP_SORT, KM_OP_FIT_STREAMED_WARM = 0, 1, 2, 3, 4, 5
KM_OP_FIT_STREAMED_RESIDENT = 6
STATUS = {0: "KM_OK", 1: "KM_ERR_INVALID_VALUE", 2: "KM_ERR_UNSUPPORTED", 3: "KM_ERR_WORKSPACE", 4: "KM_ERR_HIP"}
_DT = {torch.float32: KM_F32, torch.bfloat16: KM_BF16, torch.float16: KM_F16}


class KMeansError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lock = threading.Lock()
_lib = None


def _bind(lib):
    i64, vp, c_int, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "kmeans_workspace_bytes": (sz, [c_int, i64, i64, i64, c_int, i64]),
        "kmeans_assign": (c_int, [vp, c_int, i64, i64, vp, i64, vp, vp, vp, sz, vp]),
        "kmeans_sort_by_cluster": (c_int, [vp, i64, i64, vp, vp, vp, sz, vp]),
        "kmeans_update": (c_int, [vp, c_int, i64, i64, vp, i64, vp, vp, vp, vp, sz, vp]),
        "kmeans_fit": (c_int, [vp, c_int, i64, i64, i64, vp, ctypes.c_int32, vp, vp, vp, vp, sz, vp]),
        "kmeans_fit_streamed": (c_int, [vp, c_int, i64, i64, i64, vp, ctypes.c_int32, i64, vp, vp, vp, vp, sz, vp,
                                        vp, vp, sz]),
        "kmeans_workspace_bytes_batched": (sz, [i64, i64, i64, i64, c_int]),
        "kmeans_fit_batched": (c_int, [vp, c_int, i64, i64, i64, i64, vp, ctypes.c_int32, vp, vp, vp, vp, sz, vp]),
        "kmeans_fit_noalloc": (c_int, [vp, c_int, i64, i64, i64, vp, ctypes.c_int32, vp, vp, vp, vp]),
        "kmeans_plan_override": (c_int, [ctypes.c_char_p, i64]),
        "kmeans_plan_describe": (c_int, [i64, i64, i64, c_int, ctypes.c_char_p, sz]),
        "kmeans_status_string": (ctypes.c_char_p, [c_int]),
        "kmeans_last_error": (ctypes.c_char_p, []),
        "kmeans_timing_enable": (c_int, [c_int]),
        "kmeans_timing_read": (c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]),
        "kmeans_timing_reset": (c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def lib():
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                   "(python -m means_clustering_amd.build)")
            _lib = _bind(ctypes.CDLL(LIB_PATH))
        return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/kmeans.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(kmeans_\w+)\s*\(", text, re.M)))


def _check(status: int):
    if status != 0:
        raise KMeansError(status, lib().kmeans_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype(X: torch.Tensor) -> int:
    if X.dtype not in _DT:
        raise TypeError(f"X must be float32, bfloat16 or float16, got {X.dtype}")
    return _DT[X.dtype]


def workspace_bytes(op: int, N: int, D: int, K: int, dtype=torch.bfloat16, chunk_rows: int = 0) -> int:
    return int(lib().kmeans_workspace_bytes(op, N, D, K, _DT[dtype], chunk_rows))


class Workspace:
    """A reusable device scratch buffer for the library's calls."""

    def __init__(self, device=None):
        self.device = torch.device(device) if device is not None else None
        self.buf = None

    def get(self, nbytes: int, device) -> torch.Tensor:
        nbytes = max(int(nbytes), 256)
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


_default_ws: dict = {}


def _ws(ws: Workspace | None, nbytes: int, device) -> torch.Tensor:
    if ws is None:
        ws = _default_ws.setdefault(str(device), Workspace(device))
    return ws.get(nbytes, device)


def _need(X: torch.Tensor, C: torch.Tensor):
    if not X.is_cuda or not C.is_cuda:
        raise ValueError("X and C must be device tensors")
    if X.dim() != 2 or C.dim() != 2 or X.shape[1] != C.shape[1]:
        raise ValueError("X must be N x D and C K x D")
    if C.dtype != torch.float32:
        raise TypeError("centroids must be float32")
    if not X.is_contiguous() or not C.is_contiguous():
        raise ValueError("X and C must be contiguous")


def assign(X: torch.Tensor, C: torch.Tensor, min_dist: bool = False, out: torch.Tensor | None = None,
           ws: Workspace | None = None):
    """Nearest centroid of every row of X (FlashAssign). Returns (assign int32[N], dist fp32[N] or None)."""
    _need(X, C)
    N, D = X.shape
    K = C.shape[0]
    a = out if out is not None else torch.empty(N, dtype=torch.int32, device=X.device)
    d = torch.empty(N, dtype=torch.float32, device=X.device) if min_dist else None
    nb = workspace_bytes(KM_OP_ASSIGN, N, D, K, X.dtype)
    w = _ws(ws, nb, X.device)
    _check(lib().kmeans_assign(_ptr(X), _dtype(X), N, D, _ptr(C), K, _ptr(a), _ptr(d), _ptr(w), w.numel(),
                               ctypes.c_void_p(_stream(X.device))))
    return a, d


def sort_by_cluster(a: torch.Tensor, K: int, ws: Workspace | None = None):
    """Stable argsort of cluster ids. Returns (perm int32[N], offsets int32[K+1])."""
    if a.dtype != torch.int32 or not a.is_cuda or a.dim() != 1 or not a.is_contiguous():
        raise ValueError("a must be a contiguous int32 device vector")
    N = a.shape[0]
    perm = torch.empty(N, dtype=torch.int32, device=a.device)
    off = torch.empty(K + 1, dtype=torch.int32, device=a.device)
    nb = int(lib().kmeans_workspace_bytes(KM_OP_SORT, N, 1, K, KM_F32, 0))
    w = _ws(ws, nb, a.device)
    _check(lib().kmeans_sort_by_cluster(_ptr(a), N, K, _ptr(perm), _ptr(off), _ptr(w), w.numel(),
                                        ctypes.c_void_p(_stream(a.device))))
    return perm, off


def update(X: torch.Tensor, a: torch.Tensor, C_prev: torch.Tensor, out: torch.Tensor | None = None,
           ws: Workspace | None = None, counts_out: torch.Tensor | None = None):
    """Sort-Inverse Update. Returns (C_new fp32[K, D], counts int32[K])."""
    _need(X, C_prev)
    if a.dtype != torch.int32 or a.shape != (X.shape[0],) or not a.is_contiguous():
        raise ValueError("a must be a contiguous int32 vector of length N")
    N, D = X.shape
    K = C_prev.shape[0]
    C_new = out if out is not None else torch.empty_like(C_prev)
    counts = counts_out if counts_out is not None else torch.empty(K, dtype=torch.int32, device=X.device)
    nb = workspace_bytes(KM_OP_UPDATE, N, D, K, X.dtype)
    w = _ws(ws, nb, X.device)
    _check(lib().kmeans_update(_ptr(X), _dtype(X), N, D, _ptr(a), K, _ptr(C_prev), _ptr(C_new), _ptr(counts),
                               _ptr(w), w.numel(), ctypes.c_void_p(_stream(X.device))))
    return C_new, counts


def fit(X: torch.Tensor, C0: torch.Tensor, iters: int, objective: bool = False, inplace: bool = False,
        ws: Workspace | None = None, assign_out: torch.Tensor | None = None,
        counts_out: torch.Tensor | None = None, objective_out: torch.Tensor | None = None):
    """Lloyd iterations with X in device memory.

    Returns (C, assign, counts, objective-or-None); C is C0 itself when ``inplace``.
    Preallocated ``*_out`` tensors are used as given (no allocation in the call).
    """
    _need(X, C0)
    N, D = X.shape
    K = C0.shape[0]
    C = C0 if inplace else C0.clone()
    a = assign_out if assign_out is not None else torch.empty(N, dtype=torch.int32, device=X.device)
    counts = counts_out if counts_out is not None else torch.empty(K, dtype=torch.int32, device=X.device)
    obj = objective_out
    if objective and obj is None:
        obj = torch.empty(max(iters, 1), dtype=torch.float64, device=X.device)
    nb = workspace_bytes(KM_OP_FIT, N, D, K, X.dtype)
    w = _ws(ws, nb, X.device)
    _check(lib().kmeans_fit(_ptr(X), _dtype(X), N, D, K, _ptr(C), int(iters), _ptr(a), _ptr(counts), _ptr(obj),
                            _ptr(w), w.numel(), ctypes.c_void_p(_stream(X.device))))
    return C, a, counts, (obj[:iters] if obj is not None else None)


NOALLOC_SCRATCH_BYTES = 64 << 20  # KMEANS_NOALLOC_SCRATCH_BYTES of include/kmeans.h


def fit_noalloc(X: torch.Tensor, C: torch.Tensor, iters: int, assign_out: torch.Tensor | None = None,
                counts_out: torch.Tensor | None = None, objective_out: torch.Tensor | None = None):
    """kmeans_fit_noalloc: Lloyd iterations in place on C with the library's fixed scratch (no workspace).

    Every tensor is the caller's (outputs may be None); the call itself allocates nothing.  Shapes whose
    workspace exceeds NOALLOC_SCRATCH_BYTES raise KMeansError (KM_ERR_UNSUPPORTED).
    """
    _need(X, C)
    N, D = X.shape
    K = C.shape[0]
    _check(lib().kmeans_fit_noalloc(_ptr(X), _dtype(X), N, D, K, _ptr(C), int(iters), _ptr(assign_out),
                                    _ptr(counts_out), _ptr(objective_out), ctypes.c_void_p(_stream(X.device))))
    return C


def fit_batched(X: torch.Tensor, C0: torch.Tensor, iters: int, objective: bool = False, inplace: bool = False,
                ws: Workspace | None = None, assign_out: torch.Tensor | None = None,
                counts_out: torch.Tensor | None = None, objective_out: torch.Tensor | None = None):
    """Lloyd iterations of B independent problems: X is B x N x D, C0 is B x K x D (fp32).

    Returns (C [B, K, D], assign int32 [B, N], counts int32 [B, K], objective fp64 [iters, B] or None).
    """
    if not X.is_cuda or not C0.is_cuda:
        raise ValueError("X and C0 must be device tensors")
    if X.dim() != 3 or C0.dim() != 3 or X.shape[0] != C0.shape[0] or X.shape[2] != C0.shape[2]:
        raise ValueError("X must be B x N x D and C0 B x K x D")
    if C0.dtype != torch.float32:
        raise TypeError("centroids must be float32")
    if not X.is_contiguous() or not C0.is_contiguous():
        raise ValueError("X and C0 must be contiguous")
    B, N, D = X.shape
    K = C0.shape[1]
    C = C0 if inplace else C0.clone()
    a = assign_out if assign_out is not None else torch.empty((B, N), dtype=torch.int32, device=X.device)
    counts = counts_out if counts_out is not None else torch.empty((B, K), dtype=torch.int32, device=X.device)
    obj = objective_out
    if objective and obj is None:
        obj = torch.empty((max(iters, 1), B), dtype=torch.float64, device=X.device)
    nb = int(lib().kmeans_workspace_bytes_batched(B, N, D, K, _dtype(X)))
    w = _ws(ws, nb, X.device)
    _check(lib().kmeans_fit_batched(_ptr(X), _dtype(X), B, N, D, K, _ptr(C), int(iters), _ptr(a), _ptr(counts),
                                    _ptr(obj), _ptr(w), w.numel(), ctypes.c_void_p(_stream(X.device))))
    return C, a, counts, (obj[:iters] if obj is not None else None)


STAGE_SLOT_BYTES = 64 << 20  # default staging slot for pageable X (4 slots)

# Host buffers read or written by enqueued copies, held until the work has passed an event:
# torch's pinned-memory cache may hand a freed block out again while a DMA still uses it.
_inflight: list = []
_inflight_lock = threading.Lock()


def _hold_until_done(device, *objs):
    ev = torch.cuda.Event()
    ev.record(torch.cuda.current_stream(device))
    with _inflight_lock:
        _inflight.append((ev, objs))
        _inflight[:] = [(e, o) for (e, o) in _inflight if not e.query()]


def staging_buffer(nbytes: int = 4 * STAGE_SLOT_BYTES) -> torch.Tensor:
    """A pinned host byte buffer for streaming X that is not pinned itself."""
    return torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)


def fit_streamed(X_host: torch.Tensor, C0: torch.Tensor, iters: int, chunk_rows: int, copy_stream=None,
                 want_assign: bool = True, objective: bool = False, ws: Workspace | None = None,
                 stage: torch.Tensor | None = None, warm_start: bool = True, resident: bool | int = False):
    """Lloyd iterations with X in host memory, streamed in chunks.

    X_host may be pinned (uploaded directly) or pageable (uploaded through the
    pinned ``stage`` buffer, allocated here if not given).  ``resident``: True
    keeps a device copy of all of X (uploaded in the first iteration only), an
    int keeps that many bytes of leading chunks (needs warm_start).  Returns
    (C, assign_host int32[N] pinned or None, counts, objective-or-None).  The
    call returns once all work is enqueued on the current stream.
    """
    if X_host.is_cuda or X_host.dim() != 2 or not X_host.is_contiguous():
        raise ValueError("X_host must be a contiguous 2-D host tensor")
    if not C0.is_cuda or C0.dtype != torch.float32 or X_host.shape[1] != C0.shape[1]:
        raise ValueError("C0 must be a K x D float32 device tensor matching X_host")
    N, D = X_host.shape
    K = C0.shape[0]
    dev = C0.device
    if X_host.is_pinned():
        stage = None
    elif stage is None:
        stage = staging_buffer()
    elif stage.is_cuda or not stage.is_pinned() or stage.dtype != torch.uint8:
        raise ValueError("stage must be a pinned uint8 host tensor")
    C = C0.clone()
    a = torch.empty(N, dtype=torch.int32, pin_memory=True) if want_assign else None
    counts = torch.empty(K, dtype=torch.int32, device=dev)
    obj = torch.empty(max(iters, 1), dtype=torch.float64, device=dev) if objective else None
    # warm_start: room for every chunk's order (8 bytes a row of device memory), so iterations after the first
    # assign each chunk warm; without it the workspace holds two chunk buffers and one chunk's scratch only
    if resident is True:
        if not warm_start:
            raise ValueError("a resident copy of X needs warm_start")
        nb = workspace_bytes(KM_OP_FIT_STREAMED_RESIDENT, N, D, K, X_host.dtype, chunk_rows)
    else:
        nb = workspace_bytes(KM_OP_FIT_STREAMED_WARM if warm_start else KM_OP_FIT_STREAMED, N, D, K, X_host.dtype,
                             chunk_rows)
        if resident:
            if not warm_start or int(resident) < 0:
                raise ValueError("resident bytes must be >= 0 and need warm_start")
            nb += int(resident)
    w = _ws(ws, nb, dev)
    cs = copy_stream if copy_stream is not None else torch.cuda.Stream(dev)
    # (the size asked for, not the buffer's: a larger reused buffer must not turn the warm start on)
    st = lib().kmeans_fit_streamed(_ptr(X_host), _dtype(X_host), N, D, K, _ptr(C), int(iters), int(chunk_rows),
                                   _ptr(a), _ptr(counts), _ptr(obj), _ptr(w), nb,
                                   ctypes.c_void_p(_stream(dev)), ctypes.c_void_p(cs.cuda_stream),
                                   _ptr(stage), 0 if stage is None else stage.numel())
    _hold_until_done(dev, X_host, stage, a)  # (also after a failed call: work it enqueued may still run)
    _check(st)
    return C, a, counts, (obj[:iters] if obj is not None else None)


PLAN_KEYS = ("assign_kernel", "assign_fold", "assign_split", "reduce_tile", "radix_items", "small_update",
             "sort_scan", "sort_rank", "radix_bits")


def plan_override(key: str, value: int = 0):
    """Replace one planner choice for later calls (0 restores the planner's choice); for measurement only."""
    _check(lib().kmeans_plan_override(key.encode(), int(value)))


def plan_describe(N: int, D: int, K: int, dtype=torch.bfloat16) -> str:
    """The plan kmeans_fit makes for this shape on the current device, as one line of text."""
    buf = ctypes.create_string_buffer(1024)
    _check(lib().kmeans_plan_describe(N, D, K, _DT[dtype], buf, len(buf)))
    return buf.value.decode()


def timing_enable(on=True):
    """on: True / 1 = every kernel phase, 2 = FlashAssign launches only, False / 0 = off."""
    mode = int(on) if not isinstance(on, bool) else (1 if on else 0)
    _check(lib().kmeans_timing_enable(mode))


def timing_reset():
    _check(lib().kmeans_timing_reset())


def timing_read(phase: str):
    """(total milliseconds, launches) recorded for one kernel phase (waits for its events)."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib().kmeans_timing_read(phase.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


PHASES = ("prep", "assign", "sort", "segments", "reduce", "finalize", "objective", "h2d", "d2h")
