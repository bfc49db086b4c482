"""Seeded synthetic K-Means workloads (shared by the tests, the benchmark and the oracle checks).

Holds no clustering arithmetic: it only draws points and initial centroids,
deterministically from a seed (Philox4x32-10 + Box-Muller, see ``gen.c``).

The five workloads follow the shapes the Flash-KMeans page motivates (tech §1:
large N, large codebooks, hot clusters, data beyond device memory); the page
itself names no dataset, so every input here is a synthetic mixture:

  c1  fp32, N=16,384, D=32, K=64, 10 iterations; 64 Gaussian components,
      centres ~ N(0, 4I), sigma 1, equal weights; init = first K points.
  c2  bf16, N=1,048,576, D=128, K=1,024, 20 iterations; 1,024 components,
      centres ~ N(0, I), sigma 0.3; init = K points sampled without replacement.
  c3  bf16, N=1,048,576, D=128, K=65,536, 5 iterations; 8,192 unit centres,
      points = normalise(centre + 0.1 N(0, I)); init = K sampled points.
  c4  bf16, N=8,388,608, D=64, K=4,096, 10 iterations; 4,096 components with
      Zipf(s=1.2) weights, centres ~ N(0, 4I), sigma 1; init = K sampled points.
  c5  bf16, N=1,000,000,000, D=64, K=4,096, 3 iterations; 4,096 equal-weight
      components, centres ~ N(0, 4I), sigma 1; streamed from pinned host memory
      in chunks of 64 Mi rows; init = K sampled points.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_GPU_SRC = os.path.join(_HERE, "gen_gpu.hip")
_GPU_LIB_PATH = os.path.join(_HERE, "libsynth_gpu.so")
_lock = threading.Lock()
_lib = None
_gpu_lib = None


def build(out_path: str = _LIB_PATH, gpu_out_path: str = _GPU_LIB_PATH) -> str:
    """Compile the host generator (gcc) and its device twin (hipcc, gfx950)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=gnu11", "-ffp-contract=off",
           "-o", out_path + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out_path + ".tmp", out_path)
    hipcc = os.environ.get("HIPCC") or "/opt/rocm/bin/hipcc"
    cmd = [hipcc, "-O3", "-fPIC", "-shared", "--offload-arch=gfx950", "-ffp-contract=off",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "-o", gpu_out_path + ".tmp", _GPU_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for gen_gpu.hip:\n" + r.stderr)
    os.replace(gpu_out_path + ".tmp", gpu_out_path)
    return out_path


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            u32p = ctypes.POINTER(ctypes.c_uint32)
            lib.synth_philox4x32_10.argtypes = [u32p, u32p, u32p]
            lib.synth_philox4x32_10.restype = None
            lib.synth_bits64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
            lib.synth_bits64.restype = ctypes.c_uint64
            lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
            lib.synth_normal.restype = ctypes.c_double
            lib.synth_centers.argtypes = [ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_double, ctypes.POINTER(ctypes.c_double)]
            lib.synth_centers.restype = None
            lib.synth_points.argtypes = [ctypes.c_uint64, ctypes.POINTER(ctypes.c_double), ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                         ctypes.POINTER(ctypes.c_double), ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(ctypes.c_int32)]
            lib.synth_points.restype = ctypes.c_int
            lib.synth_num_threads.argtypes = []
            lib.synth_num_threads.restype = ctypes.c_int
            _lib = lib
        return _lib


def _load_gpu():
    global _gpu_lib
    with _lock:
        if _gpu_lib is None:
            if not os.path.exists(_GPU_LIB_PATH):
                raise RuntimeError(f"{_GPU_LIB_PATH} is not built (run synth.build())")
            lib = ctypes.CDLL(_GPU_LIB_PATH)
            lib.synth_points_device.argtypes = [ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int,
                                                ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                                ctypes.c_void_p]
            lib.synth_points_device.restype = ctypes.c_int
            _gpu_lib = lib
        return _gpu_lib


def philox4x32_10(ctr, key):
    """The raw Philox4x32-10 block (for known-answer tests)."""
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    _load().synth_philox4x32_10(c, k, o)
    return list(o)


def normals(seed: int, tag: int, n: int) -> np.ndarray:
    lib = _load()
    return np.array([lib.synth_normal(seed, tag, i) for i in range(n)])


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # storage type of X: "f32" or "bf16"
    N: int
    D: int
    K: int
    iters: int
    M: int                # mixture components
    center_scale: float   # centres ~ center_scale * N(0, I)
    sigma: float          # per-coordinate noise std
    kind: int = 0         # 0 Gaussian mixture, 1 unit-normalised ("vMF-like")
    zipf_s: float = 0.0   # 0 = equal weights
    init: str = "sample"  # "first" K points or K points "sample"d without replacement
    seed: int = 0
    chunk_rows: int = 0   # >0: X lives in pinned host memory, streamed in chunks of this many rows
    description: str = field(default="", compare=False)

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "c1": Workload("c1", "f32", 16_384, 32, 64, 10, 64, 2.0, 1.0, init="first", seed=1,
                   description="fp32 N=16384 D=32 K=64, 10 it, 64-component Gaussian mixture"),
    "c2": Workload("c2", "bf16", 1_048_576, 128, 1_024, 20, 1_024, 1.0, 0.3, seed=2,
                   description="bf16 N=1048576 D=128 K=1024, 20 it, 1024-component Gaussian mixture"),
    "c3": Workload("c3", "bf16", 1_048_576, 128, 65_536, 5, 8_192, 1.0, 0.1, kind=1, seed=3,
                   description="bf16 N=1048576 D=128 K=65536, 5 it, 8192 unit-sphere clusters"),
    "c4": Workload("c4", "bf16", 8_388_608, 64, 4_096, 10, 4_096, 2.0, 1.0, zipf_s=1.2, seed=4,
                   description="bf16 N=8388608 D=64 K=4096, 10 it, Zipf(1.2) component weights"),
    "c5": Workload("c5", "bf16", 1_000_000_000, 64, 4_096, 3, 4_096, 2.0, 1.0, seed=5,
                   chunk_rows=64 * 2**20,
                   description="bf16 N=1e9 D=64 K=4096, 3 it, streamed from host memory"),
}


def zipf_cdf(M: int, s: float) -> np.ndarray:
    w = (np.arange(1, M + 1, dtype=np.float64)) ** (-s)
    c = np.cumsum(w)
    c /= c[-1]
    c[-1] = 1.0
    return c


def centers(w: Workload) -> np.ndarray:
    out = np.empty((w.M, w.D), dtype=np.float64)
    _load().synth_centers(w.seed, w.M, w.D, w.kind, w.center_scale,
                          out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def points_into(w: Workload, out_ptr: int, row0: int, nrows: int, cent: np.ndarray | None = None,
                comp: np.ndarray | None = None) -> None:
    """Write rows [row0, row0+nrows) of X into raw memory at ``out_ptr`` (host memory)."""
    cent = centers(w) if cent is None else cent
    cdf = zipf_cdf(w.M, w.zipf_s) if w.zipf_s > 0 else None
    rc = _load().synth_points(
        w.seed, cent.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), w.M, w.D, w.kind, w.sigma,
        None if cdf is None else cdf.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        0 if w.dtype == "f32" else 1, ctypes.c_void_p(out_ptr), row0, nrows,
        None if comp is None else comp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    if rc != 0:
        raise ValueError("synth_points failed")


def points(w: Workload, row0: int = 0, nrows: int | None = None, with_components: bool = False):
    """Rows of X as numpy: float32 for "f32", raw bfloat16 bits (uint16) for "bf16"."""
    nrows = w.N - row0 if nrows is None else nrows
    out = np.empty((nrows, w.D), dtype=np.float32 if w.dtype == "f32" else np.uint16)
    comp = np.empty(nrows, dtype=np.int32) if with_components else None
    points_into(w, out.ctypes.data, row0, nrows, comp=comp)
    return (out, comp) if with_components else out


class DeviceGenerator:
    """Rows of a workload generated on a ROCm device (same definition as ``points``).

    ``fill(out, row0)`` writes rows [row0, row0 + len(out)) into the device
    tensor ``out`` (float32 for "f32", bfloat16 for "bf16") on the current
    stream of its device.
    """

    def __init__(self, w: Workload, device):
        import torch
        self.w = w
        self.device = torch.device(device)
        self.cent = torch.from_numpy(centers(w)).to(self.device)
        self.cdf = torch.from_numpy(zipf_cdf(w.M, w.zipf_s)).to(self.device) if w.zipf_s > 0 else None

    def fill(self, out, row0: int, comp=None) -> None:
        import torch
        w = self.w
        want = torch.float32 if w.dtype == "f32" else torch.bfloat16
        if out.device != self.device or out.dtype != want or not out.is_contiguous() or out.shape[-1] != w.D:
            raise ValueError("out must be a contiguous (rows, D) tensor of the workload's dtype on the device")
        nrows = out.numel() // w.D
        if row0 < 0 or row0 + nrows > w.N:
            raise ValueError("rows out of range")
        if comp is not None and (comp.dtype != torch.int32 or comp.numel() != nrows or comp.device != self.device):
            raise ValueError("comp must be an int32 device tensor with one entry per row")
        stream = torch.cuda.current_stream(self.device).cuda_stream
        rc = _load_gpu().synth_points_device(
            w.seed, self.cent.data_ptr(), w.M, w.D, w.kind, w.sigma,
            None if self.cdf is None else self.cdf.data_ptr(), 0 if w.dtype == "f32" else 1,
            out.data_ptr(), row0, nrows, None if comp is None else comp.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"synth_points_device failed ({rc})")


def host_points(w: Workload, device, pinned: bool = False, block_rows: int = 1 << 24, progress=None):
    """All of X in host memory (torch tensor, pinned or pageable), generated on ``device`` block by block.

    For the out-of-core workload: 10^9 rows are generated in seconds on the GPU
    and copied down, instead of minutes on the host cores.  ``progress(rows_done)``
    is called after every block.
    """
    import torch
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    Xh = torch.empty((w.N, w.D), dtype=dt, pin_memory=pinned)
    gen = DeviceGenerator(w, device)
    buf = torch.empty((min(block_rows, w.N), w.D), dtype=dt, device=gen.device)
    for r0 in range(0, w.N, block_rows):
        nr = min(block_rows, w.N - r0)
        gen.fill(buf[:nr], r0)
        Xh[r0:r0 + nr].copy_(buf[:nr])
        if progress is not None:
            progress(r0 + nr)
    torch.cuda.synchronize(gen.device)
    return Xh


def as_numpy_rows(Xh) -> np.ndarray:
    """Stored values of a host torch X as numpy (float32, or uint16 bfloat16 bits), without copying."""
    import torch
    if Xh.dtype == torch.bfloat16:
        return Xh.view(torch.int16).numpy().view(np.uint16)
    return Xh.numpy()


def sample_indices(seed: int, N: int, K: int) -> np.ndarray:
    """K distinct indices from [0, N), Floyd's sampling algorithm driven by Philox bits."""
    lib = _load()
    chosen: list[int] = []
    seen: set[int] = set()
    n = 0
    for j in range(N - K, N):
        t = int(((lib.synth_bits64(seed, n) * (j + 1)) >> 64))  # uniform in [0, j]
        n += 1
        if t in seen:
            t = j
        seen.add(t)
        chosen.append(t)
    return np.array(chosen, dtype=np.int64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def init_indices(w: Workload) -> np.ndarray:
    if w.init == "first":
        return np.arange(w.K, dtype=np.int64)
    return sample_indices(w.seed, w.N, w.K)


def init_centroids(w: Workload, X: np.ndarray | None = None) -> np.ndarray:
    """C0 (K x D float32): the chosen rows of X, widened exactly to fp32."""
    idx = init_indices(w)
    if X is not None:
        rows = X[idx]
    else:  # regenerate the chosen rows one by one (index-addressable generator)
        cent = centers(w)
        rows = np.empty((len(idx), w.D), dtype=np.float32 if w.dtype == "f32" else np.uint16)
        for r, i in enumerate(idx):
            points_into(w, rows[r:].ctypes.data, int(i), 1, cent=cent)
    return rows.astype(np.float32) if w.dtype == "f32" else bf16_bits_to_f32(rows)


def num_threads() -> int:
    return int(_load().synth_num_threads())
