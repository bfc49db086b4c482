"""Build the HIP library ``libkmeans_amd.so`` in-tree for gfx950 (MI355X).

Each source is compiled by hipcc to an object under ``_build/`` (in
parallel), then linked into a shared library next to this file.  Every build
compiles from scratch, so a stale library is never mistaken for a fresh one.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libkmeans_amd.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["csrc/flash_assign.hip", "csrc/sort.hip", "csrc/reduce.hip", "csrc/small_k.hip", "csrc/api.cpp",
           "csrc/noalloc.hip"]
# peak probes for the benchmark's roofline denominators, and the ablation
# baselines (libraries of their own, not part of libkmeans_amd.so)
EXTRA_LIBS = [("csrc/peaks.hip", os.path.join(HERE, "libkm_peaks.so"), []),
              ("csrc/ablation.hip", os.path.join(HERE, "libkm_ablation.so"), ["-munsafe-fp-atomics"])]
ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from emitting packed fp32 instructions.
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unused-command-line-argument",
          # MFMA results in ordinary VGPRs: the argmax epilogue reads them without accumulator copies
          "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = _hipcc()
    bdir = os.path.join(ROOT, "_build")
    os.makedirs(bdir, exist_ok=True)

    def compile_one(src, extra=()):
        obj = os.path.join(bdir, os.path.basename(src) + ".o")
        cmd = [hipcc, *CFLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(HERE, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose:
            print(" ".join(cmd))
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(compile_one, src) for src in SOURCES]
        extra = [ex.submit(compile_one, src, flags) for src, _, flags in EXTRA_LIBS]
        objs = [f.result() for f in futs]
        extra_objs = [f.result() for f in extra]
    for (_, path, _), obj in zip(EXTRA_LIBS, extra_objs):
        tmp = path + ".tmp"
        r = subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(tmp, path)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
