"""CPU sanitizer tier (no GPU): the oracle under AddressSanitizer + UndefinedBehaviorSanitizer running every
pin, and the streamed fit's host copy pool under ThreadSanitizer and AddressSanitizer.  (The library's host-side
validation and workspace carving run under ASan + UBSan from tests/test_abi.py.)"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "means_clustering_amd", "csrc")


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"{name} not available")
    return path


def _preload(lib):
    """LD_PRELOAD with the sanitizer runtime first (it must come before every other library); an existing
    preload list is kept after it."""
    old = os.environ.get("LD_PRELOAD", "")
    return lib + (":" + old if old else "")


def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = str(tmp_path / "libkmref_asan.so")
    oracle.build(out_path=lib, extra_flags=["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                                            "-fno-omit-frame-pointer", "-g"])
    env = dict(os.environ, LD_PRELOAD=_preload(_gcc_runtime("libasan.so")), OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, os.path.join(NATIVE, "run_pins_with_oracle.py"), lib], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "pins passed" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_asan_catches_a_planted_overflow(tmp_path):
    """The sanitized oracle build is live: a copy of the oracle with one array a slot too short (planted here,
    on the CPU, in a temporary copy) must be stopped by AddressSanitizer."""
    src = open(os.path.join(ROOT, "oracle", "kmref.c")).read()
    old = "calloc((size_t)K + 1, sizeof(int64_t))"
    assert src.count(old) == 1
    mut = tmp_path / "kmref_short.c"
    mut.write_text(src.replace(old, "calloc((size_t)K, sizeof(int64_t))"))
    lib = str(tmp_path / "libkmref_short.so")
    oracle.build(out_path=lib, src_path=str(mut), extra_flags=["-fsanitize=address", "-fno-omit-frame-pointer", "-g"])
    env = dict(os.environ, LD_PRELOAD=_preload(_gcc_runtime("libasan.so")), OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, os.path.join(NATIVE, "run_pins_with_oracle.py"), lib], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


@pytest.mark.parametrize("sanitizer", ["thread", "address,undefined"])
def test_copy_pool_under_sanitizer(tmp_path, sanitizer):
    exe = str(tmp_path / "copy_pool_stress")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", f"-fsanitize={sanitizer}", "-fno-omit-frame-pointer",
                    "-pthread", "-I", CSRC, os.path.join(NATIVE, "copy_pool_stress.cpp"), "-o", exe], check=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66", ASAN_OPTIONS="halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "copy pool: ok" in r.stdout, r.stdout + r.stderr[-4000:]
    assert "WARNING: ThreadSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
