"""Run tests/test_abi.py against another build of the library (a sanitizer build), in this process.

  python tests/native/run_with_lib.py <path to libkmeans_amd build> [pytest args...]

Used by tests/test_abi.py, which starts this script in a child process with the
sanitizer runtime preloaded; the child binds the given library in place of the
in-tree one and runs the ABI tests (validation, workspace carving, the
no-allocation entry point's checks), none of which reaches a GPU.
"""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import pytest  # noqa: E402

import means_clustering_amd as km  # noqa: E402

km._lib = km._bind(ctypes.CDLL(sys.argv[1]))
sys.exit(pytest.main([os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-p", "no:cacheprovider", *sys.argv[2:]]))
