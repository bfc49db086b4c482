"""Run every oracle pin against another build of the oracle (a sanitizer build), in this process.

  python tests/native/run_pins_with_oracle.py <path to libkmref build>

Used by tests/test_sanitizers.py, which starts it with the sanitizer runtime preloaded.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from tests import oracle_pins  # noqa: E402

O = oracle.Oracle(oracle.load(sys.argv[1]))
for pin in oracle_pins.ALL_PINS:
    pin(O)
    print(f"pin ok: {pin.__name__}", flush=True)
print(f"all {len(oracle_pins.ALL_PINS)} pins passed")
