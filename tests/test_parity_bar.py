"""The comparison bar itself (CPU only): each rule of tests/parity.py fails on a result that breaks it.

The "GPU" results here are fabricated from the oracle's own answers with planted deviations, so the helper that
every GPU parity test relies on is shown to catch: a mismatch beyond the near-tie gap, near-tie mismatches over
0.01% of the points, more ties at the kernel's precision than their own cap, counts that are not the histogram,
a changed empty cluster, and centroids beyond the tolerance.
"""
import numpy as np
import pytest

import oracle
from tests import parity


def _ties_case(n_ties=40, n_far=960, seed=0):
    """fp32, D = 1, centroids 0 and 1 and 5: points just above 0.5 (the oracle picks 1 by a gap of a few ulps,
    inside the kernel's fp32 error bound), the rest far from any boundary."""
    rng = np.random.default_rng(seed)
    ulp = np.float32(2.0**-24)
    ties = (np.float32(0.5) + ulp * rng.integers(1, 4, n_ties).astype(np.float32)).astype(np.float32)
    far = rng.choice(np.array([0.1, 0.9, 4.8], dtype=np.float32), n_far)
    X = np.concatenate([ties, far]).reshape(-1, 1).astype(np.float32)
    C = np.array([[0.0], [1.0], [5.0]], dtype=np.float64)
    return X, C, n_ties


def test_exact_answer_passes():
    X, C, _ = _ties_case()
    a_ref, _, _ = oracle.assign(X, C, "f32")
    nm, _ = parity.check_assign(X, "f32", C, a_ref, label="exact")
    assert nm == 0


def test_mismatch_beyond_gap_fails():
    X, C, n_ties = _ties_case()
    a_ref, _, _ = oracle.assign(X, C, "f32")
    a = a_ref.copy()
    far = n_ties + int(np.nonzero(X[n_ties:, 0] == np.float32(0.1))[0][0])
    a[far] = 2  # a far point sent to the wrong centroid
    with pytest.raises(AssertionError, match="beyond the near-tie gap"):
        parity.check_assign(X, "f32", C, a, label="planted", min_near_ties=5, precision_ties=True)


def test_near_ties_over_the_fraction_fail():
    X, C, n_ties = _ties_case()
    a_ref, _, _ = oracle.assign(X, C, "f32")
    a = a_ref.copy()
    a[:2] = 0  # two near-tie flips in 1,000 points: over 0.01%
    with pytest.raises(AssertionError, match="near-tie mismatches"):
        parity.check_assign(X, "f32", C, a, label="planted")
    parity.check_assign(X, "f32", C, a, label="allowed", min_near_ties=2)


def test_precision_ties_are_capped():
    X, C, n_ties = _ties_case()
    a_ref, d1, d2 = oracle.assign(X, C, "f32")
    assert (a_ref[:n_ties] == 1).all()
    cap = max(parity.MAX_PRECISION_TIES, int(parity.MAX_PRECISION_TIE_SHARE * n_ties))  # the 40 points are the ties
    a = a_ref.copy()
    a[:cap] = 0  # exactly the cap: accepted, not counted against 0.01%
    parity.check_assign(X, "f32", C, a, label="at cap", precision_ties=True)
    a[: cap + 1] = 0  # one more: a kernel deciding most of its near-ties the other way fails
    with pytest.raises(AssertionError, match="at the kernel's precision"):
        parity.check_assign(X, "f32", C, a, label="over cap", precision_ties=True)


def _update_case():
    X, C, _ = _ties_case()
    C = np.array([[0.0], [1.0], [5.0], [100.0]], dtype=np.float64)  # centroid 3 stays empty
    a, _, _ = oracle.assign(X, C, "f32")
    C_new, n = oracle.update(X, a, 4, C, "f32")
    return X, C, a, C_new.astype(np.float32), n.astype(np.int32)


def test_update_rules():
    X, C, a, C_new, n = _update_case()
    assert n[3] == 0
    parity.check_update(X, "f32", a, C, C_new, n, label="exact")
    bad = n.copy()
    bad[0] += 1
    bad[1] -= 1
    with pytest.raises(AssertionError, match="counts"):
        parity.check_update(X, "f32", a, C, C_new, bad, label="counts")
    moved = C_new.copy()
    moved[3, 0] = np.nextafter(np.float32(100.0), np.float32(200.0))
    with pytest.raises(AssertionError, match="empty clusters"):
        parity.check_update(X, "f32", a, C, moved, n, label="empty")
    off = C_new.copy()
    off[1, 0] *= np.float32(1.0 + 1e-3)
    with pytest.raises(AssertionError, match="centroid error"):
        parity.check_update(X, "f32", a, C, off, n, label="tolerance")
