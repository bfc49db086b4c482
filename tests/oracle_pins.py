"""Pins for the fp64 oracle: checks against what mathematics fixes, not against itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError on a
violation.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes and requires every mistake to be caught by at least one pin.

What pins what (Lloyd's algorithm, which the Flash-KMeans page keeps exact --
technical summary section 2 opening and section 3):
  distance + argmin   exact rational brute force on dyadic inputs; enumeration
                      of all K^N assignments; scipy cdist argmin; special cases
  tie rule            constructed exact ties, duplicated centroids
  second distance     brute force second-smallest distance
  update / mean       exact rational means (IEEE division of an exact sum is
                      correctly rounded); fsum column mean; symmetric clouds
  empty rule          far centroid, duplicated centroids, the X={1/2} case
  trajectory          hand-worked 1-D Lloyd run (tests/golden/trajectory_1d.txt)
  objective           monotone in exact arithmetic; rigorous bound in fp32 state
  invariances         point/dimension permutation, dyadic translation, 2^k scale
  rounding / decode   torch's and numpy's independent conversions
  library             scikit-learn Lloyd when no cluster empties
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _dyadic(rng, shape, lo=-4, hi=4, denom=4):
    return rng.integers(lo * denom, hi * denom + 1, size=shape).astype(np.float64) / denom


def _frac_rows(A):
    return [[Fraction(float(v)) for v in row] for row in A]


# ---------------------------------------------------------------- assignment

def pin_assign_brute(O):
    """Exact argmin (lowest index on ties) and exact distances on dyadic inputs."""
    rng = np.random.default_rng(11)
    for trial in range(60):
        N, K, D = rng.integers(1, 13), rng.integers(1, 6), rng.integers(1, 4)
        X = _dyadic(rng, (N, D), denom=2)  # coarse grid => many exact ties
        C = _dyadic(rng, (K, D), denom=2)
        a, d1, d2 = O.assign(X, C, "f64")
        ea, ed = brute.assign(_frac_rows(X), _frac_rows(C))
        assert list(a) == ea, (trial, list(a), ea)
        assert [Fraction(float(v)) for v in d1] == ed, trial


def pin_second_distance(O):
    """d2 = smallest distance to any centroid other than the assigned one."""
    rng = np.random.default_rng(12)
    for trial in range(40):
        N, K, D = rng.integers(1, 10), rng.integers(1, 6), rng.integers(1, 4)
        X = _dyadic(rng, (N, D), denom=2)
        C = _dyadic(rng, (K, D), denom=2)
        a, d1, d2 = O.assign(X, C, "f64")
        for i in range(N):
            ds = [brute.sqdist(_frac_rows(X)[i], c) for c in _frac_rows(C)]
            others = [d for k, d in enumerate(ds) if k != a[i]]
            want = min(others) if others else math.inf
            assert d2[i] == float(want), (trial, i)


def pin_enumeration(O):
    """Lexicographically smallest cost minimiser over all 3^6 assignments == pointwise argmin."""
    rng = np.random.default_rng(13)
    for trial in range(4):
        X = _dyadic(rng, (6, 2), denom=1)
        C = _dyadic(rng, (3, 2), denom=1)
        if trial == 0:
            C[2] = C[0]  # duplicated centroid: index 2 must never be chosen
        a, _, _ = O.assign(X, C, "f64")
        ea, cost = brute.enumerate_min_assignment(_frac_rows(X), _frac_rows(C))
        assert list(a) == ea, (trial, list(a), ea)


def pin_assign_cdist(O):
    """scipy's pairwise squared distances + first-occurrence argmin, away from near-ties."""
    from scipy.spatial.distance import cdist
    rng = np.random.default_rng(14)
    for (N, K, D) in [(500, 37, 11), (300, 5, 64), (64, 200, 3)]:
        X = rng.standard_normal((N, D))
        C = rng.standard_normal((K, D))
        a, d1, d2 = O.assign(X, C, "f64")
        dist = cdist(X, C, "sqeuclidean")
        ref = np.argmin(dist, axis=1)
        srt = np.sort(dist, axis=1)
        clear = (srt[:, 1] - srt[:, 0]) > 1e-9 if K > 1 else np.ones(N, bool)
        assert np.array_equal(a[clear], ref[clear])
        np.testing.assert_allclose(d1, dist[np.arange(N), a], rtol=1e-12, atol=1e-12)


def pin_assign_special(O):
    """K = 1; C = X (distinct rows); exact ties; duplicated centroids."""
    rng = np.random.default_rng(15)
    X = rng.standard_normal((50, 7))
    a, d1, d2 = O.assign(X, X[:1], "f64")
    assert (a == 0).all() and np.isinf(d2).all()
    a, d1, _ = O.assign(X, X, "f64")
    assert np.array_equal(a, np.arange(50)) and (d1 == 0).all()
    a, d1, d2 = O.assign(np.array([[0.5]]), np.array([[0.0], [1.0]]), "f64")
    assert a[0] == 0 and d1[0] == 0.25 and d2[0] == 0.25
    C = rng.standard_normal((10, 7))
    C[7] = C[3]
    a, _, _ = O.assign(X, C, "f64")
    assert not (a == 7).any()
    # three-way tie at the origin: centroids on the unit axes and their negatives
    a, _, _ = O.assign(np.zeros((1, 2)), np.array([[0, 1.0], [1, 0], [0, -1], [-1, 0]]), "f64")
    assert a[0] == 0


def pin_nan_rule(O):
    """A NaN distance never wins; an all-NaN row keeps index 0."""
    X = np.array([[np.nan, 0.0], [1.0, 1.0]])
    C = np.array([[5.0, 5.0], [1.0, 1.0]])
    a, _, _ = O.assign(X, C, "f64")
    assert a[0] == 0 and a[1] == 1


# ------------------------------------------------------------------- update

def pin_update_exact(O):
    """Means equal the correctly rounded exact rational mean; counts exact."""
    rng = np.random.default_rng(21)
    for trial in range(40):
        N, K, D = rng.integers(1, 30), rng.integers(1, 7), rng.integers(1, 5)
        X = _dyadic(rng, (N, D), denom=8)
        a = rng.integers(0, K, size=N).astype(np.int32)
        Cp = rng.standard_normal((K, D))
        Cn, counts = O.update(X, a, K, Cp, "f64")
        EC, ecounts = brute.update(_frac_rows(X), list(a), _frac_rows(Cp))
        assert list(counts) == ecounts, trial
        for k in range(K):
            for j in range(D):
                assert Cn[k, j] == float(EC[k][j]), (trial, k, j)


def pin_update_column_mean(O):
    """K = 1: the centroid is the column mean; compare with math.fsum (correctly rounded sum)."""
    rng = np.random.default_rng(22)
    X = rng.standard_normal((2000, 9)) * 3.0
    Cn, counts = O.update(X, np.zeros(2000, np.int32), 1, np.zeros((1, 9)), "f64")
    assert counts[0] == 2000
    for j in range(9):
        ref = math.fsum(X[:, j]) / 2000
        assert abs(Cn[0, j] - ref) <= 1e-13 * max(1.0, abs(ref)), j


def pin_update_duplicated_data(O):
    """Duplicating every point doubles the counts and leaves the means unchanged."""
    rng = np.random.default_rng(23)
    X = _dyadic(rng, (40, 3), denom=8)
    a = rng.integers(0, 5, size=40).astype(np.int32)
    Cp = rng.standard_normal((5, 3))
    C1, n1 = O.update(X, a, 5, Cp, "f64")
    C2, n2 = O.update(np.concatenate([X, X]), np.concatenate([a, a]), 5, Cp, "f64")
    assert np.array_equal(2 * n1, n2)
    assert np.array_equal(C1, C2)


def pin_empty_rule(O):
    """An empty cluster keeps its previous centroid bit for bit."""
    X = np.array([[0.5]])
    C0 = np.array([[0.0], [1.0]], dtype=np.float32)
    C, a, counts, J = O.fit(X, C0, 1, contract=False, xdtype="f64")
    assert list(a) == [0] and list(counts) == [1, 0]
    assert C[0, 0] == 0.5 and C[1, 0] == 1.0
    rng = np.random.default_rng(24)
    X = rng.standard_normal((200, 4))
    Cp = rng.standard_normal((6, 4))
    Cp[5] = [1e3, -1e3, 1e3, np.float64(np.float32(0.1))]
    a, _, _ = O.assign(X, Cp, "f64")
    assert not (a == 5).any()
    Cn, counts = O.update(X, a, 6, Cp, "f64")
    assert counts[5] == 0 and np.array_equal(Cn[5], Cp[5])
    # out-of-range assignments are ignored by the update
    Cn2, counts2 = O.update(X, np.where(a == 0, 99, a).astype(np.int32), 6, Cp, "f64")
    assert counts2[0] == 0 and np.array_equal(Cn2[0], Cp[0])


def pin_duplicated_centroids_stay_empty(O):
    """With c3 == c7, index 7 never wins the first assignment, so after one
    iteration it is empty and unchanged (c3 then moves, so later iterations may
    hand points to c7: the pin is about one iteration only)."""
    rng = np.random.default_rng(25)
    X = rng.standard_normal((300, 3)).astype(np.float32)
    C0 = X[:10].copy()
    C0[7] = C0[3]
    C, a, counts, J = O.fit(X, C0, 1, contract=True)
    assert counts[3] > 0 and counts[7] == 0 and np.array_equal(C[7], C0[7].astype(np.float64))


# --------------------------------------------------------------- trajectory

def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals


def pin_trajectory_1d(O):
    g = _read_golden("trajectory_1d.txt")
    fr = lambda s: [Fraction(t.strip()) for t in s.split(",")]
    X = np.array([[float(v)] for v in fr(g["X"])])
    C0 = np.array([[float(v)] for v in fr(g["C0"])], dtype=np.float32)
    for T in (1, 2, 3):
        C, a, counts, J = O.fit(X, C0, T, contract=False, xdtype="f64")
        assert list(a) == [int(v) for v in fr(g[f"a{T-1}"])], T
        assert [c[0] for c in C] == [float(v) for v in fr(g[f"C{T}"])], T
        assert list(J) == [float(fr(g[f"J{t}"])[0]) for t in range(T)], T
    # the exact rational driver agrees with the golden file as well
    EC, ea, _, EJ = brute.fit([[v] for v in fr(g["X"])], [[v] for v in fr(g["C0"])], 3)
    assert [c[0] for c in EC] == fr(g["C3"]) and EJ == [fr(g[f"J{t}"])[0] for t in range(3)]
    # J_t is the objective of assignment t against the centroids it was made with (C^t), exactly
    Xr = [[v] for v in fr(g["X"])]
    for t in range(3):
        Ct = [[v] for v in fr(g[f"C{t}"])]
        assert brute.objective(Xr, Ct, [int(v) for v in fr(g[f"a{t}"])]) == fr(g[f"J{t}"])[0], t


def pin_symmetric_clouds(O):
    g = _read_golden("symmetric_clouds.txt")
    cen = np.array([[float(t) for t in p.split()] for p in g["centers"].split(";")])
    off = np.array([[float(t) for t in p.split()] for p in g["offsets"].split(";")])
    X = (cen[:, None, :] + off[None, :, :]).reshape(-1, 2)
    perm = np.random.default_rng(26).permutation(len(X))
    X = X[perm]
    C, a, counts, J = O.fit(X, cen.astype(np.float32), 3, contract=True, xdtype="f64")
    assert np.array_equal(C, cen) and list(counts) == [4, 4, 4]
    assert list(J) == [float(g["J"])] * 3


# ---------------------------------------------------------------- objective

def pin_objective_monotone(O):
    """Pure mode: J_{t+1} <= J_t (Lloyd's monotonicity), on several random mixtures."""
    rng = np.random.default_rng(31)
    for trial in range(6):
        N, K, D = 400, int(rng.integers(2, 20)), int(rng.integers(1, 8))
        X = rng.standard_normal((N, D)) + 3 * rng.standard_normal((N, 1))
        C0 = X[rng.choice(N, K, replace=False)].astype(np.float32)
        _, _, _, J = O.fit(X, C0, 10, contract=False, xdtype="f64")
        assert np.all(np.diff(J) <= 1e-9 * J[:-1]), (trial, J)


def pin_objective_contract_bound(O):
    """fp32 centroid state: J_{t+1} <= J_t + sum_k n_k |delta_k|^2, delta = fp32 rounding of the mean."""
    rng = np.random.default_rng(32)
    X = (rng.standard_normal((600, 5)) * 2).astype(np.float32)
    C0 = X[:12].copy()
    Cprev = C0.astype(np.float64)
    _, _, _, J = O.fit(X, C0, 8, contract=True)
    for t in range(7):
        a, d1, _ = O.assign(X, Cprev)
        mean, n = O.update(X, a, 12, Cprev)
        nxt = O.round_to(mean, "f32")
        slack = float(np.sum(n[:, None] * (nxt - mean) ** 2))
        assert abs(d1.sum() - J[t]) <= 1e-9 * J[t]
        assert J[t + 1] <= J[t] + slack + 1e-9 * J[t], (t, J)
        Cprev = nxt


def pin_fixed_point(O):
    """Once assignments stop changing, C is fixed; fit from a fixed point returns it unchanged."""
    rng = np.random.default_rng(33)
    X = rng.standard_normal((300, 3)) + np.repeat(np.eye(3) * 8, 100, axis=0)
    C0 = X[[0, 100, 200]].astype(np.float32)
    C, a, _, _ = O.fit(X, C0, 30, contract=True, xdtype="f64")
    C2, a2, _, _ = O.fit(X, C.astype(np.float32), 5, contract=True, xdtype="f64")
    assert np.array_equal(C, C2) and np.array_equal(a, a2)


# --------------------------------------------------------------- invariances

def pin_invariances(O):
    rng = np.random.default_rng(41)
    X = _dyadic(rng, (120, 4), denom=16)
    C0 = X[rng.choice(120, 6, replace=False)].astype(np.float32)
    C, a, n, J = O.fit(X, C0, 4, contract=False, xdtype="f64")
    # point permutation: same centroids (summation order changes: ~1 ulp), permuted labels
    p = rng.permutation(120)
    Cp, ap, npc, _ = O.fit(X[p], C0, 4, contract=False, xdtype="f64")
    np.testing.assert_allclose(Cp, C, rtol=0, atol=1e-12)
    assert np.array_equal(ap, a[p]) and np.array_equal(npc, n)
    # dyadic translation: sums stay exact, so labels are identical and the means
    # move by t up to the one rounding of each division
    t = np.array([0.5, -1.25, 2.0, 0.75])
    Ct, at, _, Jt = O.fit(X + t, (C0 + t).astype(np.float32), 4, contract=False, xdtype="f64")
    assert np.array_equal(at, a)
    np.testing.assert_allclose(Ct, C + t, rtol=0, atol=1e-14)
    np.testing.assert_allclose(Jt, J, rtol=1e-13)
    # scaling by 2^3: bitwise scaled centroids, J scaled by 2^6
    Cs, as_, _, Js = O.fit(X * 8, (C0 * 8).astype(np.float32), 4, contract=False, xdtype="f64")
    assert np.array_equal(as_, a) and np.array_equal(Cs, C * 8) and np.array_equal(Js, J * 64)
    # dimension permutation
    q = np.array([2, 0, 3, 1])
    Cq, aq, _, Jq = O.fit(np.ascontiguousarray(X[:, q]), np.ascontiguousarray(C0[:, q]), 4, contract=False,
                          xdtype="f64")
    assert np.array_equal(aq, a)
    np.testing.assert_allclose(Cq, C[:, q], rtol=0, atol=1e-12)


# -------------------------------------------------------- rounding / decoding

def pin_round_vs_torch(O):
    """RNE to bf16 / fp16 / fp32 against torch's and numpy's own conversions (fp32-exact inputs)."""
    import torch
    rng = np.random.default_rng(51)
    v = (rng.standard_normal(3000) * np.exp2(rng.integers(-30, 30, 3000))).astype(np.float32)
    bits = v.view(np.uint32)
    halfway = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)          # exact bf16 ties
    halfway16 = ((bits & 0xFFFFE000) | 0x1000).view(np.float32)        # exact fp16 ties (13 dropped bits)
    sub = (rng.standard_normal(500) * 2.0 ** -130).astype(np.float32)  # fp32/bf16 subnormals
    sub16 = (rng.standard_normal(500) * 2.0 ** -18).astype(np.float32)  # fp16 subnormal range
    big = np.array([65504.0, 65519.0, 65520.0, 65536.0, -65520.0, 3.3e38, 3.4e38], dtype=np.float32)
    x = np.concatenate([v, halfway, halfway16, sub, sub16, big]).astype(np.float32)
    x64 = x.astype(np.float64)
    ref_bf = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    ref_h = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    got_bf = O.round_to(x64, "bf16")
    got_h = O.round_to(x64, "f16")
    assert np.array_equal(got_bf, ref_bf)
    assert np.array_equal(got_h, ref_h)
    y = rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000))
    assert np.array_equal(O.round_to(y, "f32"), y.astype(np.float32).astype(np.float64))


def pin_decode(O):
    rng = np.random.default_rng(52)
    bits = rng.integers(0, 2**16, 5000, dtype=np.uint64).astype(np.uint16)
    bf = O.decode(bits, "bf16")
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(bf), np.isnan(ref))
    assert np.array_equal(bf[~np.isnan(bf)], ref[~np.isnan(ref)])
    h = O.decode(bits, "f16")
    refh = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(h), np.isnan(refh))
    assert np.array_equal(h[~np.isnan(h)], refh[~np.isnan(refh)])
    f = rng.standard_normal(100).astype(np.float32)
    assert np.array_equal(O.decode(f), f.astype(np.float64))


def pin_quantized_assign(O):
    """16-bit X: the assignment uses the centroids rounded to X's type (checked with torch's rounding)."""
    import torch
    rng = np.random.default_rng(53)
    Xf = rng.standard_normal((60, 5)).astype(np.float32)
    Xb = torch.from_numpy(Xf).to(torch.bfloat16)
    Xbits = Xb.view(torch.int16).numpy().view(np.uint16)
    Xd = Xb.to(torch.float64).numpy()
    C = rng.standard_normal((7, 5)).astype(np.float32)
    Cq = torch.from_numpy(C).to(torch.bfloat16).to(torch.float64).numpy()
    a, d1, _ = O.assign(Xbits, C.astype(np.float64), "bf16")
    ea, ed = brute.assign(_frac_rows(Xd), _frac_rows(Cq))
    assert list(a) == ea and [Fraction(float(v)) for v in d1] == ed
    Xh = Xf.astype(np.float16)
    Ch = C.astype(np.float16).astype(np.float64)
    a, d1, _ = O.assign(Xh, C.astype(np.float64), "f16")
    ea, ed = brute.assign(_frac_rows(Xh.astype(np.float64)), _frac_rows(Ch))
    assert list(a) == ea


# ------------------------------------------------------------------ library

def pin_sklearn(O):
    """scikit-learn's Lloyd from the same init, on data where no cluster ever empties."""
    from sklearn.cluster import KMeans
    rng = np.random.default_rng(61)
    cen = rng.standard_normal((8, 6)) * 6
    X = (cen[rng.integers(0, 8, 2000)] + rng.standard_normal((2000, 6)))
    C0 = X[rng.choice(2000, 8, replace=False)]
    T = 25
    C, a, counts, _ = O.fit(X, C0.astype(np.float32), T, contract=False, xdtype="f64")
    assert counts.min() > 0
    km = KMeans(n_clusters=8, init=C0.astype(np.float32).astype(np.float64), n_init=1, algorithm="lloyd",
                max_iter=T, tol=0.0).fit(X)
    np.testing.assert_allclose(C, km.cluster_centers_, rtol=0, atol=1e-9)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
