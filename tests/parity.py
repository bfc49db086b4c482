"""Comparison of the HIP library's results with the fp64 oracle (test helper).

The bar (the library's stated contract for exact Lloyd K-Means):
  * assignments: a point may differ from the oracle only if the oracle's gap
    between its best and second-best distance is at most
    1e-4 * (||x||^2 + 1), and such near-tie differences stay below 0.01% of
    the points (both sides score the same rounded centroids);
  * counts: equal to the histogram of the library's own assignments, and to
    the oracle's counts whenever the assignments agree;
  * centroids: the oracle recomputes the update from the library's own
    assignments (so a near-tie flip cannot leak into the comparison); the
    error max_k ||c_k - c*_k||_inf / max(||c*_k||_inf, 1e-6) must stay within
    1e-4 for fp32 X and 2e-3 for 16-bit X; empty clusters match bit for bit.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

CENTROID_TOL = {"f32": 1e-4, "bf16": 2e-3, "f16": 2e-3}
GAP_REL = 1e-4
MAX_NEAR_TIE_FRAC = 1e-4
# ties at the kernel's own fp32 precision (see check_assign): not held to the 0.01% bar, but still bounded, so
# that a kernel deciding most of its near-ties the other way fails: at most half of the points whose oracle gap
# lies within that precision bound (never fewer than 8).  A fixed count would not do: with dense centroids (D = 1,
# thousands of centroids on a line) nearly every point lies within fp32 resolution of a tie.
MAX_PRECISION_TIES = 8
MAX_PRECISION_TIE_SHARE = 0.5


def x_to_numpy(X: torch.Tensor):
    """Stored values of a device X as numpy + the oracle's storage name."""
    if X.dtype == torch.float32:
        return X.cpu().numpy(), "f32"
    if X.dtype == torch.bfloat16:
        return X.cpu().view(torch.int16).numpy().view(np.uint16), "bf16"
    if X.dtype == torch.float16:
        return X.cpu().numpy(), "f16"
    raise TypeError(X.dtype)


def x_from_numpy(Xn: np.ndarray, xdtype: str, device) -> torch.Tensor:
    if xdtype == "bf16":
        return torch.from_numpy(Xn.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(Xn).to(device)


def check_assign(Xn, xdtype, C_state, a_gpu, rows=None, label="", min_near_ties=0, precision_ties=False):
    """Assignment of rows `rows` (all if None) against the oracle on the same centroid state.

    min_near_ties: near-tie mismatches always allowed, whatever 0.01% of the points comes to (small problems,
    where 0.01% is less than one point; the gap bound on every mismatch still holds).
    precision_ties: a mismatch whose oracle gap lies within the fp32 error of the kernel's score itself,
    (D + 2) * 2^-22 * (||x||^2 + ||c_oracle||^2 + ||c_gpu||^2) (fp32 accumulation of x.c - ||c||^2/2, two
    scores, distances twice the score), is a tie at the kernel's precision and is not counted against the
    0.01%: both sides take the decision in their own precision.  The gap bound still holds for it, and such
    ties are held to their own cap: at most half of the points within that bound (MAX_PRECISION_TIE_SHARE),
    never fewer than MAX_PRECISION_TIES."""
    Xs = Xn if rows is None else Xn[rows]
    a_ref, d1, d2 = oracle.assign(Xs, np.asarray(C_state, dtype=np.float64), xdtype)
    a_gpu = np.asarray(a_gpu if rows is None else a_gpu[rows])
    mism = np.nonzero(a_gpu != a_ref)[0]
    xn = (oracle.decode(Xs, xdtype) ** 2).sum(axis=1)
    gap = d2 - d1
    allowed = gap[mism] <= GAP_REL * (xn[mism] + 1.0)
    assert allowed.all(), (f"{label}: {int((~allowed).sum())} mismatches beyond the near-tie gap, e.g. rows "
                           f"{mism[~allowed][:5].tolist()} gpu {a_gpu[mism[~allowed][:5]].tolist()} "
                           f"oracle {a_ref[mism[~allowed][:5]].tolist()} gap {gap[mism[~allowed][:5]].tolist()}")
    counted = mism
    if precision_ties and len(mism):
        cn = (oracle.quantize(np.asarray(C_state, dtype=np.float64), xdtype) ** 2).sum(axis=1)
        D = Xs.shape[1]
        eps = (D + 2) * 2.0**-22 * (xn[mism] + cn[a_ref[mism]] + cn[a_gpu[mism]])
        counted = mism[gap[mism] > eps]
        n_prec = len(mism) - len(counted)
        # points whose own gap lies within the bound (the second-best centroid's norm taken as the best one's)
        near = int((gap <= (D + 2) * 2.0**-22 * (xn + 2.0 * cn[a_ref])).sum())
        if n_prec:
            print(f"[parity] {label}: {n_prec} tie(s) at the kernel's precision among {near} such points of "
                  f"{len(Xs)}", flush=True)
        assert n_prec <= max(MAX_PRECISION_TIES, MAX_PRECISION_TIE_SHARE * near), \
            f"{label}: {n_prec} mismatches at the kernel's precision, {near} points within it, of {len(Xs)}"
    assert len(counted) <= max(MAX_NEAR_TIE_FRAC * len(Xs), min_near_ties) + 1e-9 or len(counted) == 0, \
        f"{label}: {len(counted)} near-tie mismatches of {len(Xs)} points"
    return len(mism), a_ref


def check_objective(Xn, xdtype, C_state, a_gpu, J_gpu, label=""):
    """The objective J = sum of the kernel's per-point distances max(||x||^2 - 2 s, 0) (fp32 expanded form,
    s = x.c - ||c||^2/2) against the oracle's fp64 direct distances to the same rounded centroids.  Allowed:
    1e-5 relative, plus per point the fp32 error of the expanded form itself, (D + 2) * 2^-22 *
    (||x||^2 + ||c||^2) (cancellation when the distance is small against the norms), plus the oracle gap of
    every point the kernel assigned elsewhere (a near-tie choice of another centroid)."""
    a_ref, d1, d2 = oracle.assign(Xn, np.asarray(C_state, dtype=np.float64), xdtype)
    a_gpu = np.asarray(a_gpu)
    xn = (oracle.decode(Xn, xdtype) ** 2).sum(axis=1)
    cn = (oracle.quantize(np.asarray(C_state, dtype=np.float64), xdtype) ** 2).sum(axis=1)
    D = Xn.shape[1]
    J_ref = float(d1.sum())
    tol = 1e-5 * J_ref + 1e-6 + float(((D + 2) * 2.0**-22 * (xn + cn[a_ref])).sum())
    tol += float((d2 - d1)[a_gpu != a_ref].sum())
    assert abs(float(J_gpu) - J_ref) <= tol, f"{label}: objective {float(J_gpu)!r} vs {J_ref!r} (allowed {tol:.3e})"


def centroid_error(C_gpu, C_ref):
    C_gpu = np.asarray(C_gpu, dtype=np.float64)
    C_ref = np.asarray(C_ref, dtype=np.float64)
    num = np.abs(C_gpu - C_ref).max(axis=1)
    den = np.maximum(np.abs(C_ref).max(axis=1), 1e-6)
    return float((num / den).max()) if len(num) else 0.0


def check_update(Xn, xdtype, a_gpu, C_prev, C_gpu, counts_gpu, label=""):
    """Update from the library's own assignments against the oracle's update from the same assignments."""
    K = C_prev.shape[0]
    C_ref, n_ref = oracle.update(Xn, np.asarray(a_gpu, dtype=np.int32), K, np.asarray(C_prev, dtype=np.float64),
                                 xdtype)
    a = np.asarray(a_gpu)
    valid = (a >= 0) & (a < K)
    assert np.array_equal(np.asarray(counts_gpu), np.bincount(a[valid], minlength=K)), f"{label}: counts"
    assert np.array_equal(np.asarray(counts_gpu), n_ref), f"{label}: counts vs oracle"
    empty = n_ref == 0
    assert np.array_equal(np.asarray(C_gpu)[empty], np.asarray(C_prev, dtype=np.float32)[empty]), \
        f"{label}: empty clusters must keep their centroid bit for bit"
    err = centroid_error(np.asarray(C_gpu)[~empty], C_ref[~empty])
    assert err <= CENTROID_TOL[xdtype], f"{label}: centroid error {err:.3e} > {CENTROID_TOL[xdtype]}"
    return err
