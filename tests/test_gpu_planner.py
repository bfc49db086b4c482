"""Every alternative plan the planner study times is a correct plan: kmeans_fit under each single override of the
planner (kernel layout, cold argmax, split sweep, segment tiles, radix items, small-codebook update) against the
fp64 oracle, iteration by iteration, on shapes where the override changes the plan."""
import pytest
import torch

import means_clustering_amd as km
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [("c2", dict(N=60_000, K=1024)), ("c4", dict(N=120_000, K=4096)), ("c3", dict(N=20_000, K=9000)),
         ("c1", dict())]
OVERRIDES = [("assign_kernel", 1), ("assign_kernel", 2), ("assign_fold", 1), ("assign_fold", 2),
             ("assign_split", 1), ("assign_split", 3), ("reduce_tile", 1), ("reduce_tile", 2),
             ("radix_items", 8), ("radix_items", 16), ("radix_items", 32), ("small_update", 1)]


@pytest.mark.parametrize("override", OVERRIDES, ids=lambda o: f"{o[0]}={o[1]}")
@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_alternative_plan_matches_oracle(case, override):
    name, kw = case
    w = synth.WORKLOADS[name].scaled(**kw)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    static = km.plan_describe(w.N, w.D, w.K, tdt)
    km.plan_override(*override)
    try:
        plan = km.plan_describe(w.N, w.D, w.K, tdt)
        if plan == static:
            pytest.skip("the override does not change this shape's plan")
        print(f"[planner] {name} {override}: {plan}", flush=True)
        Xn = synth.points(w)
        C0 = synth.init_centroids(w, Xn)
        X = parity.x_from_numpy(Xn, w.dtype, DEV)
        C = torch.from_numpy(C0).to(DEV)
        C2, a2, n2, _ = km.fit(X, C, 2)  # cold then warm
        for t in range(2):
            C_prev = C.cpu().numpy()
            C, a, n, _ = km.fit(X, C, 1)
            torch.cuda.synchronize()
            an = a.cpu().numpy()
            parity.check_assign(Xn, w.dtype, C_prev, an, label=f"{name} {override} it{t}")
            parity.check_update(Xn, w.dtype, an, C_prev, C.cpu().numpy(), n.cpu().numpy(),
                                label=f"{name} {override} it{t}")
        assert torch.equal(C, C2) and torch.equal(a, a2) and torch.equal(n, n2), "2 calls != one call of 2"
    finally:
        km.plan_override(override[0], 0)
