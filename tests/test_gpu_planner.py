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
             ("radix_items", 8), ("radix_items", 16), ("radix_items", 32), ("small_update", 1),
             ("sort_scan", 1), ("sort_scan", 2), ("sort_rank", 1), ("sort_rank", 2), ("radix_bits", 6),
             ("radix_bits", 8)]


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


def _kfd_largest_cache(domain, bus, dev):
    """Size in bytes of the highest-level cache the KFD topology lists for this GPU (0 if none is found)."""
    import glob
    import os
    for node in glob.glob("/sys/class/kfd/kfd/topology/nodes/*"):
        try:
            with open(os.path.join(node, "properties")) as f:
                props = dict(line.split() for line in f if len(line.split()) == 2)
        except OSError:
            continue
        loc = int(props.get("location_id", -1))
        if int(props.get("simd_count", 0)) <= 0 or int(props.get("domain", -1)) != domain:
            continue
        if (loc >> 8) != bus or ((loc >> 3) & 31) != dev:
            continue
        best = (0, 0)
        for c in glob.glob(os.path.join(node, "caches", "*", "properties")):
            with open(c) as f:
                p = dict(line.split() for line in f if len(line.split()) == 2)
            best = max(best, (int(p.get("level", 0)), int(p.get("size", 0)) * 1024))
        return best[1]
    return 0


def test_device_query_finds_the_last_level_cache():
    """The planner's last-level cache is the highest cache level KFD lists for the device (the Infinity Cache on
    MI355X, listed after hundreds of per-CU L1 entries), never less than the L2 HIP reports; with the topology
    hidden, a gfx950 part's known 256 MiB, else the L2.  The plan description names the source."""
    props = torch.cuda.get_device_properties(0)
    kfd = _kfd_largest_cache(props.pci_domain_id, props.pci_bus_id, props.pci_device_id)
    desc = km.plan_describe(1 << 20, 128, 1024, torch.bfloat16)
    print(f"[planner] device: {desc.split('device: ')[1]}; KFD highest-level cache {kfd >> 20} MiB", flush=True)
    llc_mib = int(desc.split("LLC ")[1].split(" MiB")[0])
    source = desc.split("LLC ")[1].split("(")[1].split(")")[0]
    if kfd > props.L2_cache_size:
        assert source == "KFD topology" and llc_mib == kfd >> 20
    elif props.gcnArchName.startswith("gfx950"):  # topology hidden: the part's known Infinity Cache
        assert source == "gfx950" and llc_mib == 256
    else:
        assert source == "L2" and llc_mib == props.L2_cache_size >> 20
    if kfd:
        # the short segment tiles reach N * G * 16 bytes = half that cache: at D = 64 (G = 8), 2^20 rows on MI355X
        n_half = (kfd // 2) // (8 * 16)
        assert "segment tile 16" in km.plan_describe(n_half, 64, 4096, torch.bfloat16)
        assert "segment tile 128" in km.plan_describe(2 * n_half, 64, 4096, torch.bfloat16)
