"""The device generator writes exactly the bytes of the host generator."""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("name,row0,nrows", [("c1", 0, 16_384), ("c2", 1000, 50_000), ("c3", 7, 20_000),
                                              ("c4", 8_300_000, 88_608), ("c5", 999_900_000, 100_000),
                                              ("c5", 123_456_789, 3)])
def test_device_generator_matches_host(name, row0, nrows):
    w = synth.WORKLOADS[name]
    print(f"[synth] {name} rows {row0}..{row0 + nrows}", flush=True)
    ref, comp_ref = synth.points(w, row0, nrows, with_components=True)
    gen = synth.DeviceGenerator(w, DEV)
    out = torch.empty((nrows, w.D), dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device=DEV)
    comp = torch.empty(nrows, dtype=torch.int32, device=DEV)
    gen.fill(out, row0, comp=comp)
    torch.cuda.synchronize()
    got = out.cpu()
    got = got.numpy() if w.dtype == "f32" else got.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(comp.cpu().numpy(), comp_ref)
    diff = np.nonzero((got.view(np.uint32) if w.dtype == "f32" else got) !=
                      (ref.view(np.uint32) if w.dtype == "f32" else ref))
    assert len(diff[0]) == 0, f"{len(diff[0])} values differ, first at {diff[0][:3]}, {diff[1][:3]}"


@pytest.mark.parametrize("pinned", [True, False])
def test_host_points_small(pinned):
    w = synth.WORKLOADS["c5"].scaled(N=70_001)
    Xh = synth.host_points(w, DEV, pinned=pinned, block_rows=30_000)
    assert Xh.is_pinned() == pinned
    assert np.array_equal(synth.as_numpy_rows(Xh), synth.points(w))
