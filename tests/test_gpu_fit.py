"""Lloyd iterations (kmeans_fit, kmeans_fit_streamed) against the fp64 oracle, iteration by iteration."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _workload(name, **kw):
    w = synth.WORKLOADS[name].scaled(**kw)
    Xn = synth.points(w)
    C0 = synth.init_centroids(w, Xn)
    return w, Xn, C0


def _teacher_forced(Xn, xdtype, C0, T, label, streamed_chunk=None, stage_bytes=None, min_near_ties=0,
                    precision_ties=False):
    """Run T single iterations on the GPU; check each against the oracle fed the GPU's own state."""
    X = parity.x_from_numpy(Xn, xdtype, DEV)
    C = torch.from_numpy(C0).to(DEV)
    max_err, flips = 0.0, 0
    for t in range(T):
        print(f"[fit] {label} iteration {t}", flush=True)
        C_prev = C.cpu().numpy()
        if streamed_chunk is None:
            C, a, counts, obj = km.fit(X, C, 1, objective=True)
        else:
            if stage_bytes is None:  # pinned X, direct upload
                Xh, stage = X.cpu().pin_memory(), None
            else:  # pageable X through a pinned staging ring
                Xh, stage = X.cpu(), km.staging_buffer(stage_bytes)
            C, a, counts, obj = km.fit_streamed(Xh, C, 1, streamed_chunk, objective=True, stage=stage)
        torch.cuda.synchronize()
        an = a.cpu().numpy() if a.is_cuda else a.numpy()
        nm, _ = parity.check_assign(Xn, xdtype, C_prev, an, label=f"{label} it{t}", min_near_ties=min_near_ties,
                                    precision_ties=precision_ties)
        flips += nm
        max_err = max(max_err, parity.check_update(Xn, xdtype, an, C_prev, C.cpu().numpy(),
                                                   counts.cpu().numpy(), label=f"{label} it{t}"))
        # objective: sum of the fp32 distances, against the fp64 distances to the same centroids
        parity.check_objective(Xn, xdtype, C_prev, an, obj.cpu().numpy()[0], label=f"{label} it{t}")
    return max_err, flips


def test_fit_small_mixture_fp32():
    w, Xn, C0 = _workload("c1", N=3000, K=40)
    _teacher_forced(Xn, "f32", C0, 6, "c1-like fp32")


def test_fit_small_mixture_bf16():
    w, Xn, C0 = _workload("c2", N=20000, K=256)
    _teacher_forced(Xn, "bf16", C0, 5, "c2-like bf16")


def test_fit_small_mixture_fp16():
    w, Xn, C0 = _workload("c2", N=15000, K=200, D=72)
    X16 = synth.bf16_bits_to_f32(Xn).astype(np.float16)  # the same points stored as fp16
    _teacher_forced(X16, "f16", C0.astype(np.float16).astype(np.float32), 4, "c2-like fp16, D=72")


def test_fit_skewed_bf16():
    w, Xn, C0 = _workload("c4", N=60000, K=512)
    _teacher_forced(Xn, "bf16", C0, 4, "c4-like zipf")


def test_fit_unit_sphere_bf16():
    w, Xn, C0 = _workload("c3", N=20000, K=2048)
    _teacher_forced(Xn, "bf16", C0, 3, "c3-like sphere")


@pytest.mark.parametrize("D", [32, 64, 128])
def test_fit_long_sweep_warm_start(D):
    """K = 8192: the warm-started single-accumulator kernel from the second iteration on."""
    w, Xn, C0 = _workload("c3", N=12000, K=8192, D=D)
    _teacher_forced(Xn, "bf16", C0, 3, f"long sweep D={D}")
    X = parity.x_from_numpy(Xn, "bf16", DEV)
    C3, a3, n3, _ = km.fit(X, torch.from_numpy(C0).to(DEV), 3)
    C2, _, _, _ = km.fit(X, torch.from_numpy(C0).to(DEV), 2)
    C1, a1, n1, _ = km.fit(X, C2, 1)
    torch.cuda.synchronize()
    assert torch.equal(C3, C1) and torch.equal(a3, a1) and torch.equal(n3, n1)


@pytest.mark.parametrize("chunk", [7, 1000, 4096, 100_000])
def test_fit_streamed_matches_oracle(chunk):
    w, Xn, C0 = _workload("c4", N=9000, K=300)
    _teacher_forced(Xn, "bf16", C0, 2, f"streamed chunk={chunk}", streamed_chunk=chunk)


@pytest.mark.parametrize("chunk,stage_rows", [(1000, 4 * 37), (4096, 4 * 4096), (100_000, 4 * 333), (7, 4 * 3)])
def test_fit_streamed_pageable_matches_oracle(chunk, stage_rows):
    w, Xn, C0 = _workload("c4", N=9000, K=300)
    _teacher_forced(Xn, "bf16", C0, 2, f"streamed pageable chunk={chunk} stage={stage_rows}",
                    streamed_chunk=chunk, stage_bytes=stage_rows * w.D * 2 + 5)


def test_fit_streamed_pinned_and_pageable_agree():
    w, Xn, C0 = _workload("c4", N=20000, K=256)
    X = parity.x_from_numpy(Xn, "bf16", DEV).cpu()
    C0t = torch.from_numpy(C0).to(DEV)
    r1 = km.fit_streamed(X.pin_memory(), C0t, 3, 3000)
    r2 = km.fit_streamed(X, C0t, 3, 3000, stage=km.staging_buffer(4 * 500 * w.D * 2))
    torch.cuda.synchronize()
    assert torch.equal(r1[0], r2[0]) and torch.equal(r1[1], r2[1]) and torch.equal(r1[2], r2[2])


@pytest.mark.parametrize("resident", [True, "2.5 chunks", "1 row short of a chunk"])
@pytest.mark.parametrize("pageable", [False, True])
def test_fit_streamed_resident_copy_equals_streamed(resident, pageable):
    """A device copy of X (all of it, or the leading chunks that fit whole in the extra workspace) changes only
    where later iterations read X from: centroids, assignment, counts and objective equal the fully streamed
    fit's bit for bit, for pinned and pageable X, with a ragged last chunk."""
    w, Xn, C0 = _workload("c4", N=250_003, D=64, K=1000, M=1000)
    X = parity.x_from_numpy(Xn, "bf16", DEV).cpu()
    chunk = 60_000
    row = w.D * 2
    nbytes = {True: True, "2.5 chunks": int(2.5 * chunk * row), "1 row short of a chunk": chunk * row - row}[resident]
    Xh = X if pageable else X.pin_memory()
    stage = km.staging_buffer(4 * 7_000 * row) if pageable else None
    C0t = torch.from_numpy(C0).to(DEV)
    print(f"[fit] streamed with resident copy {resident}, pageable {pageable}", flush=True)
    rr = km.fit_streamed(Xh, C0t, 4, chunk, objective=True, stage=stage, resident=nbytes)
    torch.cuda.synchronize()
    rs = km.fit_streamed(Xh, C0t, 4, chunk, objective=True, stage=stage)
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(rr[i], rs[i]), f"resident copy changes output {i}"
    C3 = km.fit_streamed(Xh, C0t, 3, chunk, stage=stage)[0]
    torch.cuda.synchronize()
    Xs, xdt = parity.x_to_numpy(X)
    an = rr[1].numpy()
    parity.check_assign(Xs, xdt, C3.cpu().numpy(), an, label=f"resident {resident}")
    parity.check_update(Xs, xdt, an, C3.cpu().numpy(), rr[0].cpu().numpy(), rr[2].cpu().numpy(),
                        label=f"resident {resident}")


@pytest.mark.parametrize("case", [("c1", "f32", 10_007, 33, 50, 3_000), ("c2", "f16", 20_000, 200, 300, 7_000),
                                  ("c4", "bf16", 5_000, 16, 6_000, 2_048), ("c2", "bf16", 9_000, 600, 64, 9_000)],
                         ids=lambda c: f"{c[1]}-N{c[2]}-D{c[3]}-K{c[4]}-chunk{c[5]}")
def test_fit_streamed_resident_copy_shapes(case):
    """The resident copy across X types and shapes: fp32 and fp16 X, odd D, more clusters than points (most stay
    empty), a single chunk; every output equal to the fully streamed fit's, bit for bit."""
    name, xdtype, N, D, K, chunk = case
    w, Xn, C0 = _workload(name, N=N, D=D, K=min(K, N), M=min(K, 1024))
    if K > N:  # the extra centroids far from every point: they stay empty
        rng = np.random.default_rng(K)
        C0 = np.concatenate([C0, (50.0 + rng.normal(size=(K - N, D))).astype(np.float32)])
    X = parity.x_from_numpy(Xn, w.dtype, DEV)
    if xdtype == "f16":
        X = X.float().half()
    elif xdtype == "f32":
        X = X.float()
    Xh = X.cpu().pin_memory()
    C0t = torch.from_numpy(C0).to(DEV)
    print(f"[fit] streamed resident copy {case}", flush=True)
    rr = km.fit_streamed(Xh, C0t, 3, chunk, objective=True, resident=True)
    torch.cuda.synchronize()
    rs = km.fit_streamed(Xh, C0t, 3, chunk, objective=True)
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(rr[i], rs[i]), f"resident copy changes output {i}"


@pytest.mark.parametrize("case", [("c4", "bf16", 300_000, 64, 4096, 70_000), ("c2", "f16", 40_000, 48, 9000, 15_000),
                                  ("c1", "f32", 50_000, 32, 200, 16_384), ("c2", "bf16", 30_000, 600, 100, 11_000),
                                  ("c4", "bf16", 5_000, 16, 40, 1_024)],
                         ids=lambda c: f"{c[1]}-N{c[2]}-D{c[3]}-K{c[4]}-chunk{c[5]}")
def test_fit_streamed_warm_start_equals_cold(case):
    """With room for every chunk's order, iterations after the first assign each chunk warm (in the order of
    its last argsort): the results must be the cold run's bit for bit; the last iteration against the oracle."""
    name, xdtype, N, D, K, chunk = case
    w, Xn, C0 = _workload(name, N=N, D=D, K=K, M=min(K, 4096))
    X = parity.x_from_numpy(Xn, w.dtype, DEV)
    if xdtype == "f16":  # the bf16 points as fp16 values
        X = X.float().half()
    assert (X.dtype == torch.float32) == (xdtype == "f32")
    Xh = X.cpu().pin_memory()
    C0t = torch.from_numpy(C0).to(DEV)
    print(f"[fit] streamed warm vs cold {case}", flush=True)
    rw = km.fit_streamed(Xh, C0t, 3, chunk, objective=True, warm_start=True)
    rc = km.fit_streamed(Xh, C0t, 3, chunk, objective=True, warm_start=False)
    r2 = km.fit_streamed(Xh, C0t, 2, chunk, warm_start=False)
    torch.cuda.synchronize()
    for i in range(4):
        assert torch.equal(rw[i], rc[i]), f"warm-started streamed fit differs from the cold one (output {i})"
    Xs, xdt = parity.x_to_numpy(X)
    C2 = r2[0].cpu().numpy()
    an = rw[1].numpy()
    parity.check_assign(Xs, xdt, C2, an, label=f"warm streamed {case}")
    parity.check_update(Xs, xdt, an, C2, rw[0].cpu().numpy(), rw[2].cpu().numpy(), label=f"warm streamed {case}")


def test_fit_resume_and_determinism():
    w, Xn, C0 = _workload("c2", N=50000, K=512)
    X = parity.x_from_numpy(Xn, "bf16", DEV)
    C0t = torch.from_numpy(C0).to(DEV)
    C6, a6, n6, obj6 = km.fit(X, C0t, 6, objective=True)
    C6b, a6b, n6b, _ = km.fit(X, C0t, 6)
    Cs = C0t
    objs = []
    for t in range(6):  # resume from the state after every iteration
        Cs, a1, n1, o1 = km.fit(X, Cs, 1, objective=True)
        objs.append(o1)
    torch.cuda.synchronize()
    assert torch.equal(C6, C6b) and torch.equal(a6, a6b) and torch.equal(n6, n6b)
    assert torch.equal(C6, Cs) and torch.equal(a6, a1) and torch.equal(n6, n1)
    assert torch.equal(obj6, torch.cat(objs))


@pytest.mark.parametrize("shape,xdtype", [((16384, 32, 64), "f32"), ((3000, 100, 40), "f32"), ((70000, 7, 20), "f32"),
                                          ((6000, 32, 100), "f32"), ((20000, 72, 300), "bf16"),
                                          ((9000, 200, 130), "f16"), ((5000, 512, 70), "bf16"),
                                          ((30000, 24, 8192), "f32"), ((40000, 16, 9000), "bf16"),
                                          ((16384, 128, 512), "bf16"), ((3000, 64, 40), "bf16"),
                                          ((12000, 300, 100), "f16"), ((16384, 512, 64), "bf16"),
                                          ((16385, 64, 200), "bf16"), ((8000, 33, 513), "f32"),
                                          ((12000, 48, 2000), "bf16"), ((16384, 24, 2049), "f32")],
                         ids=lambda v: "x".join(map(str, v)) if isinstance(v, tuple) else v)
def test_fit_many_iterations_equal_single_steps(shape, xdtype):
    """From the second iteration of a call on, FlashAssign uses the operand fragments that the update wrote
    (the one-launch update for N <= 16384 and K <= 2048, the chunk-sum combine for fp32 K <= 64,
    the fix-up otherwise); T iterations in one call must equal T calls of one iteration (which prepare them
    afresh), bit for bit."""
    N, D, K = shape
    w = synth.WORKLOADS["c1"].scaled(N=N, D=D, K=K)
    Xn = synth.points(w)
    Xf = torch.from_numpy(Xn)
    X = (Xf if xdtype == "f32" else Xf.to(torch.bfloat16 if xdtype == "bf16" else torch.float16)).to(DEV)
    C0 = torch.from_numpy(synth.init_centroids(w, Xn)).to(DEV)
    Ca, aa, na, oa = km.fit(X, C0, 8, objective=True)
    Cs, objs = C0, []
    for _ in range(8):
        Cs, a1, n1, o1 = km.fit(X, Cs, 1, objective=True)
        objs.append(o1)
    torch.cuda.synchronize()
    assert torch.equal(Ca, Cs) and torch.equal(aa, a1) and torch.equal(na, n1)
    assert torch.equal(oa, torch.cat(objs))


def test_fit_zero_iterations_and_fixed_point():
    g = torch.Generator().manual_seed(1)
    cen = torch.tensor([[0.0, 0.0], [10.0, 0.0], [0.0, 10.0]])
    off = torch.tensor([[1.0, 0.0], [-1.0, 0.0], [0.0, 1.0], [0.0, -1.0]])
    X = (cen[:, None, :] + off[None]).reshape(-1, 2)[torch.randperm(12, generator=g)].to(DEV)
    C, a, n, obj = km.fit(X, cen.to(DEV), 0)
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), cen)
    C, a, n, obj = km.fit(X, cen.to(DEV), 3, objective=True)
    torch.cuda.synchronize()
    assert torch.equal(C.cpu(), cen) and n.cpu().tolist() == [4, 4, 4]
    assert obj.cpu().tolist() == [12.0, 12.0, 12.0]


def test_fit_trajectory_1d():
    X = torch.tensor([[0.0], [1.0], [10.0], [11.0]], device=DEV)
    C, a, n, obj = km.fit(X, torch.tensor([[0.0], [1.0]], device=DEV), 3, objective=True)
    torch.cuda.synchronize()
    assert C.cpu().flatten().tolist() == [0.5, 10.5]
    assert a.cpu().tolist() == [0, 0, 1, 1]
    np.testing.assert_allclose(obj.cpu().numpy(), [181.0, 194.0 / 9.0, 1.0], rtol=1e-5)


@pytest.mark.parametrize("pageable", [False, True])
def test_fit_streamed_injected_upload_failure_then_restart(pageable, monkeypatch):
    """A copy that fails mid-stream (forced from the host: KM_FAULT_INJECT_UPLOAD) returns KM_ERR_HIP without a
    fault, with the staging buffer drained; the same call then runs cleanly and equals a fresh run bit for bit."""
    w, Xn, C0 = _workload("c4", N=30_000, K=300)
    X = parity.x_from_numpy(Xn, "bf16", DEV).cpu()
    Xh = X if pageable else X.pin_memory()
    stage = km.staging_buffer(4 * 1000 * w.D * 2) if pageable else None
    C0t = torch.from_numpy(C0).to(DEV)
    ws = km.Workspace(DEV)
    monkeypatch.setenv("KM_FAULT_INJECT_UPLOAD", "5")  # the 5th of 2 x 7 chunk uploads (second iteration)
    with pytest.raises(km.KMeansError) as e:
        km.fit_streamed(Xh, C0t, 2, 4500, ws=ws, stage=stage)
    assert e.value.status == 4 and "h2d" in str(e.value)
    torch.cuda.synchronize()
    monkeypatch.delenv("KM_FAULT_INJECT_UPLOAD")
    r1 = km.fit_streamed(Xh, C0t, 2, 4500, ws=ws, stage=stage)
    r2 = km.fit_streamed(Xh, C0t, 2, 4500, ws=km.Workspace(DEV), stage=stage)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(r1[i], r2[i])
    C_prev = km.fit_streamed(Xh, C0t, 1, 4500, stage=stage)[0]
    torch.cuda.synchronize()
    parity.check_update(Xn, "bf16", r1[1].numpy(), C_prev.cpu().numpy(), r1[0].cpu().numpy(), r1[2].cpu().numpy(),
                        label="after an injected upload failure")


def _poisoned(byte):
    ws = km.Workspace(DEV)
    ws.get(1 << 28, DEV).fill_(byte)  # every call below fits in it
    return ws


@pytest.mark.parametrize("case", [("c1", "f32", 16_384, 32, 64), ("c1", "f32", 40_000, 32, 50),
                                  ("c2", "bf16", 16_384, 64, 600), ("c2", "bf16", 50_000, 128, 1024),
                                  ("c2", "bf16", 5_000, 64, 4_800), ("c2", "bf16", 5_000, 700, 100)],
                         ids=lambda c: f"{c[1]}-N{c[2]}-D{c[3]}-K{c[4]}")
def test_workspace_content_is_never_read_before_written(case):
    """The workspace may hold anything: fits with a workspace full of 0xFF bytes (NaN patterns, all ones) and
    full of zeros give the same results bit for bit, on every update path (one-launch and chunked small
    codebooks, sorted, split sweep, deep rows) and for the batched and streamed fits."""
    name, xdt, N, D, K = case
    w, Xn, C0 = _workload(name, N=N, D=D, K=K, M=min(K, 1024))
    X = parity.x_from_numpy(Xn, w.dtype, DEV)
    C0t = torch.from_numpy(C0).to(DEV)
    outs = []
    Xh = X.cpu().pin_memory()
    for byte in (0xFF, 0x00):
        C, a, n, J = km.fit(X, C0t, 3, objective=True, ws=_poisoned(byte))
        Cb, ab, nb, Jb = km.fit_batched(torch.stack([X, X]), torch.stack([C0t, C0t]), 2, objective=True,
                                        ws=_poisoned(byte))
        Cs, as_, ns, Js = km.fit_streamed(Xh, C0t, 2, max(N // 3, 1), objective=True, ws=_poisoned(byte))
        torch.cuda.synchronize()
        outs.append([C, a, n, J, Cb, ab, nb, Jb, Cs, as_, ns, Js])
    for i, (u, v) in enumerate(zip(*outs)):
        assert torch.equal(u.cpu(), v.cpu()), f"output {i} depends on the workspace's prior content"
