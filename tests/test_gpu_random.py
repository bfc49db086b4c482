"""Seeded random shapes through kmeans_fit against the oracle: fp32, bf16 and fp16 X, ragged D, N and K around
the tile, block and path boundaries, K above N (empty clusters), one to three iterations.  Each iteration is checked against the oracle on
the GPU's own state, and a fit of T iterations must equal T fits of one iteration, bit for bit.

The problems here are small, so 0.01% of their points is often less than one point: one near-tie mismatch
per problem and iteration is allowed, and mismatches whose oracle gap is within the fp32 error of the kernel's
own score (ties at the kernel's precision, frequent for D = 1 with dense centroids) are not counted.  Every
mismatch must still lie within the near-tie gap.  The full-size workloads keep the plain 0.01% bar."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
import synth
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _cases(n=96, seed=2026):
    rng = np.random.default_rng(seed)
    Ds = {"f32": [1, 2, 3, 5, 16, 31, 32, 33, 64, 100, 128, 200, 256],
          "bf16": [1, 3, 8, 15, 16, 17, 48, 64, 65, 100, 128, 129, 200, 256, 300, 512],
          "f16": [1, 7, 16, 40, 64, 96, 128, 160, 255, 384, 512]}
    Ks = [1, 2, 3, 31, 63, 64, 65, 96, 127, 128, 129, 255, 256, 257, 600, 1000, 2049, 4099, 8193]
    Ns = [1, 2, 33, 511, 1000, 2048, 2049, 4097, 12345, 30011, 65537]
    out = []
    while len(out) < n:
        dt = str(rng.choice(["f32", "bf16", "f16"]))
        D, K, N = int(rng.choice(Ds[dt])), int(rng.choice(Ks)), int(rng.choice(Ns))
        T = int(rng.integers(1, 4))
        if N * K * D > 1.5e9:
            continue
        out.append((dt, N, D, K, T, int(rng.integers(1 << 30))))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}-T{c[4]}" for c in CASES])
def test_random_fit(case):
    dt, N, D, K, T, seed = case
    print(f"[random] {dt} N={N} D={D} K={K} T={T} seed={seed}", flush=True)
    w = synth.WORKLOADS["c2"].scaled(N=N, D=D, K=K, M=K, dtype="f32", seed=seed)
    Xn = synth.points(w)
    if K <= N:
        C0 = torch.from_numpy(synth.init_centroids(w, Xn)).to(DEV)
    else:  # more clusters than points: random centroids, most of them stay empty
        C0 = torch.from_numpy(np.random.default_rng(seed).normal(size=(K, D)).astype(np.float32)).to(DEV)
    X = torch.from_numpy(Xn).to(TORCH_DT[dt]).to(DEV)
    Xs, name = parity.x_to_numpy(X)  # the stored values, as the oracle reads them
    C = C0
    for t in range(T):
        C_prev = C.cpu().numpy()
        C, a, counts, _ = km.fit(X, C, 1)
        torch.cuda.synchronize()
        an = a.cpu().numpy()
        parity.check_assign(Xs, name, C_prev, an, label=f"it{t}", min_near_ties=1, precision_ties=True)
        parity.check_update(Xs, name, an, C_prev, C.cpu().numpy(), counts.cpu().numpy(), label=f"it{t}")
    CT, aT, nT, _ = km.fit(X, C0, T)
    torch.cuda.synchronize()
    assert torch.equal(CT, C) and torch.equal(aT, a) and torch.equal(nT, counts)


def _batched_cases(n=24, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dt = str(rng.choice(["f32", "bf16", "f16"]))
        B, N = int(rng.choice([1, 2, 3, 5, 17])), int(rng.choice([1, 33, 1000, 2049, 5000]))
        D = int(rng.choice([1, 3, 16, 33, 64, 128, 200] + ([256, 512] if dt != "f32" else [])))
        K, T = int(rng.choice([1, 2, 31, 64, 65, 128, 300])), int(rng.integers(1, 4))
        if K > N or B * N * K * D > 1.5e9:
            continue
        out.append((dt, B, N, D, K, T, int(rng.integers(1 << 30))))
    return out


BATCHED = _batched_cases()


@pytest.mark.parametrize("case", BATCHED,
                         ids=[f"{c[0]}-B{c[1]}-N{c[2]}-D{c[3]}-K{c[4]}-T{c[5]}" for c in BATCHED])
def test_random_batched(case):
    """kmeans_fit_batched: every problem of every iteration against the oracle; T iterations in one call equal
    T calls of one iteration."""
    dt, B, N, D, K, T, seed = case
    print(f"[random batched] {case}", flush=True)
    Xs, Cs = [], []
    for b in range(B):
        w = synth.WORKLOADS["c2"].scaled(N=N, D=D, K=K, M=K, dtype="f32", seed=seed + b)
        Xn = synth.points(w)
        Xs.append(Xn)
        Cs.append(synth.init_centroids(w, Xn))
    X = torch.from_numpy(np.stack(Xs)).to(TORCH_DT[dt]).to(DEV)
    C0 = torch.from_numpy(np.stack(Cs)).to(DEV)
    C = C0
    for t in range(T):
        C_prev = C.cpu().numpy()
        C, a, counts, _ = km.fit_batched(X, C, 1)
        torch.cuda.synchronize()
        for b in range(B):
            xs, name = parity.x_to_numpy(X[b])
            an = a[b].cpu().numpy()
            parity.check_assign(xs, name, C_prev[b], an, label=f"problem {b} it{t}", min_near_ties=1,
                                precision_ties=True)
            parity.check_update(xs, name, an, C_prev[b], C[b].cpu().numpy(), counts[b].cpu().numpy(),
                                label=f"problem {b} it{t}")
    CT, aT, nT, _ = km.fit_batched(X, C0, T)
    torch.cuda.synchronize()
    assert torch.equal(CT, C) and torch.equal(aT, a) and torch.equal(nT, counts)


def _streamed_cases(n=16, seed=99):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        dt = str(rng.choice(["f32", "bf16", "f16"]))
        N = int(rng.choice([1, 1000, 4097, 30011]))
        D = int(rng.choice([1, 16, 33, 64, 128] + ([512] if dt != "f32" else [256])))
        K = int(rng.choice([1, 7, 64, 65, 300]))
        chunk = int(rng.choice([1, 7, 1000, max(N - 1, 1), N, N + 5]))
        stage = int(rng.choice([0, 4096 * 4, 1 << 20]))  # 0: pinned X
        if K > N or N * K * D > 1.5e9 or (chunk < 16 and N > 1000):
            continue
        out.append((dt, N, D, K, chunk, stage, int(rng.integers(1, 3)), int(rng.integers(1 << 30))))
    return out


STREAMED = _streamed_cases()


@pytest.mark.parametrize("case", STREAMED,
                         ids=[f"{c[0]}-N{c[1]}-D{c[2]}-K{c[3]}-chunk{c[4]}-stage{c[5]}" for c in STREAMED])
def test_random_streamed(case):
    """kmeans_fit_streamed with X in pinned or pageable host memory, every iteration against the oracle."""
    from tests.test_gpu_fit import _teacher_forced
    dt, N, D, K, chunk, stage, T, seed = case
    w = synth.WORKLOADS["c2"].scaled(N=N, D=D, K=K, M=K, dtype="f32", seed=seed)
    Xn = synth.points(w)
    C0 = synth.init_centroids(w, Xn)
    xs, name = parity.x_to_numpy(torch.from_numpy(Xn).to(TORCH_DT[dt]))
    _teacher_forced(xs, name, C0, T, f"random streamed {case}", streamed_chunk=chunk,
                    stage_bytes=stage if stage else None, min_near_ties=1, precision_ties=True)
