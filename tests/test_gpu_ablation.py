"""The comparison baselines (materialised assignment, atomic scatter update) compute the same Lloyd step."""
import numpy as np
import pytest
import torch

import means_clustering_amd as km
from means_clustering_amd import ablation
from tests import parity

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.mark.parametrize("xdtype", ["bf16", "f16"])
@pytest.mark.parametrize("shape", [(5000, 128, 1024), (3001, 64, 500), (777, 100, 37), (64, 16, 1)],
                         ids=lambda s: "x".join(map(str, s)))
def test_materialized_assign_equals_flash_assign(shape, xdtype):
    N, D, K = shape
    g = torch.Generator().manual_seed(N + D + K)
    X = torch.randn(N, D, generator=g).to(TORCH_DT[xdtype]).to(DEV)
    C = torch.randn(K, D, generator=g).to(DEV)
    print(f"[ablation] materialized {shape} {xdtype}", flush=True)
    a_mat = ablation.assign_materialized(X, C)
    a_fa, _ = km.assign(X, C)
    torch.cuda.synchronize()
    assert torch.equal(a_mat, a_fa)  # the same scores, so the same argmax
    Xn, xdt = parity.x_to_numpy(X)
    parity.check_assign(Xn, xdt, C.cpu().numpy(), a_mat.cpu().numpy(), label=f"materialized {shape}")


@pytest.mark.parametrize("xdtype", ["f32", "bf16"])
def test_atomic_update_matches_oracle(xdtype):
    N, D, K = 20000, 64, 300
    g = torch.Generator().manual_seed(7)
    X = (torch.randn(N, D, generator=g) * 2).to(TORCH_DT[xdtype]).to(DEV)
    rng = np.random.default_rng(8)
    a_np = rng.integers(0, K, N)
    a_np[::53] = -1
    C_prev = torch.randn(K, D, generator=g).to(DEV)
    print(f"[ablation] atomic update {xdtype}", flush=True)
    C_new, counts = ablation.update_atomic(X, torch.from_numpy(a_np.astype(np.int32)).to(DEV), C_prev)
    torch.cuda.synchronize()
    Xn, xdt = parity.x_to_numpy(X)
    parity.check_update(Xn, xdt, a_np, C_prev.cpu().numpy(), C_new.cpu().numpy(), counts.cpu().numpy(),
                        label=f"atomic {xdtype}")
