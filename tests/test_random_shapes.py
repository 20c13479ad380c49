"""Seeded random shapes through every tile the planner can pick (64x16,
64x64, the register-staged and LDS-DMA 128x128, 64x128 for at most 64
rows, 256x256 for long shard roots), both weight layouts and every split:
all splits and shard counts give the bits of S = 1, and sampled rows meet
the oracle's tolerance."""
import numpy as np
import pytest
import torch

from helpers import assert_bitwise, assert_gemm_parity, dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def _shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 300)),
                            int(rng.integers(300, 700))]))
        N = 8 * int(rng.choice([int(rng.integers(1, 9)), int(rng.integers(9, 200)),
                                int(rng.integers(200, 700))]))
        K = int(rng.choice([8 * int(rng.integers(1, 40)), 256 * int(rng.integers(1, 12)),
                            8192]))
        out.append((M, N, K))
    return out


def _det(X, W, S, dev):
    M, N = X.shape[0], W.shape[1]
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(X, W, Y, S, detred.workspace(M, N, X.shape[1], S, dev))
    return Y


# plus shapes that reach the 256x256 shard-root tile (T = 8, chunks of 1024)
# and the edges of the 64-row tile
@pytest.mark.parametrize("M,N,K", _shapes(24, 2024) + [(700, 3000, 8192), (64, 3000, 8192),
                                                      (65, 264, 8192), (47, 1000, 2048)])
def test_random_shape_splits_layouts_and_parity(M, N, K, dev):
    X, W = inputs.dense_inputs(M, K, N, seed=M + 3 * N + 7 * K)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    ref = _det(Xd, Wd, 1, dev)
    P = detred.policy(N, K)["chunks"]
    for S in [0] + [s for s in (2, 4, 8) if s <= P]:
        assert_bitwise(_det(Xd, Wd, S, dev), ref, "S=%d" % S)
    # the weight as a linear layer keeps it ([N, K]), transposed view
    Wt = Wd.t().contiguous().t()
    assert_bitwise(_det(Xd, Wt, 0, dev), ref, "transposed weight")
    if P == 8:
        for T in (2, 8):
            Y = torch.empty_like(ref)
            detred.tree_tp_gemm(Xd, Wd, Y, T, detred.workspace(M, N, K, T, dev))
            torch.cuda.synchronize()
            assert_bitwise(Y, ref, "tree_tp T=%d" % T)
    torch.cuda.synchronize()
    rows = sorted({0, M // 2, M - 1})
    assert_gemm_parity(ref, X, W, rows=rows)
