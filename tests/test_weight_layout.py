"""The transposed-weight entry points (det_splitk_gemm_wt, det_splitk_addmm_wt:
the right operand given as a row-major [N, K] matrix, as a linear layer
keeps its weight) against the oracle, and bit for bit against the
untransposed calls on the same values: the products and the chunk tree are
the same, only the loads differ.  Shapes cover every tile family and both
GEMM engines, ragged M and N tails, one- and eight-chunk K, a chunk that is
not a whole number of 64-wide K blocks, a padded leading dimension, and the
dense workload at full size."""
import numpy as np
import pytest
import torch

from helpers import assert_bitwise, assert_gemm_parity, dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def transposed(W_bits, dev, pad=0):
    """[K, N] view of a row-major [N, K + pad] device copy of W."""
    K, N = W_bits.shape
    Wt = np.zeros((N, K + pad), dtype=np.uint16)
    Wt[:, :K] = W_bits.T
    d = dev_bf16(Wt, dev)
    return d[:, :K].t()


def det(X, W, S, dev):
    M, K = X.shape
    N = W.shape[1]
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(X, W, Y, S, detred.workspace(M, N, K, S, dev))
    return Y


# (M, N, K): narrow (64x16 tiles), mid (64x64), wide (128x128 LDS engine),
# one-chunk K with N > 64 (64x64 register engine), K = 200 (zero-padded last
# MFMA step), K = 768 (chunks of 96: a 64-wide block and a 32-wide one)
SHAPES = [(37, 16, 4096), (100, 64, 4096), (200, 1000, 4096), (130, 520, 192),
          (70, 264, 200), (129, 136, 768), (1, 4096, 512), (300, 392, 2048), (2100, 48, 512)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_transposed_weight_matches_row_major_and_oracle(M, N, K, dev):
    X, W = inputs.dense_inputs(M, K, N, seed=3 * M + N + K)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    Wtv = transposed(W, dev)
    assert Wtv.stride(0) == 1 and not Wtv.is_contiguous()
    P = detred.policy(N, K)["chunks"]
    for S in [s for s in (1, 2, 4, 8) if s <= P]:
        ref = det(Xd, Wd, S, dev)
        got = det(Xd, Wtv, S, dev)
        torch.cuda.synchronize()
        assert_bitwise(got, ref, "Wt vs W, S=%d" % S)
    assert_gemm_parity(got, X, W)


def test_padded_leading_dimension(dev):
    M, N, K = 150, 384, 1024
    X, W = inputs.dense_inputs(M, K, N, seed=5)
    Xd = dev_bf16(X, dev)
    ref = det(Xd, dev_bf16(W, dev), 2, dev)
    got = det(Xd, transposed(W, dev, pad=40), 2, dev)
    torch.cuda.synchronize()
    assert_bitwise(got, ref, "Wt with ldwt = K + 40")


def test_addmm_transposed_weight(dev):
    M, N, K = 96, 648, 4096
    X, W = inputs.dense_inputs(M, K, N, seed=9)
    Xd, Wd, Wtv = dev_bf16(X, dev), dev_bf16(W, dev), transposed(W, dev)
    bias = torch.linspace(-1, 1, N, device=dev, dtype=torch.float32)
    for out_dtype, S in ((torch.float32, 1), (torch.bfloat16, 4)):
        ws = detred.workspace(M, N, K, S, dev)
        a = torch.empty((M, N), dtype=out_dtype, device=dev)
        b = torch.empty((M, N), dtype=out_dtype, device=dev)
        detred.det_splitk_addmm(Xd, Wd, a, bias, 0.5, 2.0, S, ws)
        detred.det_splitk_addmm(Xd, Wtv, b, bias, 0.5, 2.0, S, ws)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16) if out_dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if out_dtype == torch.bfloat16 else b.view(torch.int32))


def test_dense_workload_full_size(dev):
    """X[256,4096] x W[4096,14336] with the weight as [14336, 4096]: the
    same bits as the row-major weight, and the oracle on sampled rows."""
    M, N, K = 256, 14336, 4096
    X, W = inputs.dense_inputs(M, K, N, seed=0)
    Xd = dev_bf16(X, dev)
    ref = det(Xd, dev_bf16(W, dev), 0, dev)
    got = det(Xd, transposed(W, dev), 0, dev)
    torch.cuda.synchronize()
    assert_bitwise(got, ref, "dense workload, Wt vs W")
    assert_gemm_parity(got, X, W, rows=[0, 1, 127, 128, 255])


@pytest.mark.parametrize("M,N,K", [(300, 264, 2048), (520, 3080, 8192), (5, 1032, 8192)])
def test_tree_tp_transposed_weight(M, N, K, dev):
    """tree_tp_gemm, tree_tp_shards_gemm and tree_tp_shard_gemm with the
    weight as a row-parallel linear layer keeps it ([N, K]; per rank the
    [N, K/T] columns of it): the bits of the row-major calls for every T,
    on the 128x128 and 256x256 root tiles and the decode tile."""
    X, W = inputs.dense_inputs(M, K, N, seed=M + 7)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    Wtv = transposed(W, dev)
    ref = det(Xd, Wd, 1, dev)
    for T in (1, 2, 4, 8):
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        detred.tree_tp_gemm(Xd, Wtv, Y, T, detred.workspace(M, N, K, T, dev))
        P = torch.empty((T, M, N), dtype=torch.float32, device=dev)
        detred.tree_tp_shards_gemm(Xd, Wtv, P, T)
        Yp = torch.empty_like(Y)
        detred.tree_combine_f32(P, Yp)
        Kt = K // T
        parts = torch.empty((T, M, N), dtype=torch.float32, device=dev)
        Wt_rows = Wtv.t()  # [N, K], K contiguous
        for t in range(T):
            Xs = Xd[:, t * Kt:(t + 1) * Kt].contiguous()
            Ws = Wt_rows[:, t * Kt:(t + 1) * Kt].contiguous()  # the rank's [N, Kt] shard
            detred.tree_tp_shard_gemm(Xs, Ws.t(), parts[t], T)
        Yc = torch.empty_like(Y)
        detred.tree_combine_f32(parts, Yc)
        torch.cuda.synchronize()
        assert_bitwise(Y, ref, "tree_tp_gemm with [N,K] weight, T=%d" % T)
        assert_bitwise(Yp, ref, "tree_tp_shards_gemm with [N,K] weight + combine, T=%d" % T)
        assert_bitwise(Yc, ref, "rank shards with [N,Kt] weights + combine, T=%d" % T)
    assert_gemm_parity(ref, X, W, rows=[0, M - 1])
