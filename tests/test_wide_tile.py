"""The 192x128 eight-chunk tile for unsplit products where it takes fewer
rounds of workgroups than the 128x128 tile (1.25 x its rounds over 256 CUs
at most the 128x128 tile's): eight waves of 96x32, two saved subtree levels
in registers and the top one parked in the product's own output rows
between chunk 3 and 7, read back by LDS-DMA into the freed stage buffers.

Its bits must equal those of every other tile and split (here: 2 slices,
which run the 128x128 engine and the combine launch, and a batch prefix
short enough for the unsplit 128x128 tile), its values the oracle's; the
park must not disturb anything outside the output's M x N elements, and an
addmm whose C overlaps Y must still read C intact."""
import numpy as np
import pytest
import torch

from helpers import assert_bitwise, assert_gemm_parity, dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu

# (M, N, K, prefix): full tiles (1536 = 8 x 192 rows, 4096 = 32 x 128
# columns), ragged rows and columns, chunks of 64, 128, 512, 1024 and 1792
# (one and two K blocks per chunk: the read-back of the parked level starts
# right after it is stored); the prefix rows alone take the 128x128 tile
# (one round of workgroups either way)
SHAPES = [(1536, 4096, 4096, 1024), (1024, 14336, 4096, 512), (1100, 4104, 4096, 896),
          (2000, 4104, 8192, 896), (1030, 4200, 14336, 896), (1536, 4096, 512, 1024),
          (1100, 4104, 1024, 896)]


def det(Xd, Wd, S, dev):
    M, K = Xd.shape
    N = Wd.shape[1]
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(Xd, Wd, Y, S, detred.workspace(M, N, K, S, dev))
    return Y


@pytest.mark.parametrize("M,N,K,prefix", SHAPES)
def test_wide_tile_bits_and_parity(M, N, K, prefix, dev):
    print("case wide %dx%dx%d" % (M, N, K), flush=True)
    X, W = inputs.dense_inputs(M, K, N, seed=5)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    y1 = det(Xd, Wd, 1, dev)
    y2 = det(Xd, Wd, 2, dev)
    torch.cuda.synchronize()
    assert_bitwise(y1, y2, "split 1 (192x128 tile) vs split 2")
    # rows across the tile edges and the ragged last tile row
    rows = sorted({0, 1, 191, 192, 383, M // 2, (M // 192) * 192 - 1, (M // 192) * 192, M - 1})
    assert_gemm_parity(y1, X, W, rows=[r for r in rows if r < M])
    # the prefix rows alone run the unsplit 128x128 tile
    yp = det(Xd[:prefix], Wd, 1, dev)
    torch.cuda.synchronize()
    assert_bitwise(yp, y1[:prefix], "rows of %d alone vs the same rows in %d" % (prefix, M))


def test_wide_tile_integer_inputs_exact(dev):
    """Integer inputs are exact in every order: the 192x128 tile equals the
    oracle bit for bit at 2048 x 14336 x 4096."""
    import oracle
    M, N, K = 2048, 14336, 4096
    X = inputs.integer_bf16((M, K), -8, 8, 3, 0)
    W = inputs.integer_bf16((K, N), -8, 8, 3, 1)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    y = det(Xd, Wd, 1, dev)
    torch.cuda.synchronize()
    rows = [0, 191, 192, 1000, 2047]
    ref, _ = oracle.gemm(X[rows], W)
    got = y[rows].cpu().numpy().astype(np.float64)
    assert np.array_equal(got, ref)


def test_wide_tile_keeps_padding_and_addmm(dev):
    """Y as rows of a wider buffer: the park and the final store leave the
    padding columns alone.  addmm with a bias row and with a separate C
    matrix equals its split-2 form bit for bit; with C overlapping Y (in
    place) the product still reads C intact."""
    M, N, K = 1100, 4104, 4096
    X, W = inputs.dense_inputs(M, K, N, seed=6)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    buf = torch.full((M, N + 64), 123.0, dtype=torch.float32, device=dev)
    Y = buf[:, :N]
    detred.det_splitk_gemm(Xd, Wd, Y, 1)
    ref = det(Xd, Wd, 2, dev)
    torch.cuda.synchronize()
    assert_bitwise(Y, ref, "padded Y")
    assert bool((buf[:, N:] == 123.0).all()), "padding columns were written"

    g = torch.Generator(device=dev)
    g.manual_seed(9)
    bias = torch.randn((N,), device=dev, generator=g)
    C = torch.randn((M, N), device=dev, generator=g)
    for cc in (bias, C):
        y1 = torch.empty((M, N), dtype=torch.float32, device=dev)
        y2 = torch.empty_like(y1)
        detred.det_splitk_addmm(Xd, Wd, y1, cc, 0.5, 2.0, 1)
        detred.det_splitk_addmm(Xd, Wd, y2, cc, 0.5, 2.0, 2, detred.workspace(M, N, K, 2, dev))
        torch.cuda.synchronize()
        assert_bitwise(y1, y2, "addmm split 1 vs 2 (C %s)" % (tuple(cc.shape),))
    # in place: C is Y
    yin = C.clone()
    detred.det_splitk_addmm(Xd, Wd, yin, yin, 0.5, 2.0, 1)
    yout = torch.empty_like(yin)
    detred.det_splitk_addmm(Xd, Wd, yout, C, 0.5, 2.0, 1)
    torch.cuda.synchronize()
    assert_bitwise(yin, yout, "addmm with C = Y vs a separate C")


def test_wide_tile_transposed_weight_and_tree_tp(dev):
    """The transposed-weight layout on the 192x128 tile and tree-TP with one
    shard (which takes it) give the bits of eight shards."""
    M, N, K = 1280, 4096, 8192
    X, W = inputs.dense_inputs(M, K, N, seed=8)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    y = det(Xd, Wd, 1, dev)
    Wt = Wd.t().contiguous()
    yt = torch.empty_like(y)
    detred.det_splitk_gemm(Xd, Wt.t(), yt, 1)
    y8 = torch.empty_like(y)
    detred.tree_tp_gemm(Xd, Wd, y8, 8, detred.workspace(M, N, K, 8, dev))
    y1 = torch.empty_like(y)
    detred.tree_tp_gemm(Xd, Wd, y1, 1)
    torch.cuda.synchronize()
    assert_bitwise(yt, y, "transposed weight")
    assert_bitwise(y1, y8, "tree-TP T=1 vs T=8")
    assert_bitwise(y1, y, "tree-TP T=1 vs det")
