"""Bit invariance across every point where the launched tile or the
automatic split changes with M.  On each side of a switch the shared rows
must be bit-identical (the chunk tree fixes the bits; the tile and the split
only decide speed):
  * 64 / 65 rows:    64x128 tile -> 128x128 tile;
  * 512 / 513 rows of a 14336-column output and 1024 / 1025 rows of a
    4096-column one (eight chunks, one slice): 128x128 -> 192x128, where
    the 192x128 tile starts to take fewer rounds of workgroups;
  * 255 / 256 rows, shard roots with chunks of 1024: 128x128 -> 256x256,
    roots compared directly;
  * 255 / 256 rows at K = 14336 (chunks of 1792): the automatic split
    becomes 8 (one chunk per slice on the 256x256 root tile);
  * 1984 / 1985 rows of a 64-column output at 8 slices: 64x16 -> 64x64;
  * 1023 / 1024 rows of a 64-column output at 8 slices (4095 / 4096 rows of
    a 16-column one): the one-launch (last arriver) combine -> the
    two-launch combine."""
import pytest
import torch

from helpers import assert_bitwise, dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def det(Xd, Wd, S, dev):
    M, K = Xd.shape
    N = Wd.shape[1]
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(Xd, Wd, Y, S, detred.workspace(M, N, K, S, dev))
    return Y


@pytest.mark.parametrize("N,K,S,Ms", [
    (4096, 4096, 1, (64, 65)),           # 64x128 -> 128x128
    (4096, 4096, 0, (64, 65)),
    (14336, 4096, 1, (512, 513)),        # 128x128 -> 192x128
    (4096, 4096, 1, (1024, 1025)),       # 128x128 -> 192x128
    (8192, 14336, 0, (255, 256)),        # automatic split -> 8 on 256x256
    (64, 4096, 8, (1984, 1985)),         # 64x16 -> 64x64
    (64, 4096, 8, (1023, 1024)),         # one-launch -> two-launch combine
    (16, 4096, 8, (4095, 4096)),         # one-launch -> two-launch (16 columns)
])
def test_rows_equal_across_switch(N, K, S, Ms, dev):
    lo, hi = Ms
    print("case N=%d K=%d S=%d M=%d/%d (auto split %d/%d)" % (
        N, K, S, lo, hi, detred.auto_split(lo, N, K), detred.auto_split(hi, N, K)), flush=True)
    X, W = inputs.dense_inputs(hi, K, N, seed=21)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    y_hi = det(Xd, Wd, S, dev)
    y_lo = det(Xd[:lo], Wd, S, dev)
    y_1 = det(Xd, Wd, 1, dev)
    torch.cuda.synchronize()
    assert_bitwise(y_lo, y_hi[:lo], "rows of M=%d vs M=%d" % (lo, hi))
    assert_bitwise(y_hi, y_1, "M=%d at split %d vs unsplit" % (hi, S))


def test_shard_roots_across_256x256_switch(dev):
    """Shard roots of 8 one-chunk shards (chunks of 1024) at 255 rows
    (128x128 tile) and 256 rows (256x256 tile): the roots themselves are
    bit-identical row by row, and so are the combined products."""
    N, K = 2048, 8192
    X, W = inputs.dense_inputs(256, K, N, seed=22)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    p_hi = torch.empty((8, 256, N), dtype=torch.float32, device=dev)
    p_lo = torch.empty((8, 255, N), dtype=torch.float32, device=dev)
    detred.tree_tp_shards_gemm(Xd, Wd, p_hi, 8)
    detred.tree_tp_shards_gemm(Xd[:255], Wd, p_lo, 8)
    y_hi = torch.empty((256, N), dtype=torch.float32, device=dev)
    detred.tree_tp_gemm(Xd, Wd, y_hi, 8, detred.workspace(256, N, K, 8, dev))
    y_1 = det(Xd, Wd, 1, dev)
    torch.cuda.synchronize()
    for t in range(8):
        assert_bitwise(p_lo[t], p_hi[t, :255], "shard %d roots, 255 vs 256 rows" % t)
    assert_bitwise(y_hi, y_1, "tree-TP T=8 vs unsplit")
