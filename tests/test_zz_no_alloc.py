"""The no-allocation entry point det_splitk_gemm_noalloc (partials and
arrival counters in the library's per-device scratch) against
det_splitk_gemm with a caller workspace: the same bits, call after call,
with a smaller product following a larger one on both combine forms (the
last slice to arrive, which uses the counters, and the second streaming
launch over the slice roots)."""
import pytest
import torch

from helpers import assert_bitwise, assert_gemm_parity, dev_bf16
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def with_workspace(Xd, Wd, S, dev):
    M, K = Xd.shape
    N = Wd.shape[1]
    Y = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(Xd, Wd, Y, S, detred.workspace(M, N, K, S, dev))
    return Y


def noalloc(Xd, Wd, S, dev):
    Y = torch.full((Xd.shape[0], Wd.shape[1]), float("nan"), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm_noalloc(Xd, Wd, Y, S)
    return Y


# (M, N, K, S): narrow outputs below 65536 elements combine in the last
# arriving slice (counters); the others in a second launch over the roots
SEQUENCE = [
    (200, 64, 4096, 8),     # last arriver, 4 x 4 tiles of counters
    (16, 16, 512, 8),       # smaller, last arriver again
    (64, 4096, 4096, 0),    # roots + combine launch (automatic split)
    (8, 1024, 4096, 4),     # smaller, roots + combine
    (200, 64, 4096, 8),     # the first product again: same bits
    (33, 48, 4096, 2),      # ragged M, two slices, last arriver
]


def test_noalloc_matches_workspace_entry_point(dev):
    print("no-alloc sequence:", SEQUENCE, flush=True)
    first = None
    for i, (M, N, K, S) in enumerate(SEQUENCE):
        X, W = inputs.dense_inputs(M, K, N, seed=i % 4)
        Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
        ref = with_workspace(Xd, Wd, S, dev)
        # two calls in a row on the same scratch
        y1 = noalloc(Xd, Wd, S, dev)
        y2 = noalloc(Xd, Wd, S, dev)
        torch.cuda.synchronize()
        what = "noalloc %dx%dx%d S=%d" % (M, N, K, S)
        assert_bitwise(y1, ref, what)
        assert_bitwise(y2, ref, what + " (second call)")
        assert_gemm_parity(y1, X, W, rows=[0, M // 2, M - 1])
        if i == 0:
            first = y1
        if i == 4:
            assert_bitwise(y1, first, "the first product after the others")


def test_noalloc_rejects_beyond_its_scratch(dev):
    # 8 partial planes of 1024 x 1024 fp32 (32 MiB) exceed the scratch;
    # nothing is launched and Y keeps its contents
    X, W = inputs.dense_inputs(1024, 4096, 1024, seed=0)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    Y = torch.full((1024, 1024), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(detred.DetredError) as e:
        detred.det_splitk_gemm_noalloc(Xd, Wd, Y, 8)
    assert e.value.status == detred.EWORKSPACE
    torch.cuda.synchronize()
    assert bool((Y == 7.0).all())
    # the same product unsplit needs no scratch
    detred.det_splitk_gemm_noalloc(Xd, Wd, Y, 1)
    ref = with_workspace(Xd, Wd, 8, dev)
    torch.cuda.synchronize()
    assert_bitwise(Y, ref, "noalloc 1024x1024x4096 S=1 vs S=8 with a workspace")
