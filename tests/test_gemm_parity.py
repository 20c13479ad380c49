"""GPU parity of the GEMM entry points against the fp64 oracle.

Random bf16 inputs must meet |gpu - oracle| <= 1e-5 * sum_k |x w| + 1e-6 per
element; integer-valued inputs (every partial sum exact in fp32) must match
bit for bit at the workloads' full shapes; the last-arriver combine must
equal the oracle's fp32 tree over the partials it read."""
import numpy as np
import pytest
import torch

import oracle
from helpers import (assert_bitwise, assert_gemm_parity, dev_bf16, dev_f32, host)
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def run_det(X, W, S, dev):
    M, K = X.shape
    N = W.shape[1]
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    ws = detred.workspace(M, N, K, S, dev)
    detred.det_splitk_gemm(X, W, Y, S, ws)
    return Y, ws


# shapes spanning several tiles with ragged tails in M and N, one-chunk and
# eight-chunk K, for each tile family (N <= 16, N <= 64, larger N)
SHAPES = [
    (1, 16, 512), (16, 16, 512), (70, 16, 768), (5, 8, 256),
    (33, 64, 2304), (130, 40, 512), (64, 56, 1024),
    (1, 264, 512), (129, 136, 768), (200, 264, 2048), (17, 4096, 64), (33, 520, 16),
    (65, 72, 200), (3, 24, 8),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_det_parity_random(M, N, K, dev):
    X, W = inputs.dense_inputs(M, K, N, seed=M * 7 + N + K)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    P = detred.policy(N, K)["chunks"]
    ref = None
    for S in [s for s in (1, 2, 4, 8) if s <= P]:
        Y, _ = run_det(Xd, Wd, S, dev)
        torch.cuda.synchronize()
        assert_gemm_parity(Y, X, W)
        if ref is None:
            ref = Y
        else:
            assert_bitwise(Y, ref, "det S=%d vs S=1" % S)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_atomic_and_tp_parity_random(M, N, K, dev):
    X, W = inputs.dense_inputs(M, K, N, seed=M * 5 + N + 3 * K)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    P = detred.policy(N, K)["chunks"]
    det, _ = run_det(Xd, Wd, 1, dev)
    for S in [s for s in (1, 2, 4, 8) if s <= P]:
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        detred.atomic_splitk_gemm(Xd, Wd, Y, S)
        torch.cuda.synchronize()
        assert_gemm_parity(Y, X, W)
        Yt = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
        ws = detred.workspace(M, N, K, S, dev)
        detred.tree_tp_gemm(Xd, Wd, Yt, S, ws)
        torch.cuda.synchronize()
        assert_bitwise(Yt, det, "tree_tp T=%d vs det" % S)


def test_strided_operands(dev):
    """Leading dimensions larger than the row length."""
    M, N, K = 37, 72, 512
    X, W = inputs.dense_inputs(M, K, N, seed=4)
    Xbig = torch.zeros((M, K + 64), dtype=torch.int16, device=dev)
    Wbig = torch.zeros((K, N + 24), dtype=torch.int16, device=dev)
    Xbig[:, :K] = dev_bf16(X, dev)
    Wbig[:, :N] = dev_bf16(W, dev)
    Ybig = torch.full((M, N + 8), -7.0, dtype=torch.float32, device=dev)
    for S in (1, 4, 8):
        ws = detred.workspace(M, N, K, S, dev)
        detred.det_splitk_gemm(Xbig[:, :K], Wbig[:, :N], Ybig[:, :N], S, ws)
        torch.cuda.synchronize()
        assert_gemm_parity(Ybig[:, :N], X, W)
        assert torch.all(Ybig[:, N:] == -7.0), "wrote past the row"
    Yt = torch.full((M, N + 8), -7.0, dtype=torch.float32, device=dev)
    ws = detred.workspace(M, N, K, 4, dev)
    detred.tree_tp_gemm(Xbig[:, :K], Wbig[:, :N], Yt[:, :N], 4, ws)
    torch.cuda.synchronize()
    assert_bitwise(Yt[:, :N], Ybig[:, :N], "strided tree_tp vs det")
    assert torch.all(Yt[:, N:] == -7.0)


@pytest.mark.parametrize("M,N,K", [(300, 264, 2048), (5, 1032, 8192)])
def test_tree_tp_padded_output(M, N, K, dev):
    """tree_tp_gemm into rows ldy > N apart: the cross-shard combine walks
    the padded rows, writes nothing past N and gives det's bits for every T."""
    X, W = inputs.dense_inputs(M, K, N, seed=M + N)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    ref = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(Xd, Wd, ref, 1, detred.workspace(M, N, K, 1, dev))
    for T in (2, 4, 8):
        Yp = torch.full((M, N + 24), -7.0, dtype=torch.float32, device=dev)
        detred.tree_tp_gemm(Xd, Wd, Yp[:, :N], T, detred.workspace(M, N, K, T, dev))
        torch.cuda.synchronize()
        assert_bitwise(Yp[:, :N], ref, "padded tree_tp T=%d vs det" % T)
        assert torch.all(Yp[:, N:] == -7.0), "wrote past the row"
    assert_gemm_parity(ref, X, W, rows=[0, M // 2, M - 1])


def test_combine_equals_cpu_tree_over_partials(dev):
    """det S=8: Y is exactly the fp32 tree ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7))
    over the slice partials left in the workspace (layout: S planes of M*N)."""
    for (M, N, K) in [(16, 16, 512), (256, 64, 4096), (100, 264, 1024)]:
        X, W = inputs.dense_inputs(M, K, N, seed=1)
        Y, ws = run_det(dev_bf16(X, dev), dev_bf16(W, dev), 8, dev)
        torch.cuda.synchronize()
        parts = host(ws[: 8 * M * N * 4].view(torch.float32)).reshape(8, M, N)
        assert_bitwise(Y, oracle.tree_sum_f32(parts), "Y vs CPU tree over partials")
        for S in (2, 4):
            Ys, wss = run_det(dev_bf16(X, dev), dev_bf16(W, dev), S, dev)
            torch.cuda.synchronize()
            ps = host(wss[: S * M * N * 4].view(torch.float32)).reshape(S, M, N)
            assert_bitwise(Ys, oracle.tree_sum_f32(ps), "S=%d partial tree" % S)
            # slice s of S is the subtree over partials [s*8/S, (s+1)*8/S) of S=8
            for s in range(S):
                assert_bitwise(ps[s], oracle.tree_sum_f32(parts[s * 8 // S:(s + 1) * 8 // S]),
                               "S=%d slice %d as subtree of the 8 chunks" % (S, s))


# --- integer-valued inputs: exact in every order, so bit-exact vs oracle ---

FULL_SHAPES = [
    ("lora shrink 16x512x16", 16, 16, 512, None),
    ("lora shrink r16", 256, 16, 4096, None),
    ("lora shrink r64", 256, 64, 4096, None),
    ("lora expand r64", 256, 4096, 64, None),
    ("lora expand r16", 256, 4096, 16, None),
    ("dense 4096x4096x14336", 4096, 14336, 4096, [0, 1, 127, 128, 2047, 4095]),
    ("tp 512x8192x8192", 512, 8192, 8192, [0, 255, 511]),
]


@pytest.mark.parametrize("name,M,N,K,rows", FULL_SHAPES, ids=[s[0] for s in FULL_SHAPES])
def test_integer_inputs_bit_exact(name, M, N, K, rows, dev):
    X = inputs.integer_bf16((M, K), -8, 8, 11, 0)
    W = inputs.integer_bf16((K, N), -8, 8, 11, 1)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    sel = rows if rows is not None else list(range(M))
    Yo, _ = oracle.gemm(X[sel], W, with_magnitude=False)
    want = Yo.astype(np.float32)
    assert np.all(Yo == want), "integer oracle result not exact in fp32"
    P = detred.policy(N, K)["chunks"]
    for S in [s for s in (1, 2, 4, 8) if s <= P]:
        Y, _ = run_det(Xd, Wd, S, dev)
        torch.cuda.synchronize()
        assert_bitwise(host(Y)[sel], want, "%s det S=%d" % (name, S))
        del Y
        Ya = torch.empty((M, N), dtype=torch.float32, device=dev)
        detred.atomic_splitk_gemm(Xd, Wd, Ya, S)
        torch.cuda.synchronize()
        assert_bitwise(host(Ya)[sel], want, "%s atomic S=%d" % (name, S))
        del Ya


def test_identity_weight(dev):
    X, _ = inputs.dense_inputs(64, 512, 8, seed=3)
    eye = inputs.f32_bits_to_bf16_bits(np.eye(512, dtype=np.float32))
    for S in (1, 8):
        Y, _ = run_det(dev_bf16(X, dev), dev_bf16(eye, dev), S, dev)
        torch.cuda.synchronize()
        assert_bitwise(Y, inputs.bf16_bits_to_f32(X), "X I == X, S=%d" % S)


def test_k_zero_and_empty(dev):
    X = torch.empty((5, 0), dtype=torch.int16, device=dev)
    W = torch.empty((0, 16), dtype=torch.int16, device=dev)
    Y = torch.full((5, 16), 3.0, device=dev)
    detred.det_splitk_gemm(X, W, Y, 1)
    torch.cuda.synchronize()
    assert torch.all(Y == 0) and not torch.any(torch.signbit(Y))
    Y.fill_(3.0)
    detred.atomic_splitk_gemm(X, W, Y, 1)
    torch.cuda.synchronize()
    assert torch.all(Y == 0)
    Xe = torch.empty((0, 512), dtype=torch.int16, device=dev)
    We = torch.zeros((512, 16), dtype=torch.int16, device=dev)
    detred.det_splitk_gemm(Xe, We, torch.empty((0, 16), device=dev), 8, None)


def test_lora_shrink_cast_expand(dev):
    """Shrink (det, S=8) -> explicit bf16 cast -> expand, each step checked:
    the cast bit-exact against the oracle's nearest-even rounding of the GPU
    shrink output, the expand against the oracle on that same bf16 tensor."""
    for (M, r) in [(1, 16), (8, 64), (64, 16), (256, 64)]:
        X, A, B = inputs.lora_inputs(M, 4096, r, seed=0)
        Xd, Ad, Bd = dev_bf16(X, dev), dev_bf16(A, dev), dev_bf16(B, dev)
        Ys, _ = run_det(Xd, Ad, 8, dev)
        Yb = torch.empty((M, r), dtype=torch.int16, device=dev)
        detred.detred_f32_to_bf16(Ys, Yb)
        Z = torch.empty((M, 4096), dtype=torch.float32, device=dev)
        detred.det_splitk_gemm(Yb, Bd, Z, 0)
        torch.cuda.synchronize()
        assert_gemm_parity(Ys, X, A)
        yb = host(Yb).view(np.uint16)
        np.testing.assert_array_equal(yb, oracle.f32_to_bf16(host(Ys)))
        assert_gemm_parity(Z, yb, B)


def test_cast_matches_oracle(dev):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(4096) * 10.0 ** rng.integers(-20, 20, 4096)).astype(np.float32)
    ties = ((rng.integers(0, 2 ** 31, 1024, dtype=np.uint32) & 0x7F7F0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 3.4e38, -3.4e38, 1e-40],
                                          np.float32)])
    x = np.concatenate([x, np.zeros((-x.size) % 8, np.float32)])
    y = torch.empty(x.size, dtype=torch.int16, device=dev)
    detred.detred_f32_to_bf16(dev_f32(x, dev), y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(y).view(np.uint16), oracle.f32_to_bf16(x))


def test_rank_shard_on_root_tile_into_padded_rows(dev):
    """One rank's shard large enough for the 256x256 root tile (2048 x 8192
    output, one chunk of 1024 per shard at T = 8), its root stored straight
    from the registers into rows ldp > N apart: the bits of the contiguous
    call, nothing written past the rows."""
    M, N, Kt, T = 2048, 8192, 1024, 8
    X, W = inputs.dense_inputs(M, Kt, N, seed=17)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    ref = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.tree_tp_shard_gemm(Xd, Wd, ref, T)
    Pbig = torch.full((M, N + 8), -3.0, dtype=torch.float32, device=dev)
    detred.tree_tp_shard_gemm(Xd, Wd, Pbig[:, :N], T)
    torch.cuda.synchronize()
    assert_bitwise(Pbig[:, :N], ref, "shard root into padded rows")
    assert torch.all(Pbig[:, N:] == -3.0), "wrote past the row"
    assert_gemm_parity(ref, X, W, rows=[0, 1023, 2047])
