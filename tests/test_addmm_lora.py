"""GPU parity of the addmm epilogue, the bf16 outputs and the LoRA layer.

det_splitk_addmm: y = beta*C + alpha*p with p the canonical product, fp32
or bf16 output.  Parity against the fp64 oracle (oracle.addmm) within
1e-5 * (|beta c| + |alpha| sum_k |x w|) + 1e-6; bits independent of the
split and of M; with alpha, beta powers of two the result must equal
det_splitk_gemm followed by the same two fp32 operations bit for bit.  A bf16
output is the rounding of the fp32 output: both sides take that decision
on the same binary32 value, so it is compared bit for bit through the
oracle's own rounding.  The LoRA layer must equal its steps run one by
one, bit for bit, and the fp32 form of its last step must meet the oracle's
tolerance."""
import numpy as np
import pytest
import torch

import oracle
from helpers import GEMM_ABS, GEMM_REL, assert_bitwise, dev_bf16, dev_f32, host
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu


def check_tol(Yg, Y, A, what):
    Yg = np.asarray(Yg, dtype=np.float64)
    err = np.abs(Yg - Y)
    tol = GEMM_REL * A + GEMM_ABS
    bad = err > tol
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d out of tolerance; first (%d,%d) gpu %r oracle %r tol %r"
                             % (what, bad.sum(), bad.size, i, j, Yg[i, j], Y[i, j], tol[i, j]))


def u16(t):
    return host(t).view(np.uint16)


def addmm(Xd, Wd, C, alpha, beta, S, dev, out=torch.float32):
    M, N = Xd.shape[0], Wd.shape[1]
    K = Xd.shape[1]
    Y = torch.full((M, N), -1, dtype=torch.int16, device=dev) if out != torch.float32 else \
        torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    ws = detred.workspace(M, N, K, S, dev)
    detred.det_splitk_addmm(Xd, Wd, Y, C, alpha, beta, S, ws)
    return Y


# (M, N, K): the LDS-DMA engine (wide N, 8 chunks), the register engines
# (N <= 64, N <= 16) and one-chunk K, with ragged M and N
SHAPES = [(100, 392, 2048), (37, 40, 1024), (50, 16, 512), (33, 200, 96), (1, 4096, 256)]
COEFS = [(1.0, 1.0), (0.5, -2.0), (-1.25, 0.75)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_addmm_parity_and_split_invariance(M, N, K, dev):
    X, W = inputs.dense_inputs(M, K, N, seed=M + 3 * N + K)
    bias = inputs.bias_inputs(N, seed=N)
    Cfull = inputs.normal_f32((M, N), 0.0, 2.0, 9, 7)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    P = detred.policy(N, K)["chunks"]
    for C in (None, bias, Cfull):
        Cd = None if C is None else dev_f32(C, dev)
        for alpha, beta in COEFS:
            Y, A = oracle.addmm(X, W, C, alpha, beta)
            ref = None
            for S in [s for s in (1, 2, 8) if s <= P]:
                Yg = addmm(Xd, Wd, Cd, alpha, beta, S, dev)
                torch.cuda.synchronize()
                check_tol(host(Yg), Y, A, "addmm S=%d alpha=%g beta=%g C=%s" % (
                    S, alpha, beta, None if C is None else C.shape))
                if ref is None:
                    ref = Yg
                else:
                    assert_bitwise(Yg, ref, "addmm S=%d vs S=1" % S)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_addmm_is_gemm_then_two_fp32_ops(M, N, K, dev):
    # alpha, beta powers of two: beta*c and alpha*p are exact, so the
    # epilogue is one binary32 addition of the det product and beta*C
    X, W = inputs.dense_inputs(M, K, N, seed=7 * M + N)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    C = dev_f32(inputs.normal_f32((M, N), 0.0, 1.0, 4, 8), dev)
    bias = dev_f32(inputs.bias_inputs(N, seed=2), dev)
    S = detred.policy(N, K)["chunks"]
    Yp = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(Xd, Wd, Yp, S, detred.workspace(M, N, K, S, dev))
    for Cd, Cb in ((C, C), (bias, bias[None, :].expand(M, N))):
        Yg = addmm(Xd, Wd, Cd, 0.5, 2.0, S, dev)
        assert_bitwise(Yg, 2.0 * Cb + 0.5 * Yp, "addmm vs gemm + epilogue")
    Yg = addmm(Xd, Wd, None, -4.0, 1.0, 0, dev)
    assert_bitwise(Yg, -4.0 * Yp, "addmm without C")


def test_addmm_strided_c_and_y(dev):
    M, N, K = 70, 264, 1024
    X, W = inputs.dense_inputs(M, K, N, seed=5)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    Cbig = dev_f32(inputs.normal_f32((M, N + 40), 0.0, 1.0, 1, 9), dev)
    C = Cbig[:, 8:8 + N]
    Ybig = torch.full((M, N + 24), 7.0, dtype=torch.float32, device=dev)
    Y = Ybig[:, 16:16 + N]
    detred.det_splitk_addmm(Xd, Wd, Y, C, 1.0, 1.0, 8, detred.workspace(M, N, K, 8, dev))
    torch.cuda.synchronize()
    Yo, A = oracle.addmm(X, W, host(C), 1.0, 1.0)
    check_tol(host(Y), Yo, A, "strided addmm")
    assert torch.all(Ybig[:, :16] == 7.0) and torch.all(Ybig[:, 16 + N:] == 7.0)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_addmm_bf16_output_is_rounded_fp32_output(M, N, K, dev):
    X, W = inputs.dense_inputs(M, K, N, seed=11 * M + N)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    bias = dev_f32(inputs.bias_inputs(N, seed=3), dev)
    P = detred.policy(N, K)["chunks"]
    for S in [s for s in (1, 8) if s <= P]:
        Yf = addmm(Xd, Wd, bias, 0.75, 1.0, S, dev)
        Yb = addmm(Xd, Wd, bias, 0.75, 1.0, S, dev, out=torch.int16)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(u16(Yb), oracle.f32_to_bf16(host(Yf)))


@pytest.mark.parametrize("M,N,K", [(384, 14336, 4096), (1280, 4096, 4096)])
def test_addmm_automatic_split_bf16_and_fp32(M, N, K, dev):
    """At these shapes the automatic split keeps one slice for an fp32
    output (one round of 192x128 tiles) but splits an addmm into bf16,
    which cannot take that tile; one workspace sized for split 0 serves both
    calls, and the bf16 output is the fp32 output rounded to nearest even."""
    assert detred.auto_split(M, N, K) == 1
    X, W = inputs.dense_inputs(M, K, N, seed=13)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    bias = dev_f32(inputs.bias_inputs(N, seed=4), dev)
    ws = detred.workspace(M, N, K, 0, dev)
    assert ws is not None and ws.numel() == detred.detred_gemm_workspace_bytes(M, N, K, 2)
    Yf = torch.empty((M, N), dtype=torch.float32, device=dev)
    Yb = torch.empty((M, N), dtype=torch.int16, device=dev)
    detred.det_splitk_addmm(Xd, Wd, Yf, bias, 0.75, 1.0, 0, ws)
    detred.det_splitk_addmm(Xd, Wd, Yb, bias, 0.75, 1.0, 0, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u16(Yb), oracle.f32_to_bf16(host(Yf)))


def test_addmm_integer_inputs_exact(dev):
    # integer inputs and C, dyadic coefficients: every value exact in fp32
    M, N, K = 129, 264, 2048
    X = inputs.integer_bf16((M, K), -8, 8, 1, 0)
    W = inputs.integer_bf16((K, N), -8, 8, 1, 1)
    C = inputs.integer_f32((M, N), -100, 100, 1, 2)
    Xd, Wd, Cd = dev_bf16(X, dev), dev_bf16(W, dev), dev_f32(C, dev)
    Y, _ = oracle.addmm(X, W, C, 0.5, -2.0)
    for S in (1, 4, 8):
        Yg = addmm(Xd, Wd, Cd, 0.5, -2.0, S, dev)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(Yg).astype(np.float64), Y)


def test_addmm_batch_invariance(dev):
    M, N, K = 300, 520, 2048
    X, W = inputs.dense_inputs(M, K, N, seed=21)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    bias = dev_f32(inputs.bias_inputs(N, seed=5), dev)
    full = addmm(Xd, Wd, bias, 1.0, 1.0, 0, dev, out=torch.int16)
    for m in (1, 7, 128, 129, 257):
        part = addmm(Xd[:m].contiguous(), Wd, bias, 1.0, 1.0, 0, dev, out=torch.int16)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(u16(part), u16(full)[:m])


def test_addmm_empty_k(dev):
    M, N = 9, 40
    X = torch.empty((M, 0), dtype=torch.int16, device=dev)
    W = torch.empty((0, N), dtype=torch.int16, device=dev)
    C = dev_f32(inputs.normal_f32((M, N), 0.0, 1.0, 2, 3), dev)
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    detred.det_splitk_addmm(X, W, Y, C, 3.0, -0.5)
    torch.cuda.synchronize()
    assert_bitwise(Y, -0.5 * C + 0.0, "addmm K=0")


# --- bf16 RMSNorm ---------------------------------------------------------------

@pytest.mark.parametrize("B,H", [(1, 4096), (37, 4096), (256, 4096), (5, 8)])
def test_rmsnorm_bf16_is_rounded_fp32(B, H, dev):
    x, g = inputs.rmsnorm_inputs(B, H, seed=B + H)
    xd, gd = dev_bf16(x, dev), dev_bf16(g, dev)
    yf = torch.empty((B, H), dtype=torch.float32, device=dev)
    yb = torch.empty((B, H), dtype=torch.int16, device=dev)
    detred.inv_rmsnorm(xd, gd, yf, 1e-6)
    detred.inv_rmsnorm_bf16(xd, gd, yb, 1e-6)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u16(yb), oracle.f32_to_bf16(host(yf)))
    if B > 1:
        y1 = torch.empty((1, H), dtype=torch.int16, device=dev)
        detred.inv_rmsnorm_bf16(xd[B - 1:].contiguous(), gd, y1, 1e-6)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(u16(y1)[0], u16(yb)[B - 1])


# --- the LoRA layer ---------------------------------------------------------------

LORA = [(5, 512, 1024, 16, 2.0), (64, 2048, 2048, 64, 0.5), (256, 4096, 4096, 64, 1.0)]


@pytest.mark.parametrize("M,N,K,r,scale", LORA)
def test_lora_forward_steps_and_parity(M, N, K, r, scale, dev):
    X, W, A, B = inputs.lora_layer_inputs(M, K, N, r, seed=M + r)
    Xd, Wd, Ad, Bd = (dev_bf16(t, dev) for t in (X, W, A, B))
    Y = torch.full((M, N), -1, dtype=torch.int16, device=dev)
    detred.det_lora_forward(Xd, Wd, Ad, Bd, Y, scale, detred.lora_workspace(M, N, K, r, dev))
    # the steps one by one, the cast of the shrink as its own call
    base = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(Xd, Wd, base, 0, detred.workspace(M, N, K, 0, dev))
    z = torch.empty((M, r), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(Xd, Ad, z, 0, detred.workspace(M, r, K, 0, dev))
    zb = torch.empty((M, r), dtype=torch.int16, device=dev)
    detred.detred_f32_to_bf16(z, zb)
    Yf = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_addmm(zb, Bd, Yf, base, scale, 1.0)
    Yb = torch.empty((M, N), dtype=torch.int16, device=dev)
    detred.det_splitk_addmm(zb, Bd, Yb, base, scale, 1.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(u16(Y), u16(Yb))
    # the bf16 result is the rounding of the fp32 one, which meets the
    # oracle on the same bf16 shrink (the cast is a rounding decision taken
    # on the GPU's binary32 shrink; it is itself checked bit for bit)
    np.testing.assert_array_equal(u16(zb), oracle.f32_to_bf16(host(z)))
    np.testing.assert_array_equal(u16(Y), oracle.f32_to_bf16(host(Yf)))
    rows = np.arange(M) if M <= 64 else np.array([0, 1, 127, 128, M - 1])
    Yo, Ao = oracle.lora_forward(X[rows], W, u16(zb)[rows], B, scale)
    check_tol(host(Yf)[rows], Yo, Ao, "lora fp32")


def test_lora_forward_batch_invariance(dev):
    M, N, K, r = 96, 1024, 2048, 64
    X, W, A, B = inputs.lora_layer_inputs(M, K, N, r, seed=3)
    Xd, Wd, Ad, Bd = (dev_bf16(t, dev) for t in (X, W, A, B))
    full = torch.empty((M, N), dtype=torch.int16, device=dev)
    detred.det_lora_forward(Xd, Wd, Ad, Bd, full, 2.0, detred.lora_workspace(M, N, K, r, dev))
    for m in (1, 17, 64):
        part = torch.empty((m, N), dtype=torch.int16, device=dev)
        detred.det_lora_forward(Xd[:m].contiguous(), Wd, Ad, Bd, part, 2.0,
                                detred.lora_workspace(m, N, K, r, dev))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(u16(part), u16(full)[:m])


@pytest.mark.parametrize("S", [2, 4, 8])
def test_addmm_bf16_into_padded_rows_every_split(S, dev):
    """bf16 output into rows ldy > N apart with a bias, on the wide tile (the
    split's roots combined by the second launch, which applies the
    epilogue): the same bits as S = 1, nothing written past the rows."""
    M, N, K = 300, 1032, 4096
    X, W = inputs.dense_inputs(M, K, N, seed=S)
    Xd, Wd = dev_bf16(X, dev), dev_bf16(W, dev)
    bias = dev_f32(inputs.bias_inputs(N, seed=4), dev)
    ref = addmm(Xd, Wd, bias, 0.75, 1.0, 1, dev, out=torch.int16)
    Ybig = torch.full((M, N + 24), 77, dtype=torch.int16, device=dev)
    Y = Ybig[:, 8:8 + N]
    detred.det_splitk_addmm(Xd, Wd, Y, bias, 0.75, 1.0, S, detred.workspace(M, N, K, S, dev))
    torch.cuda.synchronize()
    assert torch.equal(Y, ref), "bf16 addmm into padded rows, S=%d" % S
    assert torch.all(Ybig[:, :8] == 77) and torch.all(Ybig[:, 8 + N:] == 77)
