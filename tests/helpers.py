"""Shared helpers for the tests: device copies and the parity tolerances."""
import numpy as np
import torch

import oracle

# Parity bar for every fp32 product element: |gpu - oracle| <= 1e-5 * sum_k |x w| + 1e-6
GEMM_REL = 1e-5
GEMM_ABS = 1e-6


def dev_bf16(bits, device="cuda"):
    """uint16 bf16 bit patterns -> torch int16 GPU tensor with those bits."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)


def dev_f32(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def host(t):
    return t.detach().cpu().numpy()


def bits(t):
    """Bit patterns of an fp32 tensor/array as uint32 (for bitwise compares)."""
    a = host(t) if isinstance(t, torch.Tensor) else np.asarray(t)
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_gemm_parity(Y_gpu, X_bits, W_bits, rows=None):
    """Element-wise parity of a GPU product against the fp64 oracle, on all
    rows or on the given row indices (the oracle computes them one by one)."""
    Yg = host(Y_gpu).astype(np.float64)
    if rows is not None:
        X_bits = X_bits[rows]
        Yg = Yg[rows]
    Y, A = oracle.gemm(X_bits, W_bits)
    err = np.abs(Yg - Y)
    tol = GEMM_REL * A + GEMM_ABS
    bad = err > tol
    if bad.any():
        i, j = np.argwhere(bad)[0]
        raise AssertionError("parity: %d of %d elements out of tolerance; first at (%d,%d): "
                             "gpu %r oracle %r tol %r" % (bad.sum(), bad.size, i, j, Yg[i, j],
                                                          Y[i, j], tol[i, j]))
    return float((err / tol).max()) if err.size else 0.0


def assert_bitwise(a, b, what):
    ba, bb = bits(a), bits(b)
    if ba.shape != bb.shape:
        raise AssertionError("%s: shapes differ %s vs %s" % (what, ba.shape, bb.shape))
    diff = ba != bb
    if diff.any():
        idx = tuple(np.argwhere(diff)[0])
        raise AssertionError("%s: %d of %d elements differ bitwise; first at %s: %r vs %r" % (
            what, diff.sum(), diff.size, idx, ba.view(np.float32)[idx], bb.view(np.float32)[idx]))
