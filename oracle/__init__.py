"""CPU oracle: plain fp64 definitions of every operation on the hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library (``invariant_reduction_amd``) and never imports it; both are
fed by the seeded generators in ``invariant_reduction_amd.inputs``, which hold
none of the method's arithmetic.

Each wrapper marshals numpy arrays to the C functions in ``oracle.c`` and
cites the passage it follows there.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def lib():
    """Load liboracle.so, compiling it first if it is not there."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    L.oracle_bf16_to_f64.argtypes = [_u16p, _f64p, ctypes.c_size_t]
    L.oracle_bf16_to_f64.restype = None
    L.oracle_gemm_f64.argtypes = [_u16p, ctypes.c_long, _u16p, ctypes.c_long,
                                  _f64p, ctypes.c_void_p,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int]
    L.oracle_gemm_f64.restype = None
    L.oracle_rmsnorm_f64.argtypes = [_u16p, _u16p, _f64p, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_double]
    L.oracle_rmsnorm_f64.restype = None
    L.oracle_log_softmax_f64.argtypes = [_f32p, _f64p, ctypes.c_int, ctypes.c_int]
    L.oracle_log_softmax_f64.restype = None
    L.oracle_mean_f64.argtypes = [_f32p, _f64p, ctypes.c_int, ctypes.c_int]
    L.oracle_mean_f64.restype = None
    L.oracle_tree_sum_f32.argtypes = [_f32p, ctypes.c_int, ctypes.c_size_t, _f32p]
    L.oracle_tree_sum_f32.restype = ctypes.c_int
    L.oracle_fold_sum_f32.argtypes = [_f32p, ctypes.c_int]
    L.oracle_fold_sum_f32.restype = ctypes.c_float
    L.oracle_f32_to_bf16_rne.argtypes = [_f32p, _u16p, ctypes.c_size_t]
    L.oracle_f32_to_bf16_rne.restype = None
    L.oracle_decode_attention_f64.argtypes = [_u16p, _u16p, _u16p, ctypes.c_long, ctypes.c_long,
                                              ctypes.c_long, np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS"),
                                              _f64p, _f64p, _f64p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_double]
    L.oracle_decode_attention_f64.restype = None
    L.oracle_num_threads.argtypes = []
    L.oracle_num_threads.restype = ctypes.c_int
    _lib = L
    return L


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns as uint16, got %s" % a.dtype)
    return a


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns, as fp64."""
    b = _u16(bits)
    out = np.empty(b.shape, np.float64)
    lib().oracle_bf16_to_f64(b.reshape(-1), out.reshape(-1), b.size)
    return out


def gemm(X, W, with_magnitude=True):
    """Y = X W in fp64 with k increasing; also sum_k |x w| (oracle.c,
    oracle_gemm_f64).  X: [M,K] uint16 bf16 bits, W: [K,N] uint16.
    Returns (Y, A) as fp64 [M,N] arrays (A is None if not requested)."""
    X = _u16(X)
    W = _u16(W)
    M, K = X.shape
    K2, N = W.shape
    if K != K2:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    Y = np.empty((M, N), np.float64)
    A = np.empty((M, N), np.float64) if with_magnitude else None
    lib().oracle_gemm_f64(X, K, W, N, Y,
                          A.ctypes.data if A is not None else None, M, N, K)
    return Y, A


def addmm(X, W, C=None, alpha=1.0, beta=1.0):
    """y = beta*C + alpha*(X W) in fp64: the addmm of the "Batch Invariant
    Ops" project summary (Highlighted Details).  C is None, a length-N bias
    added to every row, or an [M,N] array.  Returns (Y, A) with
    A = |beta*C| + |alpha| * sum_k |x w|, the magnitude that scales the
    tolerance of a binary32 result."""
    P, Am = gemm(X, W)
    if C is None:
        Cm = np.zeros_like(P)
    else:
        Cm = np.asarray(C, dtype=np.float64)
        if Cm.ndim == 1:
            if Cm.shape[0] != P.shape[1]:
                raise ValueError("a bias must have one value per output column")
            Cm = np.broadcast_to(Cm[None, :], P.shape)
        elif Cm.shape != P.shape:
            raise ValueError("C must be [M, N]")
    Y = beta * Cm + alpha * P
    return Y, abs(beta) * np.abs(Cm) + abs(alpha) * Am


def lora_forward(X, W, Zb, B, scale):
    """The LoRA-adapted layer in fp64: Y = X W + scale * (Zb B), with Zb the
    bf16 bits of the shrink output X A after its cast ("Reproducible LoRA
    Inference Through Deterministic Split-K Reduction", Highlights and Q&A:
    the base product plus the expand of the shrink).  Returns (Y, A) with
    A = sum_k |x w| + |scale| * sum_l |z b|."""
    Yb, Ab = gemm(X, W)
    Ye, Ae = gemm(Zb, B)
    return Yb + scale * Ye, Ab + abs(scale) * Ae


def decode_attention(q, k, v, lens, scale, layout="bhtd"):
    """Decode attention in fp64 (oracle.c, oracle_decode_attention_f64):
    out[b][hq] = softmax_t(scale * q[b][hq] . k[b][hq // G][t]) weighted sum
    of v[b][hq // G][t] over t < lens[b].  q: [B,Hq,D] uint16 bf16 bits;
    k, v: uint16 [B,Hkv,L,D] (layout "bhtd") or [B,L,Hkv,D] ("bthd").
    Returns (out, A, S): out and A = sum_t w_t |v_td| / sum_t w_t as
    [B,Hq,D] fp64, and S = max_t |scale| * sum_d |q_d k_td| as [B,Hq]."""
    q = _u16(q)
    k = _u16(k)
    v = _u16(v)
    B, Hq, D = q.shape
    if layout == "bhtd":
        _, Hkv, L, _ = k.shape
        sb, sh, st = Hkv * L * D, L * D, D
    else:
        _, L, Hkv, _ = k.shape
        sb, sh, st = L * Hkv * D, D, Hkv * D
    if k.shape != v.shape or Hq % Hkv:
        raise ValueError("k and v must match and Hq must be a multiple of Hkv")
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    lens = np.minimum(lens, L).astype(np.int32)
    out = np.empty((B, Hq, D), np.float64)
    A = np.empty((B, Hq, D), np.float64)
    S = np.empty((B, Hq), np.float64)
    lib().oracle_decode_attention_f64(q.reshape(-1), k.reshape(-1), v.reshape(-1), sb, sh, st,
                                      lens, out.reshape(-1), A.reshape(-1), S.reshape(-1),
                                      B, Hq, Hkv, D, float(scale))
    return out, A, S


def rmsnorm(x, gamma, eps):
    """RMSNorm rows in fp64 (oracle.c, oracle_rmsnorm_f64)."""
    x = _u16(x)
    gamma = _u16(gamma)
    rows, H = x.shape
    if gamma.shape != (H,):
        raise ValueError("gamma must have shape (%d,)" % H)
    y = np.empty((rows, H), np.float64)
    lib().oracle_rmsnorm_f64(x, gamma, y, rows, H, float(eps))
    return y


def log_softmax(x):
    """log_softmax over the last dim in fp64 (oracle.c, oracle_log_softmax_f64)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    y = np.empty((rows, cols), np.float64)
    lib().oracle_log_softmax_f64(x, y, rows, cols)
    return y


def mean(x):
    """Mean over the last dim in fp64 (oracle.c, oracle_mean_f64)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x.shape
    y = np.empty((rows,), np.float64)
    lib().oracle_mean_f64(x, y, rows, cols)
    return y


def tree_sum_f32(P):
    """Fixed binary tree over axis 0 in binary32 (oracle.c,
    oracle_tree_sum_f32).  P: [S, ...] float32, S a power of two."""
    P = np.ascontiguousarray(P, dtype=np.float32)
    S = P.shape[0]
    n = P[0].size
    Y = np.empty(P.shape[1:], np.float32)
    rc = lib().oracle_tree_sum_f32(P.reshape(-1), S, n, Y.reshape(-1))
    if rc != 0:
        raise ValueError("S must be a power of two in 1..64, got %d" % S)
    return Y


def fold_sum_f32(v):
    """Left-to-right binary32 sum (oracle.c, oracle_fold_sum_f32)."""
    v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    return np.float32(lib().oracle_fold_sum_f32(v, v.size))


def f32_to_bf16(x):
    """binary32 -> bf16 bits, round to nearest even (oracle.c,
    oracle_f32_to_bf16_rne)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().oracle_f32_to_bf16_rne(x.reshape(-1), y.reshape(-1), x.size)
    return y


def num_threads():
    """Threads the oracle's OpenMP loops run on."""
    return int(lib().oracle_num_threads())
