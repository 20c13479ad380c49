"""ctypes binding of libdetred (include/detred.h).

Argument marshalling only: each function takes torch tensors, checks dtypes
and devices, and passes raw device pointers, leading dimensions and the
current HIP stream to the C entry point of the same name.  Every operation
runs in the library's HIP kernels; there is no fallback.  A non-OK status
raises DetredError.

bf16 tensors may be given as torch.bfloat16, torch.int16 or torch.uint16
(the bit patterns are what the library reads).
"""
import ctypes
import os

import torch

from . import build as _build

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1

_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_Z = ctypes.c_size_t
_F = ctypes.c_float

# name -> argument types, in header order
SIGNATURES = {
    "detred_status_string": ([_I], ctypes.c_char_p),
    "detred_version": ([], _I),
    "detred_policy": ([_I, _I, _P, _P, _P, _P, _P], _I),
    "detred_auto_split": ([_I, _I, _I], _I),
    "detred_gemm_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "detred_workspace_init": ([_P, _Z, _P], _I),
    "det_splitk_gemm": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P, _Z, _P], _I),
    "det_splitk_addmm": ([_P, _I, _P, _I, _P, _I, _F, _F, _P, _I, _I, _I, _I, _I, _I, _P, _Z,
                          _P], _I),
    "det_splitk_gemm_wt": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P, _Z, _P], _I),
    "det_splitk_addmm_wt": ([_P, _I, _P, _I, _P, _I, _F, _F, _P, _I, _I, _I, _I, _I, _I, _P, _Z,
                             _P], _I),
    "det_splitk_gemm_noalloc": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P], _I),
    "det_lora_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "det_lora_forward": ([_P, _I, _P, _I, _P, _I, _P, _I, _F, _P, _I, _I, _I, _I, _I, _P, _Z,
                          _P], _I),
    "atomic_splitk_gemm": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P], _I),
    "tree_tp_gemm": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P, _Z, _P], _I),
    "tree_tp_shards_gemm": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _P], _I),
    "tree_tp_shard_gemm": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P], _I),
    "tree_tp_gemm_wt": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P, _Z, _P], _I),
    "tree_tp_shards_gemm_wt": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _P], _I),
    "tree_tp_shard_gemm_wt": ([_P, _I, _P, _I, _P, _I, _I, _I, _I, _I, _P], _I),
    "tree_combine_f32": ([_P, _Z, _I, _P, _Z, _P], _I),
    "detred_f32_to_bf16": ([_P, _P, _Z, _P], _I),
    "inv_rmsnorm": ([_P, _P, _P, _I, _I, _F, _P], _I),
    "inv_rmsnorm_bf16": ([_P, _P, _P, _I, _I, _F, _P], _I),
    "inv_log_softmax": ([_P, _P, _I, _I, _P], _I),
    "inv_mean": ([_P, _P, _I, _I, _P], _I),
    "inv_log_softmax_mean": ([_P, _P, _P, _I, _I, _P], _I),
    "inv_decode_attention_workspace_bytes": ([_I, _I, _I, _I], _Z),
    "inv_decode_attention": ([_P, _P, _P, ctypes.c_long, ctypes.c_long, ctypes.c_long, _P, _P,
                              _I, _I, _I, _I, _I, _F, _P, _Z, _P], _I),
}


class DetredError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s" % (where, status_string(status)))


def lib_path():
    return _build.LIB


def lib():
    """Load libdetred.so, building it first if it is not there.  Raises if
    the library cannot be built or loaded: there is no other path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    L = ctypes.CDLL(_build.LIB)
    for name, (args, res) in SIGNATURES.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def status_string(status):
    return lib().detred_status_string(int(status)).decode()


def _check(status, where):
    if status != OK:
        raise DetredError(status, where)


def _entry(marshal):
    """Turn a marshaller (torch arguments -> C name and ctypes arguments)
    into the public call; ``prepare`` keeps the marshalled arguments for
    repeated launches without re-marshalling."""
    def call(*args, **kw):
        name, cargs = marshal(*args, **kw)
        _check(getattr(lib(), name)(*cargs), name)
    call.__name__ = marshal.__name__
    call.__doc__ = marshal.__doc__
    call.marshal = marshal
    return call


def prepare(fn, *args, **kw):
    """Marshal once; return a zero-argument callable that issues the same C
    call (same pointers, sizes and stream) each time it is called.  The
    callable holds references to the tensors it was given (a workspace
    created inline stays allocated as long as the callable exists)."""
    name, cargs = fn.marshal(*args, **kw)
    cfun = getattr(lib(), name)

    def launch():
        st = cfun(*cargs)
        if st != OK:
            raise DetredError(st, name)
    launch.tensors = (args, kw)
    return launch


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_BF16_TYPES = (torch.bfloat16, torch.int16, torch.uint16)


def _mat(t, dtypes, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dim() != 2 or (t.shape[0] > 1 and t.stride(1) != 1) or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("%s must be a row-major matrix with unit column stride" % name)
    ld = t.stride(0) if t.shape[0] > 1 else t.shape[1]
    return ctypes.c_void_p(t.data_ptr()), int(ld)


def _weight(W):
    """The right operand of a product: a row-major [K, N] matrix, or a
    [K, N] view of a row-major [N, K] matrix (W = Wt.t(), as a linear
    layer's weight is used).  Returns (pointer, leading dimension,
    transposed)."""
    if not isinstance(W, torch.Tensor):
        raise TypeError("W must be a torch tensor")
    if W.dim() == 2 and W.shape[0] > 1 and W.shape[1] > 1 and W.stride(0) == 1 and W.stride(1) != 1:
        if W.dtype not in _BF16_TYPES:
            raise TypeError("W has dtype %s, expected one of %s" % (W.dtype, _BF16_TYPES))
        if not W.is_cuda:
            raise ValueError("W must be a GPU tensor")
        return ctypes.c_void_p(W.data_ptr()), int(W.stride(1)), True
    pw, ldw = _mat(W, _BF16_TYPES, "W")
    return pw, ldw, False


def policy(N, K):
    """The locked policy for (N, K): dict with chunks, chunk_k, tile_m,
    tile_n, default_split."""
    vals = [ctypes.c_int() for _ in range(5)]
    _check(lib().detred_policy(N, K, *[ctypes.byref(v) for v in vals]), "detred_policy")
    keys = ["chunks", "chunk_k", "tile_m", "tile_n", "default_split"]
    return {k: v.value for k, v in zip(keys, vals)}


detred_policy = policy


def detred_auto_split(M, N, K):
    """The split that split_k = 0 selects (it never changes the bits)."""
    return int(lib().detred_auto_split(M, N, K))


auto_split = detred_auto_split


def detred_gemm_workspace_bytes(M, N, K, split_or_shards):
    return int(lib().detred_gemm_workspace_bytes(M, N, K, split_or_shards))


def detred_workspace_init(ws, stream=None):
    _check(lib().detred_workspace_init(ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                       _stream(stream)), "detred_workspace_init")


def workspace(M, N, K, split_or_shards, device="cuda", stream=None):
    """Allocate (through torch) and zero a workspace for an M x N x K
    product with the given split or shard count (0: the automatic split);
    None when none is needed."""
    nbytes = detred_gemm_workspace_bytes(M, N, K, split_or_shards)
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("torch returned a workspace that is not 256-byte aligned")
    detred_workspace_init(ws, stream)
    return ws


def _ws(ws):
    if ws is None:
        return ctypes.c_void_p(None), 0
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _gemm_dims(X, W, Y):
    M, K = X.shape
    K2, N = W.shape
    if K2 != K or tuple(Y.shape) != (M, N):
        raise ValueError("shape mismatch: X %s, W %s, Y %s" % (tuple(X.shape), tuple(W.shape), tuple(Y.shape)))
    return M, N, K


@_entry
def det_splitk_gemm(X, W, Y, split_k=0, ws=None, stream=None):
    """Y[M,N] (fp32) = X[M,K] W[K,N] (bf16) with the fixed chunk tree.  W may
    be the transpose view of a row-major [N, K] weight (det_splitk_gemm_wt;
    same bits)."""
    px, ldx = _mat(X, _BF16_TYPES, "X")
    pw, ldw, wt = _weight(W)
    py, ldy = _mat(Y, (torch.float32,), "Y")
    M, N, K = _gemm_dims(X, W, Y)
    pws, nws = _ws(ws)
    return ("det_splitk_gemm_wt" if wt else "det_splitk_gemm"), (
        px, ldx, pw, ldw, py, ldy, M, N, K, split_k, pws, nws, _stream(stream))


@_entry
def det_splitk_gemm_noalloc(X, W, Y, split_k=0, stream=None):
    """det_splitk_gemm with no workspace argument: the partials live in the
    library's per-device scratch (for callers that cannot allocate).  W is a
    row-major [K, N] matrix.  Same bits as det_splitk_gemm."""
    px, ldx = _mat(X, _BF16_TYPES, "X")
    pw, ldw = _mat(W, _BF16_TYPES, "W")
    py, ldy = _mat(Y, (torch.float32,), "Y")
    M, N, K = _gemm_dims(X, W, Y)
    return "det_splitk_gemm_noalloc", (px, ldx, pw, ldw, py, ldy, M, N, K, split_k,
                                       _stream(stream))


@_entry
def det_splitk_addmm(X, W, Y, C=None, alpha=1.0, beta=1.0, split_k=0, ws=None, stream=None):
    """Y = beta*C + alpha*(X W) with the canonical product; Y fp32 or bf16
    (bf16/int16/uint16 dtype = bf16 output).  C: None, a length-N fp32 bias
    (broadcast to every row) or an fp32 [M, N] matrix.  W may be the
    transpose view of a row-major [N, K] weight (det_splitk_addmm_wt)."""
    px, ldx = _mat(X, _BF16_TYPES, "X")
    pw, ldw, wt = _weight(W)
    out_bf16 = Y.dtype in _BF16_TYPES
    py, ldy = _mat(Y, _BF16_TYPES + (torch.float32,), "Y")
    M, N, K = _gemm_dims(X, W, Y)
    if C is None:
        pc, ldc = ctypes.c_void_p(None), 0
    elif C.dim() == 1:
        if C.dtype != torch.float32 or not C.is_cuda or not C.is_contiguous() or C.numel() != N:
            raise ValueError("a bias C must be a contiguous fp32 GPU vector of length N")
        pc, ldc = ctypes.c_void_p(C.data_ptr()), 0
    else:
        pc, ldc = _mat(C, (torch.float32,), "C")
        if tuple(C.shape) != (M, N):
            raise ValueError("C must be [M, N]")
    pws, nws = _ws(ws)
    return ("det_splitk_addmm_wt" if wt else "det_splitk_addmm"), (
        px, ldx, pw, ldw, pc, ldc, float(alpha), float(beta), py, ldy, BF16 if out_bf16 else F32,
        M, N, K, split_k, pws, nws, _stream(stream))


def det_lora_workspace_bytes(M, N, K, r):
    return int(lib().det_lora_workspace_bytes(M, N, K, r))


def lora_workspace(M, N, K, r, device="cuda", stream=None):
    """Allocate (through torch) and zero the det_lora_forward workspace."""
    nbytes = det_lora_workspace_bytes(M, N, K, r)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("torch returned a workspace that is not 256-byte aligned")
    detred_workspace_init(ws, stream)
    return ws


@_entry
def det_lora_forward(X, W, A, B, Y, scale, ws, stream=None):
    """Y (bf16) = bf16(X W + scale * (bf16(X A) B)), every step in a fixed order."""
    px, ldx = _mat(X, _BF16_TYPES, "X")
    pw, ldw = _mat(W, _BF16_TYPES, "W")
    pa, lda = _mat(A, _BF16_TYPES, "A")
    pb, ldb = _mat(B, _BF16_TYPES, "B")
    py, ldy = _mat(Y, _BF16_TYPES, "Y")
    M, K = X.shape
    N, r = W.shape[1], A.shape[1]
    if W.shape[0] != K or A.shape[0] != K or tuple(B.shape) != (r, N) or tuple(Y.shape) != (M, N):
        raise ValueError("shape mismatch: X %s W %s A %s B %s Y %s" % (
            tuple(X.shape), tuple(W.shape), tuple(A.shape), tuple(B.shape), tuple(Y.shape)))
    pws, nws = _ws(ws)
    return "det_lora_forward", (px, ldx, pw, ldw, pa, lda, pb, ldb, float(scale), py, ldy, M, N,
                                  K, r, pws, nws, _stream(stream))


@_entry
def atomic_splitk_gemm(X, W, Y, split_k=0, stream=None):
    """The nondeterministic control: zero Y, then fp32 atomic slice adds."""
    px, ldx = _mat(X, _BF16_TYPES, "X")
    pw, ldw = _mat(W, _BF16_TYPES, "W")
    py, ldy = _mat(Y, (torch.float32,), "Y")
    M, N, K = _gemm_dims(X, W, Y)
    return "atomic_splitk_gemm", (px, ldx, pw, ldw, py, ldy, M, N, K, split_k,
                                    _stream(stream))


@_entry
def tree_tp_gemm(X, W, Y, tp_shards, ws=None, stream=None):
    """Tree-based TP-invariant product over tp_shards virtual shards.  W
    may be the transpose view of a row-major [N, K] weight (tree_tp_gemm_wt;
    same bits)."""
    px, ldx = _mat(X, _BF16_TYPES, "X")
    pw, ldw, wt = _weight(W)
    py, ldy = _mat(Y, (torch.float32,), "Y")
    M, N, K = _gemm_dims(X, W, Y)
    pws, nws = _ws(ws)
    return ("tree_tp_gemm_wt" if wt else "tree_tp_gemm"), (
        px, ldx, pw, ldw, py, ldy, M, N, K, tp_shards, pws, nws, _stream(stream))


@_entry
def tree_tp_shards_gemm(X, W, P, tp_shards, stream=None):
    """Phase 1 of tree_tp_gemm: P[t] (fp32 [T, M, N], contiguous) = shard
    t's subtree root, all shards in one launch.  W may be a transposed
    [N, K] weight's view (tree_tp_shards_gemm_wt)."""
    px, ldx = _mat(X, _BF16_TYPES, "X")
    pw, ldw, wt = _weight(W)
    M, K = X.shape
    K2, N = W.shape
    if K2 != K or tuple(P.shape) != (tp_shards, M, N) or P.dtype != torch.float32 \
            or not P.is_cuda or not P.is_contiguous():
        raise ValueError("P must be a contiguous fp32 GPU tensor of shape (T, M, N)")
    return ("tree_tp_shards_gemm_wt" if wt else "tree_tp_shards_gemm"), (
        px, ldx, pw, ldw, ctypes.c_void_p(P.data_ptr()), M, N, K, tp_shards, _stream(stream))


@_entry
def tree_tp_shard_gemm(Xt, Wt, Pt, tp_shards, stream=None):
    """One rank's shard of tree_tp_gemm: Pt = subtree root of Xt Wt (Wt
    [Kt, N], or the transpose view of the rank's [N, Kt] weight shard)."""
    px, ldx = _mat(Xt, _BF16_TYPES, "Xt")
    pw, ldw, wt = _weight(Wt)
    pp, ldp = _mat(Pt, (torch.float32,), "Pt")
    M, N, Kt = _gemm_dims(Xt, Wt, Pt)
    return ("tree_tp_shard_gemm_wt" if wt else "tree_tp_shard_gemm"), (
        px, ldx, pw, ldw, pp, ldp, M, N, Kt, tp_shards, _stream(stream))


@_entry
def tree_combine_f32(parts, Y, stream=None):
    """Y = fixed binary tree over parts[0..count) (parts: [count, ...] fp32,
    contiguous; Y: contiguous fp32 with parts[0]'s element count)."""
    if parts.dtype != torch.float32 or Y.dtype != torch.float32 or not parts.is_cuda or not Y.is_cuda:
        raise TypeError("parts and Y must be fp32 GPU tensors")
    if not parts.is_contiguous() or not Y.is_contiguous():
        raise ValueError("parts and Y must be contiguous")
    count = parts.shape[0]
    n = parts[0].numel()
    if Y.numel() != n:
        raise ValueError("Y must have %d elements" % n)
    return "tree_combine_f32", (ctypes.c_void_p(parts.data_ptr()), n, count,
                                  ctypes.c_void_p(Y.data_ptr()), n, _stream(stream))


@_entry
def detred_f32_to_bf16(x, y, stream=None):
    """y (bf16 bits) = nearest-even bf16 of x (fp32); both contiguous."""
    if x.dtype != torch.float32 or y.dtype not in _BF16_TYPES or not x.is_cuda or not y.is_cuda:
        raise TypeError("x must be fp32 and y bf16/int16 GPU tensors")
    if not x.is_contiguous() or not y.is_contiguous() or x.numel() != y.numel():
        raise ValueError("x and y must be contiguous with equal element counts")
    return "detred_f32_to_bf16", (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                    x.numel(), _stream(stream))


def _rows(t, dtypes, name):
    if t.dtype not in dtypes or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
        raise TypeError("%s must be a contiguous 2-D GPU tensor of %s" % (name, dtypes))
    return ctypes.c_void_p(t.data_ptr()), t.shape[0], t.shape[1]


@_entry
def inv_rmsnorm(x, gamma, y, eps, stream=None):
    """y[rows,hidden] fp32 = RMSNorm(x bf16) * gamma (bf16)."""
    px, rows, hidden = _rows(x, _BF16_TYPES, "x")
    py, r2, h2 = _rows(y, (torch.float32,), "y")
    if gamma.dtype not in _BF16_TYPES or not gamma.is_cuda or not gamma.is_contiguous() or gamma.numel() != hidden:
        raise TypeError("gamma must be a contiguous bf16 GPU vector of length hidden")
    if (r2, h2) != (rows, hidden):
        raise ValueError("y must match x's shape")
    return "inv_rmsnorm", (px, ctypes.c_void_p(gamma.data_ptr()), py, rows, hidden,
                             float(eps), _stream(stream))


@_entry
def inv_rmsnorm_bf16(x, gamma, y, eps, stream=None):
    """inv_rmsnorm with a bf16 output y[rows,hidden]."""
    px, rows, hidden = _rows(x, _BF16_TYPES, "x")
    py, r2, h2 = _rows(y, _BF16_TYPES, "y")
    if gamma.dtype not in _BF16_TYPES or not gamma.is_cuda or not gamma.is_contiguous() or gamma.numel() != hidden:
        raise TypeError("gamma must be a contiguous bf16 GPU vector of length hidden")
    if (r2, h2) != (rows, hidden):
        raise ValueError("y must match x's shape")
    return "inv_rmsnorm_bf16", (px, ctypes.c_void_p(gamma.data_ptr()), py, rows, hidden,
                                  float(eps), _stream(stream))


@_entry
def inv_log_softmax(x, y, stream=None):
    """y = log_softmax(x) over the last dim (fp32)."""
    px, rows, cols = _rows(x, (torch.float32,), "x")
    py, r2, c2 = _rows(y, (torch.float32,), "y")
    if (r2, c2) != (rows, cols):
        raise ValueError("y must match x's shape")
    return "inv_log_softmax", (px, py, rows, cols, _stream(stream))


@_entry
def inv_mean(x, y, stream=None):
    """y[rows] = mean of x over the last dim (fp32)."""
    px, rows, cols = _rows(x, (torch.float32,), "x")
    if y.dtype != torch.float32 or not y.is_cuda or not y.is_contiguous() or y.numel() != rows:
        raise TypeError("y must be a contiguous fp32 GPU vector with one element per row")
    return "inv_mean", (px, ctypes.c_void_p(y.data_ptr()), rows, cols, _stream(stream))


@_entry
def inv_log_softmax_mean(x, y, mu, stream=None):
    """y = log_softmax(x) and mu = mean(x) over the last dim (fp32), one pass
    over x; the bits of inv_log_softmax and inv_mean."""
    px, rows, cols = _rows(x, (torch.float32,), "x")
    py, rows2, cols2 = _rows(y, (torch.float32,), "y")
    if (rows2, cols2) != (rows, cols):
        raise ValueError("x and y must have the same shape")
    if mu.dtype != torch.float32 or not mu.is_cuda or not mu.is_contiguous() or mu.numel() != rows:
        raise TypeError("mu must be a contiguous fp32 GPU vector with one element per row")
    return "inv_log_softmax_mean", (px, py, ctypes.c_void_p(mu.data_ptr()), rows, cols,
                                    _stream(stream))


def inv_decode_attention_workspace_bytes(B, Hq, D, max_len):
    return int(lib().inv_decode_attention_workspace_bytes(B, Hq, D, max_len))


def attention_workspace(B, Hq, D, max_len, device="cuda"):
    """Allocate (through torch) the inv_decode_attention workspace."""
    nbytes = inv_decode_attention_workspace_bytes(B, Hq, D, max_len)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if ws.data_ptr() % 256:
        raise RuntimeError("torch returned a workspace that is not 256-byte aligned")
    return ws


@_entry
def inv_decode_attention(q, k, v, lens, out, scale, ws, layout="bhtd", stream=None):
    """out[B,Hq,D] fp32 = decode attention of q[B,Hq,D] (bf16) over the
    cache k, v (bf16, [B,Hkv,L,D] for layout "bhtd" or [B,L,Hkv,D] for
    "bthd", any strides with D contiguous) for the first lens[b] (int32 GPU
    vector) positions, split into fixed chunks of 256 positions."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype not in _BF16_TYPES or not t.is_cuda:
            raise TypeError("%s must be a bf16 GPU tensor" % n)
    if lens.dtype != torch.int32 or not lens.is_cuda or not lens.is_contiguous():
        raise TypeError("lens must be a contiguous int32 GPU vector")
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous():
        raise TypeError("out must be a contiguous fp32 GPU tensor")
    if not q.is_contiguous() or q.dim() != 3 or k.shape != v.shape or k.stride() != v.stride():
        raise ValueError("q must be contiguous [B,Hq,D]; k and v must share shape and strides")
    B, Hq, D = q.shape
    if layout == "bhtd":
        _, Hkv, L, D2 = k.shape
        sb, sh, st = k.stride(0), k.stride(1), k.stride(2)
    elif layout == "bthd":
        _, L, Hkv, D2 = k.shape
        sb, sh, st = k.stride(0), k.stride(2), k.stride(1)
    else:
        raise ValueError("layout must be 'bhtd' or 'bthd'")
    if k.stride(3) != 1 or D2 != D or k.shape[0] != B or tuple(out.shape) != (B, Hq, D) or lens.numel() != B:
        raise ValueError("shape mismatch")
    pws, nws = _ws(ws)
    return "inv_decode_attention", (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                      ctypes.c_void_p(v.data_ptr()), sb, sh, st,
                                      ctypes.c_void_p(lens.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                      B, Hq, Hkv, D, L, float(scale), pws, nws, _stream(stream))
