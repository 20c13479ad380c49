"""Batch-invariant drop-in replacements for torch operators, over libdetred.

The "Batch Invariant Ops" project (Highlighted Details) makes mm, addmm,
log_softmax and mean batch invariant by swapping the implementations torch
dispatches to.  ``batch_invariant_mode()`` does the same here: while it is
active, these aten operators on GPU tensors run libdetred's kernels:

  aten::mm(a, b)                   a, b bf16 -> bf16: det_splitk_addmm, no C
  aten::addmm(c, a, b, beta, alpha) bf16 -> bf16: det_splitk_addmm with C
                                   (a bias row or an [M, N] matrix, as fp32)
  aten::_log_softmax(x, -1, False) fp32 -> fp32: inv_log_softmax
  aten::mean.dim(x, [-1], keepdim) fp32 -> fp32: inv_mean

The products round the binary32 result to bf16 once, as torch's bf16 mm
does.  A call outside what the kernels cover (another dtype, another
dimension, shapes or alignments the C ABI rejects) raises
NotImplementedError instead of falling back to a kernel whose result could
depend on the batch.  A second operand that is the transpose view of a
row-major weight (F.linear passes W.t()) goes to the transposed-weight
kernels as it is; any other second operand that is not row-major is copied
to row-major first.  Operators on CPU tensors are
not affected.  Argument marshalling only: every result comes from
libdetred's HIP kernels.
"""
import contextlib
import warnings

import torch

from . import detred

_BF16 = (torch.bfloat16,)


def _row_major(t):
    if t.dim() == 2 and (t.shape[1] <= 1 or t.stride(1) == 1) and t.data_ptr() % 16 == 0 and \
            (t.shape[0] <= 1 or t.stride(0) % 8 == 0):
        return t
    return t.contiguous()


def _right_operand(b):
    """b as the library takes it: a [K, N] view of a row-major [N, K] weight
    (linear layers call addmm with weight.t()) goes as it is, to the
    transposed-weight kernels; anything else as a row-major matrix."""
    if b.dim() == 2 and b.shape[0] > 1 and b.shape[1] > 1 and b.stride(0) == 1 and \
            b.stride(1) % 8 == 0 and b.data_ptr() % 16 == 0:
        return b
    return _row_major(b)


def _check_mm(a, b):
    if a.dtype not in _BF16 or b.dtype not in _BF16:
        raise NotImplementedError("batch-invariant mm covers bf16 operands, got %s x %s" % (a.dtype, b.dtype))
    if a.dim() != 2 or b.dim() != 2 or a.shape[1] != b.shape[0]:
        raise NotImplementedError("batch-invariant mm covers 2-D operands with matching inner size")
    M, K = a.shape
    N = b.shape[1]
    if K % 8 or N % 8:
        raise NotImplementedError("batch-invariant mm needs K and N multiples of 8 (K=%d, N=%d)" % (K, N))
    return _row_major(a), _right_operand(b), M, N, K


def _product(a, b, c, alpha, beta):
    a, b, M, N, K = _check_mm(a, b)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if M == 0 or N == 0:
        return out
    ws = detred.workspace(M, N, K, 0, a.device)
    detred.det_splitk_addmm(a, b, out, c, alpha, beta, 0, ws)
    return out


def _mm(a, b):
    return _product(a, b, None, 1.0, 1.0)


def _addmm(c, a, b, *, beta=1, alpha=1):
    M, N = a.shape[0], b.shape[1]
    if beta == 0:  # torch ignores the input then, NaN included
        return _product(a, b, None, float(alpha), 1.0)
    if c.dim() == 1 and c.shape[0] == N:
        cf = c.float().contiguous()
    elif c.dim() == 2 and tuple(c.shape) == (1, N):
        cf = c[0].float().contiguous()
    elif c.dim() == 2 and tuple(c.shape) == (M, N):
        cf = c.float().contiguous()
    else:
        raise NotImplementedError("batch-invariant addmm covers a length-N bias or an [M, N] input")
    return _product(a, b, cf, float(alpha), float(beta))


def _log_softmax(x, dim, half_to_float):
    if x.dtype != torch.float32 or half_to_float:
        raise NotImplementedError("batch-invariant log_softmax covers fp32 input and output")
    if dim not in (-1, x.dim() - 1) or x.dim() < 1:
        raise NotImplementedError("batch-invariant log_softmax covers the last dimension")
    cols = x.shape[-1]
    x2 = x.contiguous().view(-1, cols)
    out = torch.empty_like(x2)
    if x2.shape[0]:
        detred.inv_log_softmax(x2, out)
    return out.view(x.shape)


def _mean_dim(x, dim, keepdim=False, *, dtype=None):
    if x.dtype != torch.float32 or (dtype is not None and dtype != torch.float32):
        raise NotImplementedError("batch-invariant mean covers fp32 input and output")
    dims = list(dim) if dim is not None else []
    if len(dims) != 1 or dims[0] not in (-1, x.dim() - 1):
        raise NotImplementedError("batch-invariant mean covers the last dimension only")
    cols = x.shape[-1]
    x2 = x.contiguous().view(-1, cols)
    out = torch.empty((x2.shape[0],), dtype=torch.float32, device=x.device)
    if x2.shape[0]:
        detred.inv_mean(x2, out)
    shape = list(x.shape[:-1]) + ([1] if keepdim else [])
    return out.view(shape)


_lib = None


def enable():
    """Register the replacements for the CUDA (HIP) dispatch key."""
    global _lib
    if _lib is not None:
        return
    detred.lib()  # fail now, loudly, if the library cannot be loaded
    lib = torch.library.Library("aten", "IMPL")
    with warnings.catch_warnings():
        # torch warns that a kernel for the key is being overridden: that is the point
        warnings.simplefilter("ignore", UserWarning)
        lib.impl("mm", _mm, "CUDA")
        lib.impl("addmm", _addmm, "CUDA")
        lib.impl("_log_softmax", _log_softmax, "CUDA")
        lib.impl("mean.dim", _mean_dim, "CUDA")
    _lib = lib


def disable():
    """Remove the replacements (torch's own kernels again)."""
    global _lib
    if _lib is not None:
        _lib._destroy()
        _lib = None


def is_enabled():
    return _lib is not None


@contextlib.contextmanager
def batch_invariant_mode():
    """Context manager: the replacements are active inside the block."""
    was = is_enabled()
    enable()
    try:
        yield
    finally:
        if not was:
            disable()
