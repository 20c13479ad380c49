"""The torch drop-in mode: inside batch_invariant_mode(), torch.mm / addmm
(F.linear) / log_softmax / mean on GPU tensors return libdetred's results bit
for bit, rows do not depend on the batch, unsupported calls raise, and
leaving the mode restores torch's kernels."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from helpers import host
from invariant_reduction_amd import detred, inputs, torch_ops

pytestmark = pytest.mark.gpu


def bf16(bits, dev):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def u16(t):
    return host(t.view(torch.int16)).view(np.uint16)


def test_mm_and_linear_are_libdetred(dev):
    M, K, N = 96, 2048, 520
    X, W = inputs.dense_inputs(M, K, N, seed=1)
    a, b = bf16(X, dev), bf16(W, dev)
    bias = torch.from_numpy(inputs.bias_inputs(N, seed=1)).to(dev).to(torch.bfloat16)
    Wt = b.t().contiguous()                       # nn.Linear's [out, in] weight
    y32 = torch.empty((M, N), dtype=torch.float32, device=dev)
    detred.det_splitk_gemm(a, b, y32, 0, detred.workspace(M, N, K, 0, dev))
    yb = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    detred.det_splitk_addmm(a, b, yb, bias.float(), 1.0, 1.0, 0, detred.workspace(M, N, K, 0, dev))
    with torch_ops.batch_invariant_mode():
        mm = torch.mm(a, b)
        lin = F.linear(a, Wt, bias)
        lin_rows = [F.linear(a[:m], Wt, bias) for m in (1, 7, 64)]
        with pytest.raises(NotImplementedError):
            torch.mm(a.float(), b.float())
    torch.cuda.synchronize()
    assert mm.dtype == torch.bfloat16 and lin.dtype == torch.bfloat16
    # mm: the rounding of the canonical fp32 product (the oracle's rounding)
    np.testing.assert_array_equal(u16(mm), oracle.f32_to_bf16(host(y32)))
    np.testing.assert_array_equal(u16(lin), u16(yb))
    for m, r in zip((1, 7, 64), lin_rows):
        np.testing.assert_array_equal(u16(r), u16(lin)[:m])
    assert not torch_ops.is_enabled()


def test_log_softmax_and_mean_are_libdetred(dev):
    x = torch.from_numpy(inputs.logits_inputs(8, 4000, seed=2)).to(dev)
    ref_l = torch.empty_like(x)
    detred.inv_log_softmax(x, ref_l)
    ref_m = torch.empty((8,), dtype=torch.float32, device=dev)
    detred.inv_mean(x, ref_m)
    with torch_ops.batch_invariant_mode():
        l = torch.log_softmax(x, dim=-1)
        m = x.mean(dim=-1)
        mk = x.mean(dim=-1, keepdim=True)
        l3 = torch.log_softmax(x.view(2, 4, 4000), dim=-1)
        with pytest.raises(NotImplementedError):
            x.mean(dim=0)
    torch.cuda.synchronize()
    assert torch.equal(l.view(torch.int32), ref_l.view(torch.int32))
    assert torch.equal(l3.view(8, 4000).view(torch.int32), ref_l.view(torch.int32))
    assert torch.equal(m.view(torch.int32), ref_m.view(torch.int32))
    assert mk.shape == (8, 1) and torch.equal(mk[:, 0], m)
    # parity with the oracle (C19 tolerance shape)
    lo = oracle.log_softmax(host(x))
    xm = host(x).max(axis=1, keepdims=True)
    tol = 1e-5 * (np.abs(host(x) - xm) + np.abs(np.log(np.exp(host(x).astype(np.float64) - xm).sum(axis=1, keepdims=True)))) + 1e-6
    assert np.all(np.abs(host(l) - lo) <= tol)
