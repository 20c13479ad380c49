"""GPU parity and invariance of decode attention with a fixed-size KV split.

Parity against the fp64 oracle per output element within
(2E + 64u) * A + 1e-6, where u = 2^-24, A = sum_t w_t |v_td| / sum_t w_t and
E = (D + 8) u S bounds the binary32 error of a score (S = max_t |scale|
sum_d |q_d k_td|): a score error e changes a weight by a factor exp(e), and
the weight sums, value sums, fold and division add a few dozen roundings
relative to A.  Invariance: a sequence's output bits do not depend on the
batch it runs in, on the other sequences, on the cache capacity or on the
cache layout; replays are identical."""
import numpy as np
import pytest
import torch

import oracle
from helpers import dev_bf16, host
from invariant_reduction_amd import detred, inputs

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def run(q, k, v, lens, scale, dev, layout="bhtd"):
    """q, k, v: uint16 numpy (k, v in [B,Hkv,L,D]); returns fp32 out."""
    B, Hq, D = q.shape
    L = k.shape[2]
    qd = dev_bf16(q, dev)
    if layout == "bhtd":
        kd, vd = dev_bf16(k, dev), dev_bf16(v, dev)
    else:
        kd = dev_bf16(np.ascontiguousarray(k.transpose(0, 2, 1, 3)), dev)
        vd = dev_bf16(np.ascontiguousarray(v.transpose(0, 2, 1, 3)), dev)
    ld = torch.tensor(np.asarray(lens, dtype=np.int32), device=dev)
    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    ws = detred.attention_workspace(B, Hq, D, L, dev)
    detred.inv_decode_attention(qd, kd, vd, ld, out, scale, ws, layout=layout)
    torch.cuda.synchronize()
    return out


def check(out, q, k, v, lens, scale):
    ref, A, S = oracle.decode_attention(q, k, v, lens, scale)
    D = q.shape[2]
    E = (D + 8) * U * S[:, :, None]
    tol = (2 * E + 64 * U) * A + 1e-6
    g = host(out).astype(np.float64)
    err = np.abs(g - ref)
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("attention: %d of %d out of tolerance; first %s gpu %r oracle %r tol %r"
                             % (bad.sum(), bad.size, i, g[i], ref[i], tol[i]))
    return float((err / tol).max())


CASES = [
    # B, Hq, Hkv, D, L, lens, layout
    (3, 8, 2, 128, 1024, [1, 255, 700], "bhtd"),
    (2, 4, 4, 64, 600, [256, 257], "bthd"),
    (4, 28, 4, 128, 4096, [1000, 33, 4096, 512], "bhtd"),
    (2, 32, 2, 64, 300, [300, 299], "bthd"),
    (3, 8, 8, 128, 513, [0, 600, 513], "bhtd"),   # empty and clamped lengths
]


@pytest.mark.parametrize("B,Hq,Hkv,D,L,lens,layout", CASES)
def test_decode_attention_parity(B, Hq, Hkv, D, L, lens, layout, dev):
    q, k, v = inputs.attention_inputs(B, Hq, Hkv, L, D, seed=B + Hq + L)
    scale = 1.0 / np.sqrt(D)
    out = run(q, k, v, lens, scale, dev, layout)
    check(out, q, k, v, lens, scale)
    for b, n in enumerate(lens):
        if n <= 0:
            assert torch.all(out[b] == 0)


def test_decode_attention_single_position_is_exact(dev):
    # one position: weight exp(0) = 1, the output is the value row exactly
    B, Hq, Hkv, D, L = 2, 8, 2, 128, 64
    q, k, v = inputs.attention_inputs(B, Hq, Hkv, L, D, seed=3)
    out = run(q, k, v, [1, 1], 0.1, dev)
    vf = inputs.bf16_bits_to_f32(v)
    for b in range(B):
        for hq in range(Hq):
            np.testing.assert_array_equal(host(out)[b, hq], vf[b, hq // 4, 0])


def test_decode_attention_uniform_weights(dev):
    # q = 0: every weight is 1 and the output is the mean of the value rows
    B, Hq, Hkv, D, L = 2, 4, 2, 64, 1500
    _, k, v = inputs.attention_inputs(B, Hq, Hkv, L, D, seed=4)
    q = np.zeros((B, Hq, D), np.uint16)
    lens = [1500, 700]
    out = run(q, k, v, lens, 0.125, dev)
    check(out, q, k, v, lens, 0.125)


def test_decode_attention_batch_capacity_and_layout_invariance(dev):
    B, Hq, Hkv, D, L = 5, 16, 4, 128, 2048
    q, k, v = inputs.attention_inputs(B, Hq, Hkv, L, D, seed=6)
    lens = [2048, 1, 777, 1536, 256]
    scale = 1.0 / np.sqrt(D)
    full = host(run(q, k, v, lens, scale, dev)).view(np.uint32)
    np.testing.assert_array_equal(host(run(q, k, v, lens, scale, dev, "bthd")).view(np.uint32), full)
    for b in range(B):
        # the sequence alone, in a cache of exactly its length
        n = lens[b]
        alone = run(q[b:b + 1], np.ascontiguousarray(k[b:b + 1, :, :n]),
                    np.ascontiguousarray(v[b:b + 1, :, :n]), [n], scale, dev)
        np.testing.assert_array_equal(host(alone).view(np.uint32)[0], full[b])
    # other sequences changed, a larger cache: row 2 unchanged
    k2, v2 = k.copy(), v.copy()
    k2[0] ^= 0x0040
    v2[4] ^= 0x0040
    kb = np.zeros((B, Hkv, L + 300, D), np.uint16)
    vb = np.zeros((B, Hkv, L + 300, D), np.uint16)
    kb[:, :, :L] = k2
    vb[:, :, :L] = v2
    other = host(run(q, kb, vb, lens, scale, dev)).view(np.uint32)
    np.testing.assert_array_equal(other[2], full[2])


def test_decode_attention_replays_identical(dev):
    B, Hq, Hkv, D, L = 8, 32, 8, 128, 4096
    q, k, v = inputs.attention_inputs(B, Hq, Hkv, L, D, seed=7)
    qd, kd, vd = dev_bf16(q, dev), dev_bf16(k, dev), dev_bf16(v, dev)
    ld = torch.tensor([4096, 3000, 17, 2049, 256, 4095, 1, 1024], dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = detred.attention_workspace(B, Hq, D, L, dev)
    fn = detred.prepare(detred.inv_decode_attention, qd, kd, vd, ld, out, 0.088, ws)
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    for _ in range(20):
        fn()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
    check(out, q, k, v, host(ld), 0.088)
