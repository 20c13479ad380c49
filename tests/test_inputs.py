"""The seeded generators: reproducible, prefix-consistent, bf16 rounding to
nearest even.  CPU only."""
import numpy as np
import torch

from invariant_reduction_amd import inputs


def test_same_seed_same_bits_and_prefix():
    a = inputs.normal_bf16((64, 300), 0.0, 1.0, 0, inputs.STREAM_X)
    b = inputs.normal_bf16((64, 300), 0.0, 1.0, 0, inputs.STREAM_X)
    np.testing.assert_array_equal(a, b)
    short = inputs.normal_bf16((5, 300), 0.0, 1.0, 0, inputs.STREAM_X)
    np.testing.assert_array_equal(short, a[:5])
    other = inputs.normal_bf16((5, 300), 0.0, 1.0, 0, inputs.STREAM_W)
    assert not np.array_equal(other, short)


def test_bf16_rounding_matches_torch():
    f = inputs.normal_f32((10000,), 0.0, 3.0, 1, 2)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(inputs.f32_bits_to_bf16_bits(f), want)
    np.testing.assert_array_equal(
        inputs.bf16_bits_to_f32(want),
        torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_distributions():
    w = inputs.bf16_bits_to_f32(inputs.normal_bf16((512, 512), 0.0, 0.02, 0, 1))
    assert abs(w.std() - 0.02) < 0.001 and abs(w.mean()) < 0.001
    g = inputs.bf16_bits_to_f32(inputs.rmsnorm_inputs(1, 4096)[1])
    assert abs(g.mean() - 1.0) < 0.01 and abs(g.std() - 0.1) < 0.01
    lg = inputs.logits_inputs(2, 151936)
    assert lg.dtype == np.float32 and abs(lg.std() - 3.0) < 0.05
    xi = inputs.bf16_bits_to_f32(inputs.integer_bf16((100, 100), -8, 8, 0, 0))
    assert xi.min() == -8 and xi.max() == 8 and np.all(xi == np.round(xi))
