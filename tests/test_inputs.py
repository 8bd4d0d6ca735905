"""The seeded generators: determinism, the stated value structure, and the
fp32 -> BF16 rounding checked against torch's own conversion."""
import numpy as np
import torch

from lossless_bit_weight_amd import inputs


def test_rne_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(0.02),
        rng.standard_normal(1000).astype(np.float32) * np.float32(1e30),
        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40, 3.3895314e38,
                  1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], dtype=np.float32),
    ])
    ours = inputs.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    nan = inputs.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


def test_deterministic_and_seeded():
    a = inputs.TINY.weights_raw()
    b = inputs.TINY.weights_raw()
    assert np.array_equal(a, b)
    c = inputs.GemmCase("x", 1024, 512, 1, 0.02, 1.0, 999, 102, 103).weights_raw()
    assert not np.array_equal(a, c)
    assert np.array_equal(inputs.TINY.activations(4), inputs.TINY.activations(4))
    assert inputs.TINY.activations(4).shape == (4, 512)


def test_value_structure():
    case = inputs.GemmCase("qkv rows", 1024, 5120, 1, 0.02, 1.0, 201, 202, 203)
    w = case.weights_raw()
    assert w.shape == (1024, 5120) and w.dtype == np.uint16
    zeros = (w & 0x7FFF) == 0
    frac = zeros.mean()
    assert 0.0008 < frac < 0.0012
    assert ((w == 0x8000) & zeros).any() and ((w == 0) & zeros).any()
    f = inputs.bf16_bits_to_f32(w[:64])
    assert abs(float(f.std()) - 0.02) < 0.0005
