"""Pins of the oracle's storage model: exact widening and nearest-even bf16
rounding (the store a bf16 kernel performs).  Checked against a library
routine (torch's float32 -> bfloat16 conversion, which rounds to nearest even),
the input generator's independent bit-trick rounding, and hand-derived
boundary cases."""
import math

import numpy as np
import torch

from hyper_connections_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits


def test_widen_is_exact(orc, rng):
    x = rng.standard_normal(1000).astype(np.float32)
    assert np.array_equal(orc.widen(x), x.astype(np.float64))
    b = f32_to_bf16_bits(x)
    assert np.array_equal(orc.widen(b), bf16_bits_to_f32(b).astype(np.float64))


def test_round_bf16_matches_torch_on_f32(orc, rng):
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),    # subnormals
        (rng.standard_normal(2000) * 1e37).astype(np.float32),     # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf], np.float32),
    ])
    ours = orc.round_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(ours, f32_to_bf16_bits(x))


def test_round_bf16_boundaries(orc):
    r = lambda v: int(orc.round_bf16(np.array([v]))[0])  # noqa: E731
    assert r(1.0) == 0x3F80
    assert r(1.0 + 2.0 ** -8) == 0x3F80            # tie -> even (down)
    assert r(1.0 + 3 * 2.0 ** -8) == 0x3F82        # tie -> even (up)
    assert r(1.0 + 2.0 ** -8 + 2.0 ** -40) == 0x3F81  # just above the tie (double only)
    assert r(-0.0) == 0x8000 and r(0.0) == 0x0000
    assert r(2.0 ** -133) == 0x0001                # smallest subnormal
    assert r(2.0 ** -134) == 0x0000                # tie to even -> zero
    assert r(3 * 2.0 ** -134) == 0x0002            # tie -> even (up)
    big = (2 - 2.0 ** -7) * 2.0 ** 127              # largest finite bf16
    assert r(big) == 0x7F7F
    assert r((2 - 2.0 ** -8) * 2.0 ** 127) == 0x7F80   # tie past the top -> inf
    assert r(math.inf) == 0x7F80 and r(-math.inf) == 0xFF80
    assert (r(math.nan) & 0x7FC0) == 0x7FC0


def test_block_tanh_is_library_tanh(orc, rng):
    x = rng.standard_normal(5000).astype(np.float32)
    np.testing.assert_allclose(orc.block_tanh(x), np.tanh(x.astype(np.float64)), rtol=1e-15, atol=1e-300)
    b = f32_to_bf16_bits(x)
    np.testing.assert_allclose(orc.block_tanh(b), np.tanh(bf16_bits_to_f32(b).astype(np.float64)), rtol=1e-15)
