"""Pins of the oracle's storage model: exact widening and nearest-even bf16
rounding (the store a bf16 kernel performs).  Checked against a library
routine (torch's float32 -> bfloat16 conversion, which rounds to nearest even),
the input generator's independent bit-trick rounding, and hand-derived
boundary cases."""
import math

import numpy as np
import torch

from hyper_connections_amd.workloads import (bf16_bits_to_f32, f32_to_bf16_bits, f32_to_fp8_bits,
                                             fp8_bits_to_f32)


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


def test_round_fp8_matches_torch_within_range(orc, rng):
    """Nearest-even E4M3 rounding equals torch's float8_e4m3fn cast wherever
    the cast does not overflow (|x| <= 464); beyond it the oracle saturates
    at +-448 where the cast gives NaN."""
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1.0, 1e-2, 30.0)] +
                       [np.linspace(-464, 464, 4001), [0.0, -0.0]]).astype(np.float32)
    ours = orc.round_fp8(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # widening: every finite code decodes to torch's value
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = orc.widen(codes)
    fin = ~np.isnan(vals)
    assert np.array_equal(got[fin], vals[fin]) and np.all(np.isnan(got[~fin]))


def test_round_fp8_boundaries(orc):
    r = lambda v: int(orc.round_fp8(np.array([v]))[0])  # noqa: E731
    assert r(1.0) == 0x38 and r(-1.0) == 0xB8
    assert r(1.0625) == 0x38                  # tie -> even (down)
    assert r(1.1875) == 0x3A                  # tie -> even (up)
    assert r(448.0) == 0x7E and r(464.0) == 0x7E
    assert r(470.0) == 0x7E and r(1e30) == 0x7E and r(math.inf) == 0x7E   # saturating
    assert r(-math.inf) == 0xFE
    assert r(2.0 ** -6) == 0x08               # smallest normal
    assert r(2.0 ** -9) == 0x01 and r(2.0 ** -10) == 0x00 and r(1.5 * 2.0 ** -10) == 0x01
    assert r(7 * 2.0 ** -9) == 0x07 and r(7.5 * 2.0 ** -9) == 0x08    # carry into the normals
    assert (r(math.nan) & 0x7F) == 0x7F


def test_round_fp8_matches_generator(orc, rng):
    """The oracle's FP8 rounding equals the input generator's independent
    table-search rounding, including saturation and ties."""
    x = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(5000) * 1e-3,
                        np.arange(-1000, 1000) * 0.5, [1e30, -1e30]]).astype(np.float32)
    ours = orc.round_fp8(x.astype(np.float64))
    assert np.array_equal(ours, f32_to_fp8_bits(x))
    assert np.array_equal(orc.widen(ours), fp8_bits_to_f32(ours).astype(np.float64))


def test_fp8_storage_reads_like_its_values(orc, rng):
    """Every oracle routine fed FP8 codes gives what it gives for the same
    values held exactly in fp32 (each FP8 value is an fp32 value)."""
    T, n, d = 6, 4, 40
    H8 = f32_to_fp8_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    F8 = f32_to_fp8_bits(rng.standard_normal((T, d)).astype(np.float32))
    H, F = fp8_bits_to_f32(H8), fp8_bits_to_f32(F8)
    w = rng.standard_normal((T, 2 * n + n * n)).astype(np.float32)
    g = rng.standard_normal(d).astype(np.float32)
    assert np.array_equal(orc.pre_mix(H8, w, g), orc.pre_mix(H, w, g))
    assert np.array_equal(orc.post_mix(H8, F8, w), orc.post_mix(H, F, w))
    assert np.array_equal(orc.block_tanh(F8), orc.block_tanh(F))


def test_f64_storage_reads_like_its_values(orc, rng):
    """Unrounded float64 inputs (the pure fp64 chain) are read as they are:
    values that fp32 holds exactly give bitwise what the fp32 array gives,
    and values fp32 cannot hold reach the arithmetic unrounded."""
    T, n, d, K = 5, 4, 24, 24
    H = rng.standard_normal((T, n, d)).astype(np.float32)
    F = rng.standard_normal((T, d)).astype(np.float32)
    W = (0.1 * rng.standard_normal((K, d))).astype(np.float32)
    w = rng.standard_normal((T, K)).astype(np.float32)
    g = rng.standard_normal(d).astype(np.float32)
    H64, F64, W64 = H.astype(np.float64), F.astype(np.float64), W.astype(np.float64)
    assert np.array_equal(orc.pre_mix(H64, w, g), orc.pre_mix(H, w, g))
    assert np.array_equal(orc.post_mix(H64, F64, w), orc.post_mix(H, F, w))
    assert np.array_equal(orc.weights(H64, W64, w[0], 0.5), orc.weights(H, W, w[0], 0.5))
    assert np.array_equal(orc.widen(H64), H64)
    # 1 + 2^-40 is not an fp32 value: with A = I, beta = 1 post adds it to F unrounded
    one = np.zeros(K)
    one[n:2 * n] = 1.0
    one[2 * n:] = np.eye(n).ravel()
    Hx = np.full((1, n, d), 1.0 + 2.0 ** -40)
    out = orc.post_mix(Hx, np.zeros((1, d)), one)
    assert np.all(out == 1.0 + 2.0 ** -40)
