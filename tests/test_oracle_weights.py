"""Pins of the oracle's per-token weight step (RMSNorm per stream, mean over
streams, projection, tanh / mHC transform).

The pages give no formula for per-token weights; the reading is pinned here
by: W = 0 reproduces the static record bitwise; on n copies of x the result is
the library rms_norm(x) projected (torch, float64); scaled copies c_i x give a
closed form that separates "mean of per-stream norms" from "norm of the mean"
and from "sum over streams"; 60-digit decimal brute force on tiny shapes."""
import numpy as np
import pytest
import torch

import exact
from hyper_connections_amd.workloads import f32_to_bf16_bits, identity_record


def test_zero_projection_is_static(orc, rng):
    n, d = 4, 64
    H = rng.standard_normal((9, n, d)).astype(np.float32)
    ws = rng.standard_normal(24)
    w = orc.weights(H, np.zeros((24, d), np.float32), ws, 0.01, 1e-6, 0)
    assert np.array_equal(w, np.broadcast_to(ws, w.shape))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_copies_reduce_to_rmsnorm_projection(orc, rng, n):
    K, d, T = 2 * n + n * n, 48, 5
    x = rng.standard_normal((T, d)).astype(np.float32)
    H = np.repeat(x[:, None, :], n, axis=1)
    W = (0.3 * rng.standard_normal((K, d))).astype(np.float32)
    ws = identity_record(n).astype(np.float64)
    w = orc.weights(H, W, ws, 0.5, 1e-6, 0)
    xn = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (d,), eps=1e-6)
    z = (xn @ torch.from_numpy(W.astype(np.float64)).T).numpy()
    np.testing.assert_allclose(w, ws + 0.5 * np.tanh(z), rtol=1e-13, atol=1e-14)


def test_scaled_copies_closed_form(orc, rng):
    """H_i = c_i x: r_i c_i = c_i / sqrt(c_i^2 ms + eps), so
    hbar = x * mean_i(c_i / sqrt(c_i^2 ms + eps))."""
    n, d, eps = 4, 32, 1e-3
    c = np.array([1.0, -2.0, 0.5, 4.0])
    x = rng.standard_normal(d).astype(np.float32)
    H = (c[:, None] * x[None, :]).astype(np.float32)[None]
    assert np.array_equal(H[0].astype(np.float64), c[:, None] * x.astype(np.float64))
    W = rng.standard_normal((24, d)).astype(np.float32)
    ms = np.mean(x.astype(np.float64) ** 2)
    coef = np.mean(c / np.sqrt(c * c * ms + eps))
    z = coef * (W.astype(np.float64) @ x.astype(np.float64))
    w = orc.weights(H, W, np.zeros(24), 1.0, eps, 0)
    np.testing.assert_allclose(w[0], np.tanh(z), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("n,d,iters", [(1, 8, 0), (2, 8, 0), (3, 16, 0), (4, 8, 0), (4, 8, 3), (2, 8, 2)])
def test_brute_force_decimal(orc, rng, n, d, iters):
    K, T = 2 * n + n * n, 2
    H = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    W = f32_to_bf16_bits(rng.standard_normal((K, d)).astype(np.float32))
    ws = rng.standard_normal(K).astype(np.float32).astype(np.float64)
    w = orc.weights(H, W, ws, 0.25, 1e-6, iters)
    Hf, Wf = orc.widen(H), orc.widen(W)
    for t in range(T):
        ref = exact.dyn_weights_exact(Hf[t], Wf, ws, 0.25, 1e-6, iters)
        np.testing.assert_allclose(w[t], [float(v) for v in ref], rtol=1e-13, atol=1e-15)


def test_mhc_mode_is_sinkhorn_of_logits(orc, rng):
    n, d, T = 4, 32, 6
    x = rng.standard_normal((T, d)).astype(np.float32)
    H = np.repeat(x[:, None, :], n, axis=1)
    W = rng.standard_normal((24, d)).astype(np.float32)
    ws = rng.standard_normal(24)
    w = orc.weights(H, W, ws, 0.1, 1e-6, 7)
    xn = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (d,), eps=1e-6)
    logits = ws + 0.1 * (xn @ torch.from_numpy(W.astype(np.float64)).T).numpy()
    np.testing.assert_allclose(w, orc.sinkhorn(logits, n, 7), rtol=1e-12, atol=1e-14)
