"""Pins of the oracle's post step (stream-mix + write-back).

Pins: the Kronecker-matrix formulation in exact rationals (brute force); a
non-symmetric permutation matrix (catches a transposed A); conservation of the
stream sum under a column-stochastic A; linearity in (H, F); the identity and
n = 1 invariants reduce to the ordinary residual x + f(x) bitwise."""
import numpy as np
import pytest

import exact
from hyper_connections_amd.workloads import f32_to_bf16_bits, identity_record


def record(alpha, beta, A):
    return np.concatenate([alpha, beta, np.asarray(A).reshape(-1)]).astype(np.float64)


@pytest.mark.parametrize("n,d", [(1, 4), (2, 3), (3, 4), (4, 2), (4, 5)])
def test_kronecker_brute_force(orc, rng, n, d):
    T = 2
    H = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    F = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w = rng.standard_normal((T, 2 * n + n * n)).astype(np.float32).astype(np.float64)
    out = orc.post_mix(H, F, w)
    Hf, Ff = orc.widen(H), orc.widen(F)
    for t in range(T):
        A = w[t, 2 * n:].reshape(n, n)
        ref = exact.kron_stream_mix(Hf[t], Ff[t], A, w[t, n:2 * n])
        for i in range(n):
            for k in range(d):
                assert abs(out[t, i, k] - float(ref[i][k])) <= 1e-15 * max(1.0, abs(float(ref[i][k])))


def test_permutation_routes_streams(orc, rng):
    """A[i][j] = 1 iff j = pi(i): output stream i is input stream pi(i)."""
    n, d = 4, 16
    pi = [2, 0, 3, 1]                       # not an involution: a transposed A differs
    A = np.zeros((n, n))
    A[np.arange(n), pi] = 1.0
    H = rng.standard_normal((3, n, d)).astype(np.float32)
    F = rng.standard_normal((3, d)).astype(np.float32)
    out = orc.post_mix(H, F, record(np.zeros(n), np.zeros(n), A))
    for i in range(n):
        assert np.array_equal(out[:, i, :], H[:, pi[i], :].astype(np.float64))


def test_column_stochastic_conserves_sum(orc, rng):
    n, d, T = 4, 32, 5
    M = rng.random((n, n)) + 0.1
    A = M / M.sum(axis=0, keepdims=True)     # columns sum to 1
    beta = rng.standard_normal(n)
    H = rng.standard_normal((T, n, d)).astype(np.float32)
    F = rng.standard_normal((T, d)).astype(np.float32)
    out = orc.post_mix(H, F, record(np.zeros(n), beta, A))
    lhs = out.sum(axis=1)
    rhs = H.astype(np.float64).sum(axis=1) + beta.sum() * F.astype(np.float64)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_linearity(orc, rng):
    n, d, T = 3, 20, 4
    w = rng.standard_normal(2 * n + n * n)
    H1 = rng.standard_normal((T, n, d)).astype(np.float32)
    H2 = rng.standard_normal((T, n, d)).astype(np.float32)
    F1 = rng.standard_normal((T, d)).astype(np.float32)
    F2 = rng.standard_normal((T, d)).astype(np.float32)
    a = orc.post_mix(H1, F1, w) + orc.post_mix(H2, F2, w)
    b = orc.post_mix((H1.astype(np.float64) + H2).astype(np.float32),
                     (F1.astype(np.float64) + F2).astype(np.float32), w)
    np.testing.assert_allclose(a, b, rtol=1e-6, atol=1e-6)   # float32 re-rounding of the sums


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_identity_is_plain_residual_bitwise(orc, rng, n):
    """Identity weights on n copies of x: every stream becomes x + F, and its
    bf16 store equals the rounded ordinary residual (explainer, "Jargon":
    identity initialization computes exactly what the old mechanism did)."""
    T, d = 8, 64
    x = f32_to_bf16_bits(rng.standard_normal((T, 1, d)).astype(np.float32))
    F = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    H = np.repeat(x, n, axis=1)
    out = orc.post_mix(H, F, identity_record(n))
    plain = orc.widen(x)[:, 0, :] + orc.widen(F)
    for i in range(n):
        assert np.array_equal(out[:, i, :], plain)
        assert np.array_equal(orc.round_bf16(out[:, i, :]), orc.round_bf16(plain))
