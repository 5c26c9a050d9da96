"""Pins of the oracle's mHC transform (sigmoid read/write weights,
Sinkhorn-normalised exp(logits) stream mix).

The glossary page "Hyper-connections (mHC)" (definition) fixes only that the
mixing is made doubly stochastic with a few Sinkhorn iterations.  Pins:
rank-1 logits give the uniform matrix after one iteration; the cross-ratios
A_ij A_kl / (A_il A_kj) are invariant under any number of iterations (row and
column scalings cancel); the n = 2 limit has a closed form; column sums are 1
after every iteration and rows converge; sigmoid special values; 60-digit
decimal brute force."""
import numpy as np
import pytest

import exact


def A_of(w, n):
    return w[:, 2 * n:].reshape(-1, n, n)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_rank_one_logits_uniform(orc, rng, n):
    K = 2 * n + n * n
    r, c = rng.standard_normal((5, n)), rng.standard_normal((5, n))
    lg = rng.standard_normal((5, K))
    lg[:, 2 * n:] = (r[:, :, None] + c[:, None, :]).reshape(5, -1)
    for iters in (1, 2, 20):
        A = A_of(orc.sinkhorn(lg, n, iters), n)
        np.testing.assert_allclose(A, 1.0 / n, rtol=1e-14)


def test_cross_ratio_invariance(orc, rng):
    n = 4
    lg = rng.standard_normal((20, 24))
    L = lg[:, 8:].reshape(20, n, n)
    for iters in (1, 5, 20):
        A = A_of(orc.sinkhorn(lg, n, iters), n)
        for (i, j, k, l) in [(0, 1, 2, 3), (1, 0, 3, 2), (0, 0, 3, 3), (2, 1, 0, 3)]:
            got = np.log(A[:, i, j] * A[:, k, l] / (A[:, i, l] * A[:, k, j]))
            want = L[:, i, j] + L[:, k, l] - L[:, i, l] - L[:, k, j]
            np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_two_by_two_limit_closed_form(orc, rng):
    """For n = 2 the doubly stochastic limit is [[p, 1-p], [1-p, p]] with
    p = sqrt(e00 e11) / (sqrt(e00 e11) + sqrt(e01 e10))."""
    lg = rng.standard_normal((50, 8))
    A = A_of(orc.sinkhorn(lg, 2, 400), 2)
    e = np.exp(lg[:, 4:])
    s1, s2 = np.sqrt(e[:, 0] * e[:, 3]), np.sqrt(e[:, 1] * e[:, 2])
    p = s1 / (s1 + s2)
    np.testing.assert_allclose(A[:, 0, 0], p, rtol=1e-12)
    np.testing.assert_allclose(A[:, 1, 1], p, rtol=1e-12)
    np.testing.assert_allclose(A[:, 0, 1], 1 - p, rtol=1e-11)


def test_doubly_stochastic(orc, rng):
    n, T = 4, 4096
    lg = rng.standard_normal((T, 24))
    # every iteration ends with the column normalisation
    for iters in (1, 3, 20):
        A = A_of(orc.sinkhorn(lg, n, iters), n)
        np.testing.assert_allclose(A.sum(axis=1), 1.0, atol=1e-13)
    # run long enough, rows converge too: doubly stochastic within 1e-12
    A = A_of(orc.sinkhorn(lg, n, 400), n)
    np.testing.assert_allclose(A.sum(axis=1), 1.0, atol=1e-12)
    np.testing.assert_allclose(A.sum(axis=2), 1.0, atol=1e-12)
    # at the fixed count of 20, almost every N(0,1) token has rows within 1e-6
    A20 = A_of(orc.sinkhorn(lg, n, 20), n)
    row_err = np.abs(A20.sum(axis=2) - 1).max(axis=1)
    assert np.mean(row_err <= 1e-6) > 0.97


def test_sigmoid_and_zero_iterations(orc, rng):
    n = 3
    lg = rng.standard_normal((4, 15))
    lg[0, :2 * n] = 0.0
    w = orc.sinkhorn(lg, n, 0)
    assert np.all(w[0, :2 * n] == 0.5)
    np.testing.assert_allclose(w[1:, :2 * n] + orc.sinkhorn(-lg, n, 0)[1:, :2 * n], 1.0, rtol=1e-15)
    np.testing.assert_allclose(w[:, 2 * n:], np.exp(lg[:, 2 * n:]), rtol=1e-15)


def test_dominant_diagonal_gives_identity(orc):
    lg = np.zeros((1, 24))
    lg[0, 8:] = (30.0 * np.eye(4)).reshape(-1)
    A = A_of(orc.sinkhorn(lg, 4, 20), 4)[0]
    np.testing.assert_allclose(A, np.eye(4), atol=1e-12)


@pytest.mark.parametrize("n,iters", [(2, 3), (3, 4), (4, 2)])
def test_brute_force_decimal(orc, rng, n, iters):
    lg = rng.standard_normal((3, 2 * n + n * n))
    w = orc.sinkhorn(lg, n, iters)
    for t in range(3):
        ref = exact.sinkhorn_exact(lg[t], n, iters)
        np.testing.assert_allclose(w[t], [float(v) for v in ref], rtol=1e-14, atol=1e-16)
