"""Exact / high-precision brute force for tiny cases (test infrastructure).

Independent of the oracle: nothing here imports it, and the formulations are
different where possible (the stream-mix is written as one Kronecker-product
matrix acting on the stacked streams; reductions are done in exact rationals;
square roots, exponentials and tanh in 60-digit decimal arithmetic).
Inputs are python floats / numpy float64 values, which Fraction holds exactly.
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

getcontext().prec = 60


def fr(x) -> Fraction:
    return Fraction(float(x))


def dec(q: Fraction) -> Decimal:
    return Decimal(q.numerator) / Decimal(q.denominator)


def dsqrt(q: Fraction) -> Decimal:
    return dec(q).sqrt()


def dexp(x: Decimal) -> Decimal:
    return x.exp()


def dtanh(x: Decimal) -> Decimal:
    e = (2 * x).exp()
    return (e - 1) / (e + 1)


def dsigmoid(x: Decimal) -> Decimal:
    return 1 / (1 + (-x).exp())


def kron_stream_mix(H: np.ndarray, F: np.ndarray, A: np.ndarray, beta: np.ndarray) -> list:
    """One token: stack the streams as vec(H) (length n*d) and form
    M = A (x) I_d explicitly, then vec(H') = M vec(H) + beta (x) F, exactly."""
    n, d = H.shape
    vecH = [fr(H[j, k]) for j in range(n) for k in range(d)]
    out = []
    for row in range(n * d):
        i, k = divmod(row, d)
        acc = Fraction(0)
        for col in range(n * d):
            j, kk = divmod(col, d)
            m = fr(A[i, j]) if kk == k else Fraction(0)   # (A (x) I_d)[row, col]
            acc += m * vecH[col]
        acc += fr(beta[i]) * fr(F[k])                       # (beta (x) F)[row]
        out.append(acc)
    return [[out[i * d + k] for k in range(d)] for i in range(n)]


def rmsnorm_exact(x: list, gamma, eps) -> list:
    """gamma_k x_k / sqrt(mean x^2 + eps) with the mean square exact."""
    d = len(x)
    ms = sum((xi * xi for xi in x), Fraction(0)) / d
    root = dsqrt(ms + fr(eps))
    return [dec(fr(gamma[k]) * x[k]) / root for k in range(d)]


def read_mix_exact(H: np.ndarray, alpha) -> list:
    n, d = H.shape
    return [sum((fr(alpha[i]) * fr(H[i, k]) for i in range(n)), Fraction(0)) for k in range(d)]


def dyn_weights_exact(H: np.ndarray, W: np.ndarray, w_static, scale, eps, iters=0) -> list:
    """Per-token weights for one token, in 60-digit decimal arithmetic."""
    n, d = H.shape
    r = []
    for i in range(n):
        ms = sum((fr(H[i, k]) ** 2 for k in range(d)), Fraction(0)) / d
        r.append(1 / dsqrt(ms + fr(eps)))
    hbar = [sum(r[i] * dec(fr(H[i, k])) for i in range(n)) / n for k in range(d)]
    z = [sum(hbar[k] * dec(fr(W[c, k])) for k in range(d)) for c in range(W.shape[0])]
    if iters == 0:
        return [dec(fr(w_static[c])) + dec(fr(scale)) * dtanh(z[c]) for c in range(len(z))]
    lg = [dec(fr(w_static[c])) + dec(fr(scale)) * z[c] for c in range(len(z))]
    return sinkhorn_exact(lg, n, iters)


def sinkhorn_exact(logits, n: int, iters: int) -> list:
    """Record [sigmoid(l_a) | sigmoid(l_b) | SK_iters(exp(l_A))] in decimal."""
    lg = [x if isinstance(x, Decimal) else dec(fr(x)) for x in logits]
    a = [dsigmoid(lg[i]) for i in range(n)]
    b = [dsigmoid(lg[n + i]) for i in range(n)]
    M = [[dexp(lg[2 * n + i * n + j]) for j in range(n)] for i in range(n)]
    for _ in range(iters):
        M = [[M[i][j] / sum(M[i]) for j in range(n)] for i in range(n)]
        cols = [sum(M[i][j] for i in range(n)) for j in range(n)]
        M = [[M[i][j] / cols[j] for j in range(n)] for i in range(n)]
    return a + b + [M[i][j] for i in range(n) for j in range(n)]
