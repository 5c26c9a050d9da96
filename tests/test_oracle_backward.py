"""Pins of the oracle's backward (gradients of pre and post).

Pins: torch.autograd in float64 through torch's own rms_norm and tensor ops (a
library routine); central finite differences of the forward oracle (itself
pinned) in the weights and the gain, perturbed exactly in float64; the
adjoint identity <dH', post(H, F)> = <dH, H> + <dF, F> of the linear post map."""
import numpy as np
import pytest
import torch

from hyper_connections_amd.workloads import identity_record


def rand_case(rng, T, n, d, per_token):
    K = 2 * n + n * n
    H = rng.standard_normal((T, n, d)).astype(np.float32)
    F = rng.standard_normal((T, d)).astype(np.float32)
    shape = (T, K) if per_token else (K,)
    w = (np.broadcast_to(identity_record(n), shape) + 0.3 * rng.standard_normal(shape)).astype(np.float64)
    g = 1 + 0.1 * rng.standard_normal(d)
    return H, F, w, g


def torch_layer(H, F, w, g, eps, n):
    """Forward with torch ops in float64; returns (u, H') and the leaves."""
    Ht = torch.tensor(H.astype(np.float64), requires_grad=True)
    Ft = torch.tensor(F.astype(np.float64), requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    W2 = wt if wt.dim() == 2 else wt.unsqueeze(0).expand(Ht.shape[0], -1)
    alpha, beta = W2[:, :n], W2[:, n:2 * n]
    A = W2[:, 2 * n:].reshape(-1, n, n)
    x = (alpha[:, :, None] * Ht).sum(1)
    u = torch.nn.functional.rms_norm(x, (x.shape[-1],), gt, eps)
    Hp = torch.einsum("tij,tjk->tik", A, Ht) + beta[:, :, None] * Ft[:, None, :]
    return u, Hp, (Ht, Ft, wt, gt)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("per_token", [False, True])
def test_post_backward_matches_autograd(orc, rng, n, per_token):
    T, d = 5, 24
    H, F, w, g = rand_case(rng, T, n, d, per_token)
    dHo = rng.standard_normal((T, n, d)).astype(np.float32)
    dH, dF, dw = orc.post_mix_backward(dHo, H, F, w)
    _, Hp, (Ht, Ft, wt, _) = torch_layer(H, F, w, g, 1e-6, n)
    (Hp * torch.tensor(dHo.astype(np.float64))).sum().backward()
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dF, Ft.grad.numpy(), rtol=1e-12, atol=1e-12)
    dw_ref = wt.grad.numpy()
    got = dw if per_token else dw.sum(axis=0)
    np.testing.assert_allclose(got, dw_ref, rtol=1e-12, atol=1e-11)
    assert np.all(dw[:, :n] == 0)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("per_token", [False, True])
def test_pre_backward_matches_autograd(orc, rng, n, per_token):
    T, d, eps = 6, 40, 1e-5
    H, F, w, g = rand_case(rng, T, n, d, per_token)
    du = rng.standard_normal((T, d)).astype(np.float32)
    dH_in = rng.standard_normal((T, n, d))
    dH, dw, dg = orc.pre_mix_backward(du, H, w, g, eps, dH_in=dH_in)
    u, _, (Ht, _, wt, gt) = torch_layer(H, F, w, g, eps, n)
    (u * torch.tensor(du.astype(np.float64))).sum().backward()
    np.testing.assert_allclose(dH, Ht.grad.numpy() + dH_in, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dg, gt.grad.numpy(), rtol=1e-11, atol=1e-11)
    got = dw if per_token else dw.sum(axis=0)
    np.testing.assert_allclose(got, wt.grad.numpy(), rtol=1e-11, atol=1e-11)
    assert np.all(dw[:, n:] == 0)
    dH0, _, _ = orc.pre_mix_backward(du, H, w, g, eps)
    np.testing.assert_allclose(dH0 + dH_in, dH, rtol=1e-14, atol=1e-14)


def test_weight_and_gain_gradients_by_finite_differences(orc, rng):
    """Central differences of the forward oracle, one weight entry or gain
    entry at a time (float64 perturbations, exact)."""
    T, n, d, h = 3, 3, 16, 1e-6
    H, F, w, g = rand_case(rng, T, n, d, per_token=True)
    du = rng.standard_normal((T, d)).astype(np.float32)
    dHo = rng.standard_normal((T, n, d)).astype(np.float32)
    Lpost = lambda ww: float(np.sum(orc.post_mix(H, F, ww) * dHo))          # noqa: E731
    Lpre = lambda ww, gg: float(np.sum(orc.pre_mix(H, ww, gg, 1e-6) * du))  # noqa: E731
    _, _, dw_post = orc.post_mix_backward(dHo, H, F, w)
    _, dw_pre, dg = orc.pre_mix_backward(du, H, w, g, 1e-6)
    for t in range(T):
        for c in range(2 * n + n * n):
            wp, wm = w.copy(), w.copy()
            wp[t, c] += h
            wm[t, c] -= h
            fd_post = (Lpost(wp) - Lpost(wm)) / (2 * h)
            fd_pre = (Lpre(wp, g) - Lpre(wm, g)) / (2 * h)
            assert abs(fd_post - dw_post[t, c]) <= 1e-6 * max(1.0, abs(fd_post))
            assert abs(fd_pre - dw_pre[t, c]) <= 1e-6 * max(1.0, abs(fd_pre))
    for k in range(d):
        gp, gm = g.copy(), g.copy()
        gp[k] += h
        gm[k] -= h
        fd = (Lpre(w, gp) - Lpre(w, gm)) / (2 * h)
        assert abs(fd - dg[k]) <= 1e-6 * max(1.0, abs(fd))


def test_post_adjoint_identity(orc, rng):
    """post is linear in (H, F): <dH', post(H, F)> = <dH, H> + <dF, F>."""
    T, n, d = 7, 4, 32
    H, F, w, g = rand_case(rng, T, n, d, per_token=True)
    dHo = rng.standard_normal((T, n, d)).astype(np.float32)
    dH, dF, _ = orc.post_mix_backward(dHo, H, F, w)
    lhs = float(np.sum(dHo.astype(np.float64) * orc.post_mix(H, F, w)))
    rhs = float(np.sum(dH * H) + np.sum(dF * F))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))
