"""Pins of the oracle's gradients of the per-token weights and of the mHC
(Sinkhorn) transform.

Pins: torch.autograd in float64 through torch's own tanh, sigmoid, exp,
sums and matmul (library routines differentiating the forward formula);
central finite differences of the forward oracle (itself pinned), perturbing
float64 logits exactly and fp32-stored inputs by a power of two (exact)."""
import numpy as np
import pytest
import torch

from hyper_connections_amd.workloads import identity_record


def torch_mhc(l, n, iters):
    """The mHC transform on (T, K) logits with torch ops."""
    alpha, beta = torch.sigmoid(l[:, :n]), torch.sigmoid(l[:, n:2 * n])
    M = torch.exp(l[:, 2 * n:]).reshape(-1, n, n)
    for _ in range(iters):
        M = M / M.sum(dim=2, keepdim=True)
        M = M / M.sum(dim=1, keepdim=True)
    return torch.cat([alpha, beta, M.reshape(-1, n * n)], dim=1)


def torch_weights(H, W, ws, scale, eps, iters):
    Ht = torch.tensor(H.astype(np.float64), requires_grad=True)
    Wt = torch.tensor(W.astype(np.float64), requires_grad=True)
    wst = torch.tensor(ws.astype(np.float64), requires_grad=True)
    r = 1.0 / torch.sqrt((Ht * Ht).mean(dim=2, keepdim=True) + eps)
    hbar = (r * Ht).mean(dim=1)
    z = hbar @ Wt.T
    n = H.shape[1]
    if iters == 0:
        w = wst + scale * torch.tanh(z)
    else:
        w = torch_mhc(wst + scale * z, n, iters)
    return w, (Ht, Wt, wst)


def case(rng, T, n, d):
    K = 2 * n + n * n
    H = rng.standard_normal((T, n, d)).astype(np.float32)
    W = (0.3 * rng.standard_normal((K, d))).astype(np.float32)
    ws = (identity_record(n) + 0.2 * rng.standard_normal(K)).astype(np.float64)
    dw = rng.standard_normal((T, K))
    return H, W, ws, dw


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 1, 5, 20])
def test_weights_backward_matches_autograd(orc, rng, n, iters):
    T, d, scale, eps = 4, 24, 0.7, 1e-5
    H, W, ws, dw = case(rng, T, n, d)
    dH, dW, dws = orc.weights_backward(H, W, ws, scale, dw, eps, iters)
    w, (Ht, Wt, wst) = torch_weights(H, W, ws, scale, eps, iters)
    np.testing.assert_allclose(w.detach().numpy(), orc.weights(H, W, ws, scale, eps, iters),
                               rtol=1e-12, atol=1e-13)
    (w * torch.tensor(dw)).sum().backward()
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(dws, wst.grad.numpy(), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 1, 3, 20])
def test_sinkhorn_backward_matches_autograd_and_differences(orc, rng, n, iters):
    T, K = 5, 2 * n + n * n
    lg = rng.standard_normal((T, K))
    dw = rng.standard_normal((T, K))
    got = orc.sinkhorn_backward(lg, dw, n, iters)
    lt = torch.tensor(lg, requires_grad=True)
    (torch_mhc(lt, n, iters) * torch.tensor(dw)).sum().backward()
    np.testing.assert_allclose(got, lt.grad.numpy(), rtol=1e-10, atol=1e-12)
    # central differences of the forward oracle, every logit of token 0
    h = 1e-6
    for c in range(K):
        lp, lm = lg.copy(), lg.copy()
        lp[0, c] += h
        lm[0, c] -= h
        fd = ((orc.sinkhorn(lp, n, iters) - orc.sinkhorn(lm, n, iters))[0] * dw[0]).sum() / (2 * h)
        assert abs(fd - got[0, c]) <= 1e-6 * max(1.0, abs(fd)), (c, fd, got[0, c])


def test_weights_backward_by_finite_differences(orc, rng):
    """Central differences of the forward oracle in W, H and w_static with
    fp32 storage: the perturbation 2^-12 is exact for |x| < 2^11."""
    T, n, d, scale, eps = 3, 3, 16, 0.5, 1e-6
    H, W, ws, dw = case(rng, T, n, d)
    for iters in (0, 4):
        dH, dW, dws = orc.weights_backward(H, W, ws, scale, dw, eps, iters)
        loss = lambda H_, W_, ws_: float((orc.weights(H_, W_, ws_, scale, eps, iters) * dw).sum())  # noqa: E731
        h = np.float32(2.0 ** -12)
        for (c, k) in [(0, 0), (n, 5), (2 * n + 1, 11), (2 * n + n * n - 1, d - 1)]:
            Wp, Wm = W.copy(), W.copy()
            Wp[c, k] += h
            Wm[c, k] -= h
            fd = (loss(H, Wp, ws) - loss(H, Wm, ws)) / (2 * float(h))
            assert abs(fd - dW[c, k]) <= 2e-5 * max(1.0, abs(fd)), ("W", iters, c, k, fd, dW[c, k])
        for (t, i, k) in [(0, 0, 0), (1, 2, 7), (2, 1, d - 1)]:
            Hp, Hm = H.copy(), H.copy()
            Hp[t, i, k] += h
            Hm[t, i, k] -= h
            fd = (loss(Hp, W, ws) - loss(Hm, W, ws)) / (2 * float(h))
            assert abs(fd - dH[t, i, k]) <= 2e-5 * max(1.0, abs(fd)), ("H", iters, t, i, k, fd)
        for c in range(0, 2 * n + n * n, 5):
            wp, wm = ws.copy(), ws.copy()
            wp[c] += 1e-6
            wm[c] -= 1e-6
            fd = (loss(H, W, wp) - loss(H, W, wm)) / 2e-6
            assert abs(fd - dws[c]) <= 1e-6 * max(1.0, abs(fd)), ("w_static", iters, c, fd)


def test_zero_projection_gradients(orc, rng):
    """W = 0: z = 0, so in tanh mode dz = scale * dw, dW[c] = sum_t dz_c hbar,
    dH = 0 (dhbar = W^T dz = 0) and dw_static = sum_t dw."""
    T, n, d, scale = 4, 4, 32, 0.01
    H, W, ws, dw = case(rng, T, n, d)
    W[:] = 0
    dH, dW, dws = orc.weights_backward(H, W, ws, scale, dw, 1e-6, 0)
    assert not dH.any()
    np.testing.assert_allclose(dws, dw.sum(axis=0), rtol=1e-14, atol=1e-14)
    Hd = H.astype(np.float64)
    r = 1 / np.sqrt((Hd * Hd).mean(axis=2, keepdims=True) + 1e-6)
    hbar = (r * Hd).mean(axis=1)
    np.testing.assert_allclose(dW, scale * dw.T @ hbar, rtol=1e-12, atol=1e-14)
