"""GPU parity of the backward kernels (gradients of post and pre, the
deterministic sums) against the oracle's gradients, through the C ABI.

Gradient records are sums over d of products accumulated in fp32; with
random signs they cancel, so they are held to 1e-4 of the record's RMS
(TOL_GRAD); storage outputs (dH, dF) to the storage tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, need_gpu, rel_err, record_margin
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import f32_to_bf16_bits, identity_record, make_inputs, workload

pytestmark = pytest.mark.gpu

TOL_GRAD = 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def storage(x, dt):
    return f32_to_bf16_bits(x) if dt == "bf16" else x.astype(np.float32)


def grad_check(got, ref, what):
    e = rel_err(np.asarray(got, np.float64), np.asarray(ref, np.float64))
    record_margin(what, e, TOL_GRAD)
    assert e <= TOL_GRAD, f"{what}: {e:.3g} > {TOL_GRAD}"


def dalpha_check(got, ref, du, H, w, g, eps, what):
    """dalpha_i = sum_k dx_k H_ik cancels by construction (RMSNorm is scale
    invariant, so sum_i alpha_i dalpha_i = sum_k dx_k x_k ~ 0; at n = 1 dalpha
    itself is ~0), so it is compared against its Cauchy-Schwarz bound
    |dx| |H_i| rather than its own size."""
    Hf = oracle.widen(H)
    T, n, d = Hf.shape
    W = np.broadcast_to(w, (T, w.shape[-1])).astype(np.float64)
    x = np.einsum("ti,tid->td", W[:, :n], Hf)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    dy = g[None, :] * oracle.widen(du)
    dx = r * (dy - x * r * r * np.mean(dy * x, axis=1, keepdims=True))
    bound = np.linalg.norm(dx, axis=1)[:, None] * np.linalg.norm(Hf, axis=2)
    got = np.asarray(got, np.float64).reshape(-1, W.shape[1])[:, :n]
    ref = np.asarray(ref, np.float64).reshape(-1, W.shape[1])[:, :n]
    if got.shape[0] == 1:          # shared record: summed over tokens
        bound = bound.sum(axis=0, keepdims=True)
    e = np.max(np.abs(got - ref) / np.maximum(bound, 1e-30))
    record_margin(what + " (of the Cauchy-Schwarz bound)", e, 1e-5)
    assert e <= 1e-5, f"{what}: {e:.3g} of the Cauchy-Schwarz bound"


def case(rng, dt, T, n, d, per_token):
    K = 2 * n + n * n
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    F = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    G = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    du = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    shape = (T, K) if per_token else (K,)
    w = (np.broadcast_to(identity_record(n), shape) + 0.3 * rng.standard_normal(shape)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return H, F, G, du, w, g


# every launch shape: 1..4 vectors per thread (bf16 d > 8192, fp32 d > 4096)
SHAPES = [("bf16", 8), ("bf16", 520), ("bf16", 4096), ("bf16", 6144), ("bf16", 8200),
          ("bf16", 12288), ("bf16", 16384), ("f32", 4), ("f32", 1024), ("f32", 4100),
          ("f32", 8192), ("f32", 12288), ("f32", 12296), ("f32", 16384)]


@pytest.mark.parametrize("dt,d", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_post_backward_parity(dt, d, n):
    rng = np.random.default_rng(d * 11 + n)
    T = 9
    H, F, G, du, w, g = case(rng, dt, T, n, d, per_token=(d % 3 == 0))
    dH, dF, dw = hc.post_mix_backward(dev(G), dev(H), dev(F), dev(w))
    rdH, rdF, rdw = oracle.post_mix_backward(G, H, F, w.astype(np.float64))
    check(host(dH), rdH, f"post dH n={n} d={d}")
    check(host(dF), rdF, f"post dF n={n} d={d}")
    if w.ndim == 1:                 # shared record: the gradient is the sum over tokens
        rdw = rdw.sum(axis=0)[None]
        got = host(dw)[None]
    else:
        got = host(dw)
    grad_check(got, rdw, f"post dw n={n} d={d}")


@pytest.mark.parametrize("dt,d", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("acc", [False, True])
def test_pre_backward_parity(dt, d, n, acc):
    rng = np.random.default_rng(d * 13 + n + 7 * acc)
    T = 21          # several dgamma groups, the last one partial
    H, F, G, du, w, g = case(rng, dt, T, n, d, per_token=(d % 3 != 0))
    dH_in = G if acc else None
    dH, dw, dg = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), 1e-6,
                                     dH_in=dev(dH_in) if acc else None)
    rdH, rdw, rdg = oracle.pre_mix_backward(du, H, w.astype(np.float64), g, 1e-6,
                                            dH_in=oracle.widen(dH_in) if acc else None)
    check(host(dH), rdH, f"pre dH n={n} d={d}")
    if w.ndim == 1:
        rdw = rdw.sum(axis=0)
    dalpha_check(host(dw), rdw, du, H, w, g, 1e-6, f"pre dalpha n={n} d={d}")
    assert np.all(host(dw).reshape(-1, 2 * n + n * n)[:, n:] == 0)
    grad_check(host(dg)[None, :], rdg[None, :], f"pre dgamma n={n} d={d}")


@pytest.mark.parametrize("dt,d", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_backward_fold_parity(dt, d, n):
    """post_mix_backward without dH, then pre_mix_backward given dH_out: dH is
    the write-back's H gradient plus the pre gradient, formed in one pass and
    rounded once, so it meets the one-ulp bound; dF and the post records are
    bitwise those of the unfolded call."""
    rng = np.random.default_rng(d * 17 + n)
    T = 11
    H, F, G, du, w, g = case(rng, dt, T, n, d, per_token=(d % 2 == 0))
    dH0, dF0, dw0 = hc.post_mix_backward(dev(G), dev(H), dev(F), dev(w))
    none, dF, dwp = hc.post_mix_backward(dev(G), dev(H), dev(F), dev(w), h_grad=False)
    assert none is None
    assert np.array_equal(host(dF), host(dF0)) and np.array_equal(host(dwp), host(dw0))
    dH, dwq, dg = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), 1e-6, dH_out=dev(G))
    w64 = w.astype(np.float64)
    rdH_post = oracle.post_mix_backward(G, H, F, w64)[0]
    rdH, rdw, rdg = oracle.pre_mix_backward(du, H, w64, g, 1e-6, dH_in=rdH_post)
    check(host(dH), rdH, f"folded dH n={n} d={d}")
    # the pre records and dgamma do not depend on the addend
    _, dwq0, dg0 = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), 1e-6)
    assert np.array_equal(host(dwq), host(dwq0)) and np.array_equal(host(dg), host(dg0))


@pytest.mark.parametrize("per_token", [False, True])
def test_pre_backward_records_only(per_token):
    """dH = NULL: the records and dgamma alone, bitwise those of the full call."""
    rng = np.random.default_rng(6 + per_token)
    H, F, G, du, w, g = case(rng, "bf16", 300, 4, 4096, per_token=per_token)
    dH, dw, dg = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), 1e-6, h_grad=False)
    assert dH is None
    _, dw0, dg0 = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), 1e-6)
    assert np.array_equal(host(dw), host(dw0)) and np.array_equal(host(dg), host(dg0))
    # dalpha alone (no dgamma): one token per workgroup for per-token
    # records; the same sums per token and wave, so the same bits
    _, dw1, dg1 = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), 1e-6, h_grad=False,
                                      g_grad=False)
    assert dg1 is None
    if per_token:
        assert np.array_equal(host(dw1), host(dw0))
    else:
        rdw = oracle.pre_mix_backward(du, H, w.astype(np.float64), g, 1e-6)[1].sum(axis=0)
        dalpha_check(host(dw1), rdw, du, H, w, g, 1e-6, "pre dalpha alone")


def test_pre_backward_accumulates_in_place():
    rng = np.random.default_rng(3)
    H, F, G, du, w, g = case(rng, "bf16", 17, 4, 4096, per_token=True)
    ref_dH, _, _ = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), dH_in=dev(G))
    acc = dev(G)
    ptr = acc.data_ptr()
    out, _, _ = hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), dH_in=acc, out=acc)
    assert out.data_ptr() == ptr
    assert np.array_equal(host(acc), host(ref_dH))


def test_backward_deterministic():
    rng = np.random.default_rng(4)
    H, F, G, du, w, g = case(rng, "bf16", 300, 4, 4096, per_token=False)
    runs = [[host(x) for x in hc.pre_mix_backward(dev(du), dev(H), dev(w), dev(g), dH_in=dev(G))]
            for _ in range(2)]
    for a, b in zip(*runs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("T,K", [(1, 24), (255, 24), (8192, 24), (1000, 3), (37, 15)])
def test_sum_records(T, K):
    rng = np.random.default_rng(T + K)
    rec = rng.standard_normal((T, K)).astype(np.float32)
    got = host(hc.sum_records(dev(rec)))
    ref = rec.astype(np.float64).sum(axis=0)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5 * np.sqrt(T))


def test_static_layer_backward_full_size():
    """T=8192, n=4, d=4096 bf16 with shared weights: post backward, then pre
    backward accumulating into the same dH; dgamma and the shared weight
    gradients (summed records), dH and dF against the oracle over all
    tokens."""
    wl = workload("static-bf16")
    inp = make_inputs(wl)
    rng = np.random.default_rng(77)
    T, n, d = wl.T, wl.n, wl.d
    G = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    du = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Hd, Fd, wd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["w"]), dev(inp["gamma"])
    dH, dF, dw_post = hc.post_mix_backward(dev(G), Hd, Fd, wd)
    dH, dw_pre, dg = hc.pre_mix_backward(dev(du), Hd, wd, gd, wl.eps, dH_in=dH, out=dH)
    gw = host(dw_post) + host(dw_pre)
    w64 = inp["w"].astype(np.float64)
    oracle.set_threads(0)
    r_post = oracle.post_mix_backward(G, inp["H"], inp["F"], w64)
    r_pre = oracle.pre_mix_backward(du, inp["H"], w64, inp["gamma"], wl.eps,
                                    dH_in=oracle.widen(oracle.round_bf16(r_post[0])))
    grad_check(gw[None, n:], r_post[2].sum(0)[None, n:], "shared dbeta, dA")
    dalpha_check(gw[None, :], r_pre[1].sum(0)[None, :], du, inp["H"], inp["w"], inp["gamma"], wl.eps,
                 "shared dalpha")
    grad_check(host(dg)[None, :], r_pre[2][None, :], "dgamma")
    # every token, in chunks; dH on the GPU is the bf16-stored post gradient
    # plus the pre gradient, rounded again: two roundings, so only the bf16
    # tolerance applies
    dFh, dHh = host(dF), host(dH)
    for t0 in range(0, T, 1024):
        sl = slice(t0, t0 + 1024)
        check(dFh[sl], r_post[1][sl], f"dF {t0}+")
        check(dHh[sl], r_pre[0][sl], f"dH {t0}+", one_ulp=False)


def test_static_layer_backward_folded_full_size():
    """The same static layer (T=8192, n=4, d=4096 bf16) through the folded
    pair: post without dH, pre adding A^T dH' itself; every token of dH
    against the oracle's exact sum at the one-ulp bound (one rounding), dF and
    the shared records bitwise those of the unfolded pair."""
    wl = workload("static-bf16")
    inp = make_inputs(wl)
    rng = np.random.default_rng(77)
    T, n, d = wl.T, wl.n, wl.d
    G = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    du = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Hd, Fd, wd, gd, Gd = dev(inp["H"]), dev(inp["F"]), dev(inp["w"]), dev(inp["gamma"]), dev(G)
    dH0, dF0, dwp0 = hc.post_mix_backward(Gd, Hd, Fd, wd)
    _, dwq0, dg0 = hc.pre_mix_backward(dev(du), Hd, wd, gd, wl.eps, dH_in=dH0, out=dH0)
    _, dF, dwp = hc.post_mix_backward(Gd, Hd, Fd, wd, h_grad=False)
    dH, dwq, dg = hc.pre_mix_backward(dev(du), Hd, wd, gd, wl.eps, dH_out=Gd)
    assert np.array_equal(host(dF), host(dF0)) and np.array_equal(host(dwp), host(dwp0))
    assert np.array_equal(host(dwq), host(dwq0)) and np.array_equal(host(dg), host(dg0))
    w64 = inp["w"].astype(np.float64)
    oracle.set_threads(0)
    r_post = oracle.post_mix_backward(G, inp["H"], inp["F"], w64)
    r_pre = oracle.pre_mix_backward(du, inp["H"], w64, inp["gamma"], wl.eps, dH_in=r_post[0])
    dHh = host(dH)
    for t0 in range(0, T, 1024):
        sl = slice(t0, t0 + 1024)
        check(dHh[sl], r_pre[0][sl], f"folded dH {t0}+")


def test_dynamic_layer_backward_folded_full_size():
    """The dynamic workload's shape (T=16384, n=4, d=4096 bf16) with one record
    per token, drawn on the host: post without dH, pre forming the whole dH.
    Every token of dH (one-ulp bound) and dF, the per-token dbeta/dA records,
    dalpha (Cauchy-Schwarz bound) and dgamma against the oracle, in chunks of
    2048 tokens (the gradients are per token, so a chunk is exact)."""
    wl = workload("dynamic-bf16")
    inp = make_inputs(wl)
    assert "F" in inp
    rng = np.random.default_rng(79)
    T, n, d, K = wl.T, wl.n, wl.d, wl.K
    w = (identity_record(n)[None, :] + 0.3 * rng.standard_normal((T, K))).astype(np.float32)
    G = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    du = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    Hd, Fd, wd, Gd = dev(inp["H"]), dev(inp["F"]), dev(w), dev(G)
    none, dF, dwp = hc.post_mix_backward(Gd, Hd, Fd, wd, h_grad=False)
    dH, dwq, dg = hc.pre_mix_backward(dev(du), Hd, wd, dev(inp["gamma"]), wl.eps, dH_out=Gd)
    assert none is None
    dHh, dFh, dwph, dwqh, dgh = host(dH), host(dF), host(dwp), host(dwq), host(dg)
    w64 = w.astype(np.float64)
    oracle.set_threads(0)
    rdg = np.zeros(d)
    for t0 in range(0, T, 2048):
        sl = slice(t0, t0 + 2048)
        r_post = oracle.post_mix_backward(G[sl], inp["H"][sl], inp["F"][sl], w64[sl])
        r_pre = oracle.pre_mix_backward(du[sl], inp["H"][sl], w64[sl], inp["gamma"], wl.eps,
                                        dH_in=r_post[0])
        check(dHh[sl], r_pre[0], f"folded dH {t0}+")
        check(dFh[sl], r_post[1], f"dF {t0}+")
        grad_check(dwph[sl][:, n:], r_post[2][:, n:], f"post records {t0}+")
        assert np.all(dwph[sl][:, :n] == 0)
        dalpha_check(dwqh[sl], r_pre[1], du[sl], inp["H"][sl], w[sl], inp["gamma"], wl.eps,
                     f"dalpha {t0}+")
        rdg += r_pre[2]
    grad_check(dgh[None, :], rdg[None, :], "dgamma")
