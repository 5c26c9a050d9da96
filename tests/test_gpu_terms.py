"""GPU parity of the weight producer's gradient returned as its two factors
(hc_weights_backward_terms: dhbar and the per-token coefficients) and of the
layer boundary's gradient that adds them at H' (hc_post_pre_mix_backward_terms),
against the oracle, through the C ABI.

The gradient the producer sends to stream i is a_i dhbar + b_i H_i; the
oracle's weights_backward returns it whole (dH), so the factors are checked
through that sum, formed on the host in float64 from the GPU's fp32 outputs
(gradient tolerance: 1e-4 of the RMS).  The boundary's expected values chain
the oracle: G = dH_out + the producer's term on the stored H', then the
read-mix and write-back gradients as in the boundary tests."""
import numpy as np
import pytest

import oracle
from gpu_util import check, dev, host, need_gpu, rel_err, record_margin
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import f32_to_bf16_bits, identity_record, make_inputs, workload
from test_gpu_backward import dalpha_check, grad_check, storage
from test_gpu_boundary_backward import unambiguous

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def producer_case(rng, dt, T, n, d, wsd=0.05):
    K = 2 * n + n * n
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    W = storage((wsd * rng.standard_normal((K, d))).astype(np.float32), dt)
    ws = (identity_record(n) + 0.1 * rng.standard_normal(K)).astype(np.float32)
    dw = rng.standard_normal((T, K)).astype(np.float32)
    return H, W, ws, dw


def term_of(dhbar, coef, H):
    """a_i dhbar + b_i H_i in float64 from the returned factors."""
    n = coef.shape[1] // 2
    a, b = coef[:, :n].astype(np.float64), coef[:, n:].astype(np.float64)
    return a[:, :, None] * dhbar.astype(np.float64)[:, None, :] + b[:, :, None] * oracle.widen(H)


# d: one column group, ragged column groups, the workload width; T ragged
@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 264), ("bf16", 4096),
                                  ("f32", 4), ("f32", 132), ("f32", 1024)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 20])
def test_weights_backward_terms_parity(dt, d, n, iters):
    """The factors' term against the oracle's dH; dW and dw_static against
    the oracle and bitwise those of hc_weights_backward (the same sums)."""
    rng = np.random.default_rng(d * 11 + n * 5 + iters)
    T = 37
    H, W, ws, dw = producer_case(rng, dt, T, n, d)
    scale = 0.5
    dhbar, coef, dW, dws = hc.weights_backward_terms(dev(H), dev(W), dev(ws), scale, dev(dw), 1e-6,
                                                     iters)
    rdH, rdW, rdws = oracle.weights_backward(H, W, ws.astype(np.float64), scale,
                                             dw.astype(np.float64), 1e-6, iters)
    what = f"n={n} d={d} {dt} iters={iters}"
    grad_check(term_of(host(dhbar), host(coef), H), rdH, f"terms {what}")
    grad_check(host(dW), rdW, f"terms dW {what}")
    grad_check(host(dws)[None], rdws[None], f"terms dw_static {what}")
    _, dW2, dws2 = hc.weights_backward(dev(H), dev(W), dev(ws), scale, dev(dw), 1e-6, iters)
    assert np.array_equal(host(dW), host(dW2)), f"dW differs from hc_weights_backward's ({what})"
    assert np.array_equal(host(dws), host(dws2)), f"dw_static differs ({what})"


def test_weights_backward_terms_with_saved_and_dw2():
    """The kept projections and a second record gradient give the same
    factors as recomputing them with dw + dw2 in one record."""
    rng = np.random.default_rng(5)
    T, n, d = 300, 4, 2048
    H, W, ws, dw = producer_case(rng, "bf16", T, n, d)
    dw2 = rng.standard_normal(dw.shape).astype(np.float32)
    Hd, Wd, wsd = dev(H), dev(W), dev(ws)
    _, saved = hc.weights_save(Hd, Wd, wsd, 0.01, 1e-6, 0)
    a = [host(x) for x in hc.weights_backward_terms(Hd, Wd, wsd, 0.01, dev(dw), dw2=dev(dw2),
                                                    saved=saved)]
    rdH, rdW, rdws = oracle.weights_backward(H, W, ws.astype(np.float64), 0.01,
                                             dw.astype(np.float64) + dw2.astype(np.float64))
    grad_check(term_of(a[0], a[1], H), rdH, "terms (saved, dw2)")
    grad_check(a[2], rdW, "terms dW (saved, dw2)")
    grad_check(a[3][None], rdws[None], "terms dw_static (saved, dw2)")


def boundary_terms_case(rng, dt, T, n, d):
    K = 2 * n + n * n
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    F = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    G = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    du = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    w = (identity_record(n)[None, :] + 0.3 * rng.standard_normal((T, K))).astype(np.float32)
    wn = (identity_record(n)[None, :] + 0.3 * rng.standard_normal((T, K))).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    dhbar = rng.standard_normal((T, d)).astype(np.float32)
    coef = np.concatenate([0.5 + 0.1 * rng.standard_normal((T, n)),
                           0.01 * rng.standard_normal((T, n))], axis=1).astype(np.float32)
    H, F = unambiguous(H, F, w)
    return H, F, G, du, w, wn, g, dhbar, coef


def oracle_boundary_terms(G, du, H, F, w, wn, g, eps, term):
    """The oracle's boundary gradients with the producer's term (float64, on
    the stored H') added to the gradient arriving at H': (dH, dF, dw, dw_next,
    dgamma, H' as stored)."""
    w64, wn64 = w.astype(np.float64), wn.astype(np.float64)
    Hp = oracle.post_mix(H, F, w64)
    Hs = oracle.round_bf16(Hp) if H.dtype == np.uint16 else oracle.round_f32(Hp)
    Gt, rdwn, rdg = oracle.pre_mix_backward(du, Hs, wn64, g, eps,
                                            dH_in=oracle.widen(G) + term(Hs))
    rdH, rdF, rdw = oracle.post_mix_backward(Gt, oracle.widen(H), oracle.widen(F), w64)
    return rdH, rdF, rdw, rdwn, rdg, Hs


def compare_terms(got, ref, du, wn, g, eps, n, what, dgamma=True):
    dH, dF, dw, dwn = got[:4]
    rdH, rdF, rdw, rdwn, rdg, Hs = ref
    check(dH, rdH, f"{what} dH")
    check(dF, rdF, f"{what} dF")
    assert np.all(dw[:, :n] == 0) and np.all(dwn[:, n:] == 0), f"{what}: zero slots"
    grad_check(dw[:, n:], rdw[:, n:], f"{what} dbeta, dA")
    dalpha_check(dwn, rdwn, du, Hs, wn, g, eps, f"{what} dalpha")
    if dgamma:
        grad_check(got[4][None, :], rdg[None, :], f"{what} dgamma")


# every vectors-per-thread launch shape of the boundary kernel
@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 520), ("bf16", 4096), ("bf16", 8200),
                                  ("bf16", 16384), ("f32", 4), ("f32", 1024), ("f32", 4100),
                                  ("f32", 12296)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_boundary_backward_terms_parity(dt, d, n):
    rng = np.random.default_rng(d * 3 + n)
    T, eps = 13, 1e-6
    H, F, G, du, w, wn, g, dhbar, coef = boundary_terms_case(rng, dt, T, n, d)
    got = [host(x) for x in hc.post_pre_mix_backward(dev(G), dev(du), dev(H), dev(F), dev(w),
                                                     dev(wn), dev(g), eps,
                                                     terms=(dev(dhbar), dev(coef)))]
    ref = oracle_boundary_terms(G, du, H, F, w, wn, g, eps, lambda Hs: term_of(dhbar, coef, Hs))
    compare_terms(got, ref, du, wn, g, eps, n, f"terms boundary n={n} d={d} {dt}")


def test_boundary_backward_terms_zero_is_plain_call():
    """With dhbar = 0 and coef = 0 the terms add exact zeros: every output is
    bitwise the plain hc_post_pre_mix_backward's."""
    rng = np.random.default_rng(77)
    T, n, d, eps = 40, 4, 4096, 1e-6
    H, F, G, du, w, wn, g, _, _ = boundary_terms_case(rng, "bf16", T, n, d)
    args = (dev(du), dev(H), dev(F), dev(w), dev(wn), dev(g), eps)
    plain = [host(x) for x in hc.post_pre_mix_backward(dev(G), *args)]
    zero = (dev(np.zeros((T, d), np.float32)), dev(np.zeros((T, 2 * n), np.float32)))
    terms = [host(x) for x in hc.post_pre_mix_backward(dev(G), *args, terms=zero)]
    for a, b, name in zip(plain, terms, ("dH", "dF", "dw", "dw_next", "dgamma")):
        assert np.array_equal(a, b), name


@pytest.mark.timeout(600)
def test_stack_with_per_token_weights_through_terms():
    """Three layers whose records are produced from the streams (tanh mode,
    W shared, fp32 storage, T = 64, d = 1024), with the producer's gradient
    carried as its factors: per layer, the read-mix's dalpha alone, the
    producer's factors (hc_weights_backward_terms), then the boundary's
    gradient adding them at H' (hc_post_pre_mix_backward_terms); the first
    layer ends with the producer's dH and the read-mix's gradient.  Against
    the oracle's chain: dH at the input, every layer's dF, records, dW and
    dgamma."""
    rng = np.random.default_rng(29)
    L, T, n, d, eps, scale = 3, 64, 4, 1024, 1e-6, 0.01
    K = 2 * n + n * n
    f32 = lambda *sh: rng.standard_normal(sh).astype(np.float32)  # noqa: E731
    H0 = f32(T, n, d)
    Fs = [f32(T, d) for _ in range(L)]
    dus = [f32(T, d) for _ in range(L)]
    dHL = f32(T, n, d)
    W = (0.02 * rng.standard_normal((K, d))).astype(np.float32)
    wst = identity_record(n).astype(np.float32)
    gs = [(1 + 0.1 * rng.standard_normal(d)).astype(np.float32) for _ in range(L)]

    Hs, ws = [H0], []
    for l in range(L):
        ws.append(oracle.weights(Hs[l], W, wst.astype(np.float64), scale, eps, 0).astype(np.float32))
        if l < L - 1:
            Hs.append(oracle.round_f32(oracle.post_mix(Hs[l], Fs[l], ws[l].astype(np.float64))))
    w64 = [w.astype(np.float64) for w in ws]

    r_dF, r_dw, r_dW, r_dg = [None] * L, [np.zeros((T, K)) for _ in range(L)], [None] * L, [None] * L
    gH, r_dF[L - 1], rw = oracle.post_mix_backward(oracle.widen(dHL), oracle.widen(Hs[L - 1]),
                                                  oracle.widen(Fs[L - 1]), w64[L - 1])
    r_dw[L - 1] += rw
    for l in range(L - 1, -1, -1):
        _, rwn, r_dg[l] = oracle.pre_mix_backward(dus[l], Hs[l], w64[l], gs[l], eps)
        r_dw[l] += rwn
        dHw, r_dW[l], _ = oracle.weights_backward(Hs[l], W, wst.astype(np.float64), scale, r_dw[l], eps, 0)
        Gt, _, _ = oracle.pre_mix_backward(dus[l], Hs[l], w64[l], gs[l], eps, dH_in=gH + dHw)
        if l == 0:
            r_dH0 = Gt
            break
        gH, r_dF[l - 1], rw = oracle.post_mix_backward(Gt, oracle.widen(Hs[l - 1]),
                                                       oracle.widen(Fs[l - 1]), w64[l - 1])
        r_dw[l - 1] += rw

    Hd, wd, gd = [dev(x) for x in Hs], [dev(x) for x in ws], [dev(x) for x in gs]
    Wd, wsd = dev(W), dev(wst)
    dF, dW, dg, post_part = [None] * L, [None] * L, [None] * L, [None] * L
    buf, dF[L - 1], post_part[L - 1] = hc.post_mix_backward(dev(dHL), Hd[L - 1], dev(Fs[L - 1]), wd[L - 1])
    for l in range(L - 1, -1, -1):
        _, dalpha, dg[l] = hc.pre_mix_backward(dev(dus[l]), Hd[l], wd[l], gd[l], eps, h_grad=False)
        if l == 0:
            buf, dW[0], _ = hc.weights_backward(Hd[0], Wd, wsd, scale, dalpha, eps, 0, dH_in=buf,
                                                out=buf, dw2=post_part[0])
            dH0, _, _ = hc.pre_mix_backward(dev(dus[0]), Hd[0], wd[0], gd[0], eps, dH_in=buf)
            break
        dhbar, coef, dW[l], _ = hc.weights_backward_terms(Hd[l], Wd, wsd, scale, dalpha, eps, 0,
                                                          dw2=post_part[l])
        buf, dF[l - 1], post_part[l - 1], _, _ = hc.post_pre_mix_backward(
            buf, dev(dus[l]), Hd[l - 1], dev(Fs[l - 1]), wd[l - 1], wd[l], gd[l], eps, out=buf,
            terms=(dhbar, coef))

    grad_check(host(dH0), r_dH0, "terms stack dH0")
    for l in range(L):
        grad_check(host(dF[l]), r_dF[l], f"terms stack dF layer {l}")
        grad_check(host(post_part[l])[:, n:], r_dw[l][:, n:], f"terms stack dbeta, dA layer {l}")
        e = rel_err(host(dW[l]), r_dW[l])
        record_margin(f"terms stack dW layer {l}", e, 1e-3)
        assert e <= 1e-3, f"terms stack dW layer {l}: {e:.3g}"
        grad_check(host(dg[l])[None, :], r_dg[l][None, :], f"terms stack dgamma layer {l}")


@pytest.mark.timeout(900)
def test_dynamic_boundary_backward_terms_full_size():
    """The dynamic workload's shape (T=16384, n=4, d=4096 bf16) as the
    benchmark's backward runs it: the producer's factors from the stored H'
    (hc_post_mix's output, bitwise what the boundary recomputes), then the
    boundary's gradient adding them.  Every token's dH, dF and records, and
    dgamma, dW and dw_static, against the oracle in chunks of 2048 tokens."""
    wl = workload("dynamic-bf16")
    inp = make_inputs(wl)
    rng = np.random.default_rng(91)
    T, n, d, K, eps, scale = wl.T, wl.n, wl.d, wl.K, wl.eps, 0.01
    w = (identity_record(n)[None, :] + 0.3 * rng.standard_normal((T, K))).astype(np.float32)
    wn = (identity_record(n)[None, :] + 0.3 * rng.standard_normal((T, K))).astype(np.float32)
    G = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    du = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    dwp = rng.standard_normal((T, K)).astype(np.float32)
    W = f32_to_bf16_bits((0.02 * rng.standard_normal((K, d))).astype(np.float32))
    wst = identity_record(n).astype(np.float32)
    oracle.set_threads(0)
    H, F = unambiguous(inp["H"], inp["F"], w)
    Hd, Fd, wd = dev(H), dev(F), dev(w)
    Hp = hc.post_mix(Hd, Fd, wd)
    dhbar, coef, dW, dws = hc.weights_backward_terms(Hp, dev(W), dev(wst), scale, dev(dwp), eps)
    got = [host(x) for x in hc.post_pre_mix_backward(dev(G), dev(du), Hd, Fd, wd, dev(wn),
                                                     dev(inp["gamma"]), eps, terms=(dhbar, coef))]
    Hp_h = host(Hp)
    del Hp, dhbar, coef
    rdg, rdW, rdws = np.zeros(d), np.zeros((K, d)), np.zeros(K)
    for t0 in range(0, T, 2048):
        sl = slice(t0, t0 + 2048)
        rdHw, cW, cws = oracle.weights_backward(Hp_h[sl], W, wst.astype(np.float64), scale,
                                                dwp[sl].astype(np.float64), eps, 0)
        rdW += cW
        rdws += cws
        ref = oracle_boundary_terms(G[sl], du[sl], H[sl], F[sl], w[sl], wn[sl], inp["gamma"], eps,
                                    lambda Hs: rdHw)
        # the oracle's stored H' is the GPU's (the inputs are off the rounding midpoints)
        assert np.array_equal(ref[5], Hp_h[sl]), f"stored H' {t0}+"
        compare_terms([x[sl] for x in got[:4]], ref, du[sl], wn[sl], inp["gamma"], eps, n,
                      f"terms full size {t0}+", dgamma=False)
        rdg += ref[4]
    grad_check(got[4][None, :], rdg[None, :], "terms full size dgamma")
    grad_check(host(dW), rdW, "terms full size dW")
    grad_check(host(dws)[None], rdws[None], "terms full size dw_static")


def test_terms_rejects():
    rng = np.random.default_rng(3)
    T, n, d = 8, 4, 512
    H, F, G, du, w, wn, g, dhbar, coef = boundary_terms_case(rng, "bf16", T, n, d)
    K = 2 * n + n * n
    shared = identity_record(n).astype(np.float32)
    with pytest.raises(ValueError):      # shared records take no terms
        hc.post_pre_mix_backward(dev(G), dev(du), dev(H), dev(F), dev(shared), dev(shared), dev(g),
                                 terms=(dev(dhbar), dev(coef)))
    with pytest.raises(ValueError):      # coef of the wrong width
        hc.post_pre_mix_backward(dev(G), dev(du), dev(H), dev(F), dev(w), dev(wn), dev(g),
                                 terms=(dev(dhbar), dev(coef[:, :n])))
    H8 = rng.integers(0, 120, (T, n, d), dtype=np.uint8)
    W8 = rng.integers(0, 120, (K, d), dtype=np.uint8)
    with pytest.raises(hc.HCError):      # FP8 storage takes no gradient
        hc.weights_backward_terms(dev(H8), dev(W8), dev(shared), 0.1,
                                  dev(rng.standard_normal((T, K)).astype(np.float32)))
