"""GPU parity of the gradients of the per-token weight producer (tanh and
mHC modes) and of the Sinkhorn step against the oracle, through the C ABI.

dH is a storage output (storage tolerance); dW, dw_static and dlogits are
fp32 sums of products with mixed signs, held to 1e-4 of their RMS like the
other gradient records."""
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


def case(rng, dt, T, n, d, wsd=0.05):
    K = 2 * n + n * n
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    W = storage((wsd * rng.standard_normal((K, d))).astype(np.float32), dt)
    ws = (identity_record(n) + 0.1 * rng.standard_normal(K)).astype(np.float32)
    dw = rng.standard_normal((T, K)).astype(np.float32)
    return H, W, ws, dw


# d: a single column group, ragged groups, the workload width, the largest; T: one token,
# partial tiles, several dW splits
@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 264), ("bf16", 4096), ("bf16", 16384),
                                  ("f32", 4), ("f32", 132), ("f32", 1024), ("f32", 16384)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 5])
def test_weights_backward_parity(dt, d, n, iters):
    rng = np.random.default_rng(d * 7 + n * 3 + iters)
    T = 37
    H, W, ws, dw = case(rng, dt, T, n, d)
    scale = 0.5
    dH, dW, dws = hc.weights_backward(dev(H), dev(W), dev(ws), scale, dev(dw), 1e-6, iters)
    rdH, rdW, rdws = oracle.weights_backward(H, W, ws.astype(np.float64), scale,
                                             dw.astype(np.float64), 1e-6, iters)
    check(host(dH), rdH, f"dH n={n} d={d} {dt} iters={iters}")
    grad_check(host(dW), rdW, f"dW n={n} d={d} {dt} iters={iters}")
    grad_check(host(dws)[None], rdws[None], f"dw_static n={n} d={d} iters={iters}")


@pytest.mark.parametrize("T", [1, 3, 17, 600, 1100])
def test_weights_backward_token_counts(T):
    n, d = 4, 512
    rng = np.random.default_rng(T + 5)
    H, W, ws, dw = case(rng, "bf16", T, n, d)
    dH, dW, dws = hc.weights_backward(dev(H), dev(W), dev(ws), 0.01, dev(dw))
    rdH, rdW, rdws = oracle.weights_backward(H, W, ws.astype(np.float64), 0.01,
                                             dw.astype(np.float64))
    check(host(dH), rdH, f"dH T={T}")
    grad_check(host(dW), rdW, f"dW T={T}")
    grad_check(host(dws)[None], rdws[None], f"dws T={T}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_weights_backward_accumulates(dt):
    """dH = dH_in + this path, also in place."""
    n, d, T = 4, 1024, 21
    rng = np.random.default_rng(31)
    H, W, ws, dw = case(rng, dt, T, n, d)
    G = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    a, _, _ = hc.weights_backward(dev(H), dev(W), dev(ws), 0.3, dev(dw), dH_in=dev(G))
    acc = dev(G)
    b, _, _ = hc.weights_backward(dev(H), dev(W), dev(ws), 0.3, dev(dw), dH_in=acc, out=acc)
    assert np.array_equal(host(a), host(b))
    rdH, _, _ = oracle.weights_backward(H, W, ws.astype(np.float64), 0.3, dw.astype(np.float64))
    check(host(a), rdH + oracle.widen(G), "dH + dH_in", one_ulp=False)


def test_weights_backward_deterministic():
    n, d, T = 4, 2048, 700
    rng = np.random.default_rng(8)
    H, W, ws, dw = case(rng, "bf16", T, n, d)
    runs = [[host(x) for x in hc.weights_backward(dev(H), dev(W), dev(ws), 0.01, dev(dw), 1e-6, 3)]
            for _ in range(3)]
    for r in runs[1:]:
        assert all(np.array_equal(a, b) for a, b in zip(runs[0], r))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 1, 20, 25])
def test_sinkhorn_backward_parity(n, iters):
    """Up to 20 iterations the matrices stay in registers; 25 takes the
    workspace."""
    rng = np.random.default_rng(n * 100 + iters)
    T, K = 1000, 2 * n + n * n
    lg = rng.standard_normal((T, K)).astype(np.float32)
    dw = rng.standard_normal((T, K)).astype(np.float32)
    got = host(hc.sinkhorn_backward(dev(lg), dev(dw), n, iters))
    ref = oracle.sinkhorn_backward(lg.astype(np.float64), dw.astype(np.float64), n, iters)
    grad_check(got, ref, f"dlogits n={n} iters={iters}")


@pytest.mark.parametrize("n", [1, 4])
def test_sinkhorn_backward_two_gradients(n):
    """dw2 (the records' gradient from a second call) is added to dw: against
    the oracle's gradient of dw + dw2, at the configured 20 iterations."""
    rng = np.random.default_rng(n * 7 + 1)
    T, K = 1000, 2 * n + n * n
    lg = rng.standard_normal((T, K)).astype(np.float32)
    dw = rng.standard_normal((T, K)).astype(np.float32)
    dw2 = rng.standard_normal((T, K)).astype(np.float32)
    got = host(hc.sinkhorn_backward(dev(lg), dev(dw), n, 20, dw2=dev(dw2)))
    ref = oracle.sinkhorn_backward(lg.astype(np.float64),
                                   dw.astype(np.float64) + dw2.astype(np.float64), n, 20)
    grad_check(got, ref, f"dlogits from two gradients n={n}")


def test_dynamic_workload_backward_full_size():
    """T=16384, n=4, d=4096 bf16 (the dynamic workload): dH of every token,
    dW and dw_static over all tokens, against the oracle (run in chunks of
    2048 tokens, whose dW and dw_static are summed in fp64); the benchmark's
    form (projections kept by hc_weights_save) bitwise equal to the
    recomputing one."""
    wl = workload("dynamic-bf16")
    inp = make_inputs(wl)
    rng = np.random.default_rng(41)
    dw = (rng.standard_normal((wl.T, wl.K)) * 0.1).astype(np.float32)
    Hd, Wd, wsd = dev(inp["H"]), dev(inp["W"]), dev(inp["w_static"])
    dH, dW, dws = hc.weights_backward(Hd, Wd, wsd, wl.scale, dev(dw), wl.eps)
    # the benchmark's launch: the projections kept by the training forward
    _, saved = hc.weights_save(Hd, Wd, wsd, wl.scale, wl.eps, 0)
    dHs, dWs, dwss = hc.weights_backward(Hd, Wd, wsd, wl.scale, dev(dw), wl.eps, saved=saved)
    assert torch.equal(dH, dHs) and torch.equal(dW, dWs) and torch.equal(dws, dwss)
    del dHs, dWs, dwss, saved
    dH, dW, dws = host(dH), host(dW), host(dws)
    oracle.set_threads(0)
    rdW = np.zeros(dW.shape)
    rdws = np.zeros(dws.shape)
    ws64 = inp["w_static"].astype(np.float64)
    for t0 in range(0, wl.T, 2048):
        sl = slice(t0, t0 + 2048)
        rdH, cW, cws = oracle.weights_backward(inp["H"][sl], inp["W"], ws64, wl.scale,
                                               dw[sl].astype(np.float64), wl.eps)
        check(dH[sl], rdH, f"dynamic dH {t0}+")
        rdW += cW
        rdws += cws
    grad_check(dW, rdW, "dynamic dW")
    grad_check(dws[None], rdws[None], "dynamic dw_static")


def test_weights_backward_two_gradient_records():
    """dw + dw2 (the gradients from pre and post) give the same as their sum
    passed as one record."""
    n, d, T = 4, 1024, 50
    rng = np.random.default_rng(12)
    H, W, ws, dw = case(rng, "bf16", T, n, d)
    dw2 = rng.standard_normal(dw.shape).astype(np.float32)
    a = hc.weights_backward(dev(H), dev(W), dev(ws), 0.2, dev(dw), dw2=dev(dw2))
    b = hc.weights_backward(dev(H), dev(W), dev(ws), 0.2, dev(dw + dw2))
    for x, y in zip(a, b):
        assert np.array_equal(host(x), host(y))


@pytest.mark.parametrize("dt,d", [("bf16", 264), ("bf16", 4096), ("f32", 132)])
@pytest.mark.parametrize("n", [1, 2, 4])
@pytest.mark.parametrize("iters", [0, 5])
def test_weights_backward_with_saved_state(dt, d, n, iters):
    """The state hc_weights_save keeps gives bitwise the gradients of the
    recomputing path (the same kernel forms P and r either way)."""
    rng = np.random.default_rng(d + 5 * n + iters)
    T = 53
    H, W, ws, dw = case(rng, dt, T, n, d)
    Hd, Wd, wsd, dwd = dev(H), dev(W), dev(ws), dev(dw)
    _, saved = hc.weights_save(Hd, Wd, wsd, 0.3, 1e-6, iters)
    a = hc.weights_backward(Hd, Wd, wsd, 0.3, dwd, 1e-6, iters)
    b = hc.weights_backward(Hd, Wd, wsd, 0.3, dwd, 1e-6, iters, saved=saved)
    for x, y in zip(a, b):
        assert np.array_equal(host(x), host(y))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 4])
def test_weights_backward_saturated_tanh(dt, n):
    """Projections of several units (|z| up to ~11): tanh saturates and its
    derivative is a tiny number that 1 - tanh^2 would lose in fp32 (errors of
    ~0.5%); whole tokens then carry only such terms.  bf16 rows are held to one
    ulp.  fp32 rows to 1e-4: at |z| ~ 10 the derivative 4 e^(-2|z|) turns an
    absolute error dz of z into a relative error 2 |z| dz, and fp32 forms z
    (a sum over d of products of size ~|z|) to a few 1e-7 of |z|."""
    rng = np.random.default_rng(77 + n)
    T, d = 64, 1024
    H, W, ws, dw = case(rng, dt, T, n, d, wsd=0.15 * np.sqrt(n))
    dH, dW, dws = hc.weights_backward(dev(H), dev(W), dev(ws), 0.5, dev(dw))
    rdH, rdW, rdws = oracle.weights_backward(H, W, ws.astype(np.float64), 0.5, dw.astype(np.float64))
    if dt == "bf16":
        check(host(dH), rdH, f"saturated dH n={n} {dt}")
    else:
        e = rel_err(host(dH), rdH)
        record_margin(f"saturated dH n={n} {dt}", e, 1e-4)
        assert e <= 1e-4, f"saturated dH n={n} {dt}: {e:.3g} > 1e-4"
    grad_check(host(dW), rdW, f"saturated dW n={n} {dt}")
    grad_check(host(dws)[None], rdws[None], f"saturated dw_static n={n} {dt}")


@pytest.mark.parametrize("dt,d", [("bf16", 4096), ("f32", 1024)])
def test_weights_backward_mhc_configured_iterations_many_tokens(dt, d):
    """The weight producer's gradient in mHC mode at the configured 20
    iterations over 1024 tokens (several dW splits), logits of about unit
    scale: dH, dW and dw_static against the oracle."""
    n, T = 4, 1024
    rng = np.random.default_rng(2021)
    H, W, ws, dw = case(rng, dt, T, n, d, wsd=0.03 * (4096 / d) ** 0.5)
    dH, dW, dws = hc.weights_backward(dev(H), dev(W), dev(ws), 1.0, dev(dw), 1e-6, 20)
    rdH, rdW, rdws = oracle.weights_backward(H, W, ws.astype(np.float64), 1.0,
                                             dw.astype(np.float64), 1e-6, 20)
    check(host(dH), rdH, f"dH mhc 20 {dt}")
    grad_check(host(dW), rdW, f"dW mhc 20 {dt}")
    grad_check(host(dws)[None], rdws[None], f"dw_static mhc 20 {dt}")
