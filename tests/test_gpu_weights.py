"""GPU parity of the per-token weight kernel (MFMA projection, tanh or mHC)
and of the Sinkhorn kernel against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_RECORD, check, dev, host, need_gpu, rel_err
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import (TID_LOGITS, f32_to_bf16_bits, f32_to_fp8_bits,
                                             identity_record, make_inputs, normal_rows, workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def storage(x, dt):
    if dt == "fp8":
        return f32_to_fp8_bits(x)
    return f32_to_bf16_bits(x) if dt == "bf16" else x.astype(np.float32)


def record_check(got: np.ndarray, ref: np.ndarray, what: str):
    e = rel_err(got, ref)
    assert e <= TOL_RECORD, f"{what}: max rel err {e:.3g} > {TOL_RECORD}"
    return e


# d: one partial chunk, exact chunks, a ragged last chunk, the largest; T: partial tiles
@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 264), ("bf16", 4096), ("bf16", 6152),
                                  ("bf16", 16384), ("f32", 4), ("f32", 132), ("f32", 1024),
                                  ("f32", 16384), ("fp8", 16), ("fp8", 528), ("fp8", 4096),
                                  ("fp8", 6160), ("fp8", 16384)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 5])
def test_weights_parity(dt, d, n, iters):
    K = 2 * n + n * n
    rng = np.random.default_rng(d * 10 + n + iters)
    T = 37
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    W = storage((0.05 * rng.standard_normal((K, d))).astype(np.float32), dt)
    ws = (identity_record(n) + 0.1 * rng.standard_normal(K)).astype(np.float32)
    got = host(hc.weights(dev(H), dev(W), dev(ws), 0.5, 1e-6, iters))
    ref = oracle.weights(H, W, ws.astype(np.float64), 0.5, 1e-6, iters)
    record_check(got, ref, f"weights n={n} d={d} {dt} iters={iters}")


@pytest.mark.parametrize("T", [1, 3, 4, 5, 16, 17, 63, 64, 65])
def test_weights_ragged_tokens(T):
    n, d, K = 4, 512, 24
    rng = np.random.default_rng(T)
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), "bf16")
    W = storage((0.05 * rng.standard_normal((K, d))).astype(np.float32), "bf16")
    ws = identity_record(n)
    out = torch.full((T + 3, K), 7.0, device="cuda")   # guard rows after the output
    hc.weights(dev(H), dev(W), dev(ws), 0.01, 1e-6, 0, out=out[:T])
    got = host(out)
    record_check(got[:T], oracle.weights(H, W, ws.astype(np.float64), 0.01, 1e-6, 0), f"T={T}")
    assert np.all(got[T:] == 7.0)


@pytest.mark.parametrize("dt", ["bf16", "f32", "fp8"])
def test_zero_projection_is_static_bitwise(dt):
    n, d, K = 4, 1024, 24
    rng = np.random.default_rng(2)
    H = storage(rng.standard_normal((21, n, d)).astype(np.float32), dt)
    W = storage(np.zeros((K, d), np.float32), dt)
    ws = (identity_record(n) + 0.05 * rng.standard_normal(K)).astype(np.float32)
    got = host(hc.weights(dev(H), dev(W), dev(ws), 0.01, 1e-6, 0))
    assert np.array_equal(got, np.broadcast_to(ws, got.shape))


def test_dynamic_path_with_zero_projection_equals_static_path():
    """W = 0: per-token records equal the static one, so pre/post through the
    per-token records are bitwise the static-weight results."""
    n, d, K, T = 4, 4096, 24, 40
    rng = np.random.default_rng(4)
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), "bf16")
    F = storage(rng.standard_normal((T, d)).astype(np.float32), "bf16")
    ws = (identity_record(n) + 0.05 * rng.standard_normal(K)).astype(np.float32)
    g = np.ones(d, np.float32)
    Hd, Fd, wsd, gd = dev(H), dev(F), dev(ws), dev(g)
    w = hc.weights(Hd, dev(storage(np.zeros((K, d), np.float32), "bf16")), wsd, 0.01, 1e-6, 0)
    assert np.array_equal(host(hc.pre_mix(Hd, w, gd)), host(hc.pre_mix(Hd, wsd, gd)))
    assert np.array_equal(host(hc.post_mix(Hd, Fd, w)), host(hc.post_mix(Hd, Fd, wsd)))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 1, 20])
def test_sinkhorn_parity(n, iters):
    K = 2 * n + n * n
    rng = np.random.default_rng(n * 100 + iters)
    T = 1000
    lg = rng.standard_normal((T, K)).astype(np.float32)
    got = host(hc.sinkhorn(dev(lg), n, iters))
    ref = oracle.sinkhorn(lg.astype(np.float64), n, iters)
    record_check(got, ref, f"sinkhorn n={n} iters={iters}")


def test_sinkhorn_large_logits_stay_finite():
    """Logits far beyond exp's fp32 range: the max shift keeps A finite and
    doubly stochastic in the columns."""
    lg = np.zeros((2, 24), np.float32)
    lg[0, 8:] = np.linspace(60, 120, 16)
    lg[1, 8:] = -np.linspace(60, 120, 16)
    got = host(hc.sinkhorn(dev(lg), 4, 20))
    A = got[:, 8:].reshape(2, 4, 4)
    assert np.all(np.isfinite(A))
    np.testing.assert_allclose(A.sum(axis=1), 1.0, atol=1e-6)
    record_check(got, oracle.sinkhorn(lg.astype(np.float64), 4, 20), "large logits")


def test_mhc_workload_full():
    """T=32768 per-token logits ~ N(0,1), 20 iterations, all tokens checked:
    elementwise against the oracle, every column sum within 1e-6 of 1, and
    every row sum within 1e-6 of the oracle's own row sum (which is itself
    within 1e-6 of 1 for all but the slowest-converging ~1.5% of tokens)."""
    wl = workload("mhc-bf16")
    lg = normal_rows(wl.seed, TID_LOGITS, wl.T, (wl.K,))
    got = host(hc.sinkhorn(dev(lg), wl.n, wl.iters))
    ref = oracle.sinkhorn(lg.astype(np.float64), wl.n, wl.iters)
    record_check(got, ref, "mhc records")
    A, Ar = got[:, 8:].reshape(-1, 4, 4).astype(np.float64), ref[:, 8:].reshape(-1, 4, 4)
    assert np.abs(A.sum(axis=1) - 1).max() <= 1e-6
    assert np.abs(A.sum(axis=2) - Ar.sum(axis=2)).max() <= 1e-6
    assert np.mean(np.abs(Ar.sum(axis=2) - 1).max(axis=1) <= 1e-6) > 0.97


@pytest.mark.parametrize("name", ["dynamic-bf16", "dynamic-fp8"])
def test_dynamic_workload_full_size_sampled(name):
    """T=16384, n=4, d=4096 (bf16, or FP8 E4M3 H, W and F) with W ~ N(0,
    0.02): records checked against the oracle on 256 sampled tokens, then
    pre/post with them."""
    wl = workload(name)
    inp = make_inputs(wl)
    Hd, Fd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["gamma"])
    w = hc.weights(Hd, dev(inp["W"]), dev(inp["w_static"]), wl.scale, wl.eps, 0)
    u = hc.pre_mix(Hd, w, gd, wl.eps)
    Hp = hc.post_mix(Hd, Fd, w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(17)
    idx = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 256, replace=False)]))
    sub = make_inputs(wl, tokens=idx)
    ti = torch.from_numpy(idx).cuda()
    w_ref = oracle.weights(sub["H"], inp["W"], inp["w_static"].astype(np.float64), wl.scale, wl.eps, 0)
    w_got = host(w[ti])
    record_check(w_got, w_ref, "dynamic records")
    # pre/post on the GPU's own records (fp32 values, fed exactly to the oracle)
    w64 = w_got.astype(np.float64)
    check(host(u[ti]), oracle.pre_mix(sub["H"], w64, inp["gamma"], wl.eps), "dynamic pre")
    check(host(Hp[ti]), oracle.post_mix(sub["H"], sub["F"], w64), "dynamic post")


def test_mhc_workload_pre_post_sampled():
    """T=32768, n=4, d=4096 bf16: Sinkhorn records then pre/post, sampled."""
    wl = workload("mhc-bf16")
    inp = make_inputs(wl)
    Hd, Fd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["gamma"])
    w = hc.sinkhorn(dev(inp["logits"]), wl.n, wl.iters)
    u = hc.pre_mix(Hd, w, gd, wl.eps)
    Hp = hc.post_mix(Hd, Fd, w)
    torch.cuda.synchronize()
    rng = np.random.default_rng(19)
    idx = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 256, replace=False)]))
    sub = make_inputs(wl, tokens=idx)
    ti = torch.from_numpy(idx).cuda()
    w_ref = oracle.sinkhorn(sub["logits"].astype(np.float64), wl.n, wl.iters)
    w_got = host(w[ti])
    record_check(w_got, w_ref, "mhc records")
    w64 = w_got.astype(np.float64)
    check(host(u[ti]), oracle.pre_mix(sub["H"], w64, inp["gamma"], wl.eps), "mhc pre")
    check(host(Hp[ti]), oracle.post_mix(sub["H"], sub["F"], w64), "mhc post")


@pytest.mark.parametrize("dt,d", [("bf16", 264), ("bf16", 4096), ("f32", 132), ("fp8", 528)])
@pytest.mark.parametrize("n", [1, 3, 4])
@pytest.mark.parametrize("iters", [0, 5])
def test_weights_save_records_equal_weights(dt, d, n, iters):
    """The training forward's records are bitwise those of hc_weights; the
    saved norms are the per-stream 1/rms of H."""
    K = 2 * n + n * n
    rng = np.random.default_rng(d + 11 * n + iters)
    T = 45
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    W = storage((0.05 * rng.standard_normal((K, d))).astype(np.float32), dt)
    ws = (identity_record(n) + 0.1 * rng.standard_normal(K)).astype(np.float32)
    Hd, Wd, wsd = dev(H), dev(W), dev(ws)
    a = host(hc.weights(Hd, Wd, wsd, 0.5, 1e-6, iters))
    b, saved = hc.weights_save(Hd, Wd, wsd, 0.5, 1e-6, iters)
    assert np.array_equal(a, host(b))
    off = (T * n * K + 3) // 4 * 4
    r = host(saved)[off:off + T * n].reshape(T, n).astype(np.float64)
    Hw = oracle.widen(H)
    np.testing.assert_allclose(r, 1 / np.sqrt((Hw * Hw).mean(axis=2) + 1e-6), rtol=1e-5)


@pytest.mark.parametrize("name", ["dynamic-bf16", "dynamic-fp8"])
def test_dynamic_workload_full_size_every_token(name):
    """T=16384, n=4, d=4096: every token's record against the oracle, then
    pre and post on the GPU's records, in chunks of 2048 tokens."""
    wl = workload(name)
    inp = make_inputs(wl)
    Hd, Fd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["gamma"])
    w = hc.weights(Hd, dev(inp["W"]), dev(inp["w_static"]), wl.scale, wl.eps, 0)
    u, Hp, w = host(hc.pre_mix(Hd, w, gd, wl.eps)), host(hc.post_mix(Hd, Fd, w)), host(w)
    ws64 = inp["w_static"].astype(np.float64)
    for t0 in range(0, wl.T, 2048):
        sl = slice(t0, t0 + 2048)
        record_check(w[sl], oracle.weights(inp["H"][sl], inp["W"], ws64, wl.scale, wl.eps, 0),
                     f"records {t0}+")
        w64 = w[sl].astype(np.float64)
        check(u[sl], oracle.pre_mix(inp["H"][sl], w64, inp["gamma"], wl.eps), f"pre {t0}+")
        check(Hp[sl], oracle.post_mix(inp["H"][sl], inp["F"][sl], w64), f"post {t0}+")


def test_mhc_workload_full_size_every_token():
    """T=32768, n=4, d=4096 bf16: Sinkhorn records, then pre and post with
    them, every token against the oracle (records fed back exactly)."""
    wl = workload("mhc-bf16")
    inp = make_inputs(wl)
    Hd, Fd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["gamma"])
    w = hc.sinkhorn(dev(inp["logits"]), wl.n, wl.iters)
    u, Hp, w = host(hc.pre_mix(Hd, w, gd, wl.eps)), host(hc.post_mix(Hd, Fd, w)), host(w)
    for t0 in range(0, wl.T, 2048):
        sl = slice(t0, t0 + 2048)
        w64 = w[sl].astype(np.float64)
        check(u[sl], oracle.pre_mix(inp["H"][sl], w64, inp["gamma"], wl.eps), f"pre {t0}+")
        check(Hp[sl], oracle.post_mix(inp["H"][sl], inp["F"][sl], w64), f"post {t0}+")


@pytest.mark.parametrize("dt", ["bf16", "fp8", "f32"])
def test_weights_mhc_configured_iterations_many_tokens(dt):
    """mHC mode inside the weights kernel at the configured 20 iterations
    ("a few Sinkhorn iterations": hfviewer glossary "Hyper-connections
    (mHC)", definition) over 2048 tokens, logits of about unit scale (W ~
    N(0, 0.03^2) on rows of unit RMS): every record against the oracle, and
    every token's columns sum to 1 within 1e-6."""
    n, d, T, K = 4, 4096, 2048, 24
    rng = np.random.default_rng(2020)
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    W = storage((0.03 * rng.standard_normal((K, d))).astype(np.float32), dt)
    ws = (identity_record(n) + 0.1 * rng.standard_normal(K)).astype(np.float32)
    got = host(hc.weights(dev(H), dev(W), dev(ws), 1.0, 1e-6, 20))
    ref = oracle.weights(H, W, ws.astype(np.float64), 1.0, 1e-6, 20)
    record_check(got, ref, f"mhc 20 iterations {dt}")
    A = got[:, 2 * n:].reshape(T, n, n).astype(np.float64)
    assert np.max(np.abs(A.sum(axis=1) - 1.0)) <= 1e-6
