"""GPU parity of hc_post_mix_weights: the write-back fused with the next
layer's per-token weights.  Its H' must be bitwise hc_post_mix's (the same
operations in the same order), and its records must match the oracle's
weight rule applied to that stored H' within the record tolerance, in tanh
and mHC modes, at every launch shape (one or two vectors per lane, ragged
rows, fewer tokens than workgroups, more), shared and per-token input
records, in place, and at the dynamic workload's full size."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_RECORD, check, dev, host, need_gpu, rel_err
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import (f32_to_bf16_bits, f32_to_fp8_bits, identity_record,
                                             make_inputs, workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def storage(x, dt):
    return f32_to_fp8_bits(x) if dt == "fp8" else f32_to_bf16_bits(x)


def record_check(got, ref, what):
    e = rel_err(got, ref)
    assert e <= TOL_RECORD, f"{what}: max rel err {e:.3g} > {TOL_RECORD}"
    return e


def case(rng, T, n, d, dt, shared, wsd=0.05):
    K = 2 * n + n * n
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    F = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    shape = (K,) if shared else (T, K)
    w = (identity_record(n) + 0.05 * rng.standard_normal(shape)).astype(np.float32)
    W = storage((wsd * rng.standard_normal((K, d))).astype(np.float32), dt)
    ws = (identity_record(n) + 0.1 * rng.standard_normal(K)).astype(np.float32)
    return H, F, w, W, ws


def run_and_check(H, F, w, W, ws, scale, iters, what, in_place=False):
    Hd, Fd, wd, Wd, wsd = dev(H), dev(F), dev(w), dev(W), dev(ws)
    ref_post = hc.post_mix(Hd, Fd, wd)
    out = Hd if in_place else None
    Ho, wo = hc.post_mix_weights(Hd, Fd, wd, Wd, wsd, scale, 1e-6, iters, out=out)
    got_h, got_w = host(Ho), host(wo)
    assert np.array_equal(got_h, host(ref_post)), f"{what}: H' differs from hc_post_mix"
    check(got_h, oracle.post_mix(H, F, w.astype(np.float64)), what)
    ref_w = oracle.weights(got_h, W, ws.astype(np.float64), scale, 1e-6, iters)
    return record_check(got_w, ref_w, what)


# d: one vector per lane (8, ragged 264, full 2048), two per lane (ragged 2056,
# full 4096); FP8 one vector per lane
@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 264), ("bf16", 2048), ("bf16", 2056),
                                  ("bf16", 4096), ("fp8", 16), ("fp8", 528), ("fp8", 4096)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 20])
@pytest.mark.parametrize("shared", [True, False])
def test_post_weights_parity(dt, d, n, iters, shared):
    rng = np.random.default_rng(d * 100 + n * 10 + iters + shared)
    H, F, w, W, ws = case(rng, 37, n, d, dt, shared)
    run_and_check(H, F, w, W, ws, 0.5, iters, f"{dt} d={d} n={n} iters={iters} shared={shared}")


# fewer tokens than workgroups, exactly a grid, one more, several rounds of
# the prefetch ring; a guard row after the records
@pytest.mark.parametrize("T", [1, 2, 3, 255, 256, 257, 769, 1000])
def test_post_weights_tokens(T):
    n, d, K = 4, 4096, 24
    rng = np.random.default_rng(T)
    H, F, w, W, ws = case(rng, T, n, d, "bf16", False)
    Hd, Fd, wd, Wd, wsd = dev(H), dev(F), dev(w), dev(W), dev(ws)
    rec = torch.full((T + 2, K), 7.0, device="cuda")
    Ho, _ = hc.post_mix_weights(Hd, Fd, wd, Wd, wsd, 0.01, 1e-6, 0, w_out=rec[:T])
    got = host(rec)
    assert np.all(got[T:] == 7.0)
    assert np.array_equal(host(Ho), host(hc.post_mix(Hd, Fd, wd)))
    record_check(got[:T], oracle.weights(host(Ho), W, ws.astype(np.float64), 0.01, 1e-6, 0), f"T={T}")


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_post_weights_in_place(dt):
    rng = np.random.default_rng(11)
    H, F, w, W, ws = case(rng, 300, 4, 4096 if dt == "bf16" else 2048, dt, False)
    run_and_check(H, F, w, W, ws, 0.3, 0, f"in place {dt}", in_place=True)


def test_post_weights_zero_projection_is_static_bitwise():
    """W = 0: tanh(0) = 0, so every record is w_static bitwise."""
    rng = np.random.default_rng(5)
    H, F, w, W, ws = case(rng, 70, 4, 4096, "bf16", True)
    W = np.zeros_like(W)
    _, wo = hc.post_mix_weights(dev(H), dev(F), dev(w), dev(W), dev(ws), 0.01, 1e-6, 0)
    got = host(wo)
    assert np.array_equal(got, np.broadcast_to(ws, got.shape))


@pytest.mark.parametrize("iters", [0, 20])
def test_post_weights_saved_state(iters):
    """The kept projections and norms are hc_weights_save's on the same H'
    (to fp32 rounding), so the backward can take either."""
    rng = np.random.default_rng(17 + iters)
    T, n, d = 129, 4, 4096
    H, F, w, W, ws = case(rng, T, n, d, "bf16", False)
    Hd, Fd, wd, Wd, wsd = dev(H), dev(F), dev(w), dev(W), dev(ws)
    Ho, wo, sv = hc.post_mix_weights(Hd, Fd, wd, Wd, wsd, 0.01, 1e-6, iters, saved=True)
    w2, sv2 = hc.weights_save(Ho, Wd, wsd, 0.01, 1e-6, iters)
    K = 24
    P, P2 = host(sv)[:T * n * K].reshape(T * n, K), host(sv2)[:T * n * K].reshape(T * n, K)
    ro = int(np.ceil(T * n * K / 4) * 4)
    r, r2 = host(sv)[ro:ro + T * n], host(sv2)[ro:ro + T * n]
    assert rel_err(P, P2.astype(np.float64)) <= TOL_RECORD
    # r = 1/sqrt(mean H'^2 + eps): the two kernels sum the squares in another
    # order, which moves r by a few fp32 ulps (half the sum's relative error)
    assert np.max(np.abs(r / r2 - 1)) <= TOL_RECORD
    record_check(host(wo), host(w2).astype(np.float64), "records vs hc_weights_save")


@pytest.mark.parametrize("name", ["dynamic-bf16", "dynamic-fp8"])
def test_post_weights_dynamic_workload_full_size(name):
    """The dynamic workload at full size in the benchmark's launch
    configuration: the first layer's records from hc_weights, then the fused
    write-back; every token's H' is bitwise hc_post_mix's and every record
    matches the oracle on the stored H'."""
    wl = workload(name)
    inp = make_inputs(wl)
    Hd, Fd, Wd, wsd = dev(inp["H"]), dev(inp["F"]), dev(inp["W"]), dev(inp["w_static"])
    w0 = hc.weights(Hd, Wd, wsd, wl.scale, wl.eps, 0)
    Ho, w1 = hc.post_mix_weights(Hd, Fd, w0, Wd, wsd, wl.scale, wl.eps, 0)
    ref_h = hc.post_mix(Hd, Fd, w0)
    assert torch.equal(Ho.view(torch.uint8) if Ho.dtype == torch.float8_e4m3fn else Ho.view(torch.int16),
                       ref_h.view(torch.uint8) if ref_h.dtype == torch.float8_e4m3fn else ref_h.view(torch.int16))
    got_w = host(w1)
    del ref_h
    for c0 in range(0, wl.T, 2048):
        sl = slice(c0, c0 + 2048)
        Hc = host(Ho[sl])
        record_check(got_w[sl], oracle.weights(Hc, inp["W"], inp["w_static"].astype(np.float64),
                                               wl.scale, wl.eps, 0), f"{name} tokens {c0}..")


def test_post_weights_mhc_many_tokens():
    """mHC mode at the configured 20 iterations over 2048 tokens, with
    logits of about unit scale (W ~ N(0, 0.03^2) on rows of unit RMS, so
    z = W hbar has a standard deviation near 1): records against the oracle,
    and every token's columns sum to 1."""
    rng = np.random.default_rng(404)
    T, n, d = 2048, 4, 4096
    H, F, w, W, ws = case(rng, T, n, d, "bf16", False, wsd=0.03)
    e = run_and_check(H, F, w, W, ws, 1.0, 20, "mhc 2048 tokens")
    assert e <= TOL_RECORD
    Ho, wo = hc.post_mix_weights(dev(H), dev(F), dev(w), dev(W), dev(ws), 1.0, 1e-6, 20)
    A = host(wo)[:, 2 * n:].reshape(T, n, n).astype(np.float64)
    assert np.max(np.abs(A.sum(axis=1) - 1.0)) <= 1e-6


def test_post_weights_rejects():
    rng = np.random.default_rng(1)
    H, F, w, W, ws = case(rng, 4, 4, 4104, "bf16", True)
    with pytest.raises(hc.HCError) as e:
        hc.post_mix_weights(dev(H), dev(F), dev(w), dev(W), dev(ws), 0.01)
    assert e.value.status == 2          # HC_ERR_SHAPE: W would not fit the registers
    Hf = torch.zeros((4, 4, 256), device="cuda")
    with pytest.raises(hc.HCError) as e:
        hc.post_mix_weights(Hf, torch.zeros((4, 256), device="cuda"), torch.zeros(24, device="cuda"),
                            torch.zeros((24, 256), device="cuda"), torch.zeros(24, device="cuda"), 0.01)
    assert e.value.status == 3          # HC_ERR_DTYPE: fp32 storage
