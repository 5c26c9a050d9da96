"""GPU parity of hc_post_weights_pre_mix: the write-back of one layer, the
next layer's per-token weights and the next layer's read-mix in one pass.

What is fixed and what is compared:
 - H' is bitwise hc_post_mix's (same operations, same order);
 - the records are hc_post_mix_weights' bitwise past alpha; alpha (formed
   by every wave from the same partials, in another order of addition) is
   within the record tolerance of the oracle's weight rule on the stored H';
 - u is within the storage tolerance of the oracle's read-mix on the stored
   H' with the stored alpha, and within one unit in the last place of
   hc_pre_mix on the same H' and records (only the RMSNorm sum is added in
   another order).
At every launch shape (one, two or four vectors per lane, ragged rows, n = 1
to 4), tanh and mHC modes, shared and per-token input records, fewer tokens
than workgroups and more, in place, chained over layers, and at the dynamic
workload's full size."""
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


def case(rng, T, n, d, dt, shared, wsd=0.05):
    K = 2 * n + n * n
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    F = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    shape = (K,) if shared else (T, K)
    w = (identity_record(n) + 0.05 * rng.standard_normal(shape)).astype(np.float32)
    W = storage((wsd * rng.standard_normal((K, d))).astype(np.float32), dt)
    ws = (identity_record(n) + 0.1 * rng.standard_normal(K)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return H, F, w, W, ws, g


def ulps(a: np.ndarray, b: np.ndarray) -> int:
    """Largest distance in units in the last place between two arrays of
    bf16 bits (uint16) or FP8 codes (uint8), both sign-magnitude."""
    sign = 0x8000 if a.dtype == np.uint16 else 0x80

    def lin(x):
        x = x.astype(np.int64)
        m = x & (sign - 1)
        return np.where(x & sign, -m, m)
    return int(np.max(np.abs(lin(a) - lin(b)))) if a.size else 0


def run_boundary(H, F, w, W, ws, g, scale, iters, n, what, in_place=False, eps=1e-6, pre_eps=1e-6):
    Hd, Fd, wd, Wd, wsd, gd = dev(H), dev(F), dev(w), dev(W), dev(ws), dev(g)
    ref_post = host(hc.post_mix(Hd, Fd, wd))
    _, ref_rec = hc.post_mix_weights(Hd, Fd, wd, Wd, wsd, scale, eps, iters)
    ref_rec = host(ref_rec)
    out = Hd if in_place else None
    Ho, wo, u = hc.post_weights_pre_mix(Hd, Fd, wd, Wd, wsd, scale, gd, eps, pre_eps, iters, out=out)
    got_h, got_w, got_u = host(Ho), host(wo), host(u)
    assert np.array_equal(got_h, ref_post), f"{what}: H' differs from hc_post_mix"
    # records: past alpha bitwise the fused write-back's; all within the
    # record tolerance of the oracle on the stored H'
    assert np.array_equal(got_w[..., n:], ref_rec[..., n:]), f"{what}: records past alpha differ"
    e_w = rel_err(got_w, oracle.weights(got_h, W, ws.astype(np.float64), scale, eps, iters))
    assert e_w <= TOL_RECORD, f"{what}: records {e_w:.3g}"
    # u: the oracle's read-mix of the stored H' with the stored alpha
    check(got_u, oracle.pre_mix(got_h, got_w.astype(np.float64), g, pre_eps), what)
    # and one ulp of hc_pre_mix on the same operands
    u_ref = host(hc.pre_mix(Ho, wo, gd, pre_eps))
    assert ulps(got_u, u_ref) <= 1, f"{what}: u more than one ulp from hc_pre_mix"
    return got_h, got_w, got_u


@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 264), ("bf16", 2048), ("bf16", 2056),
                                  ("bf16", 4096), ("fp8", 16), ("fp8", 528), ("fp8", 4096)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("iters", [0, 20])
@pytest.mark.parametrize("shared", [True, False])
def test_boundary_parity(dt, d, n, iters, shared):
    rng = np.random.default_rng(d * 100 + n * 10 + iters + shared + 7)
    H, F, w, W, ws, g = case(rng, 37, n, d, dt, shared)
    run_boundary(H, F, w, W, ws, g, 0.5, iters, n, f"{dt} d={d} n={n} iters={iters} shared={shared}")


# one token per workgroup (the drain alone), two (the first round), a grid,
# one more, several rounds of the record ring; guard rows after u and the
# records
@pytest.mark.parametrize("T", [1, 2, 3, 255, 256, 257, 769, 1000])
def test_boundary_tokens(T):
    n, d, K = 4, 4096, 24
    rng = np.random.default_rng(1000 + T)
    H, F, w, W, ws, g = case(rng, T, n, d, "bf16", False)
    Hd, Fd, wd, Wd, wsd, gd = dev(H), dev(F), dev(w), dev(W), dev(ws), dev(g)
    rec = torch.full((T + 2, K), 7.0, device="cuda")
    ub = torch.full((T + 2, d), 3.0, dtype=torch.bfloat16, device="cuda")
    Ho, _, _ = hc.post_weights_pre_mix(Hd, Fd, wd, Wd, wsd, 0.01, gd, w_out=rec[:T], u_out=ub[:T])
    got_w, got_u = host(rec), host(ub)
    assert np.all(got_w[T:] == 7.0)
    assert np.all(got_u[T:] == host(torch.full((1,), 3.0, dtype=torch.bfloat16))[0])
    got_h = host(Ho)
    assert np.array_equal(got_h, host(hc.post_mix(Hd, Fd, wd)))
    e = rel_err(got_w[:T], oracle.weights(got_h, W, ws.astype(np.float64), 0.01, 1e-6, 0))
    assert e <= TOL_RECORD
    check(got_u[:T], oracle.pre_mix(got_h, got_w[:T].astype(np.float64), g, 1e-6), f"T={T}")
    assert ulps(got_u[:T], host(hc.pre_mix(Ho, rec[:T], gd))) <= 1


@pytest.mark.parametrize("dt", ["bf16", "fp8"])
def test_boundary_in_place(dt):
    rng = np.random.default_rng(12)
    H, F, w, W, ws, g = case(rng, 300, 4, 4096 if dt == "bf16" else 2048, dt, False)
    run_boundary(H, F, w, W, ws, g, 0.3, 0, 4, f"in place {dt}", in_place=True)


def test_boundary_distinct_epsilons():
    """The weights' norm and the read-mix's RMSNorm take their own epsilon."""
    rng = np.random.default_rng(13)
    H, F, w, W, ws, g = case(rng, 64, 4, 4096, "bf16", False)
    H = f32_to_bf16_bits(0.01 * rng.standard_normal((64, 4, 4096)).astype(np.float32))
    run_boundary(H, F, w, W, ws, g, 0.5, 0, 4, "eps", eps=1e-3, pre_eps=1e-2)


def test_boundary_saved_state():
    """The kept projections and norms are hc_post_mix_weights' bitwise."""
    rng = np.random.default_rng(14)
    T, n, d = 129, 4, 4096
    H, F, w, W, ws, g = case(rng, T, n, d, "bf16", False)
    Hd, Fd, wd, Wd, wsd, gd = dev(H), dev(F), dev(w), dev(W), dev(ws), dev(g)
    _, _, sv = hc.post_mix_weights(Hd, Fd, wd, Wd, wsd, 0.01, 1e-6, 0, saved=True)
    _, _, _, sv2 = hc.post_weights_pre_mix(Hd, Fd, wd, Wd, wsd, 0.01, gd, saved=True)
    assert np.array_equal(host(sv), host(sv2))


def test_boundary_layer_chain():
    """Twelve layers chained through the fused boundary against the same
    layers run as hc_pre_mix + hc_post_mix_weights: the streams stay bitwise
    equal (the write-back reads [beta | A] only, which both form alike), the
    records past alpha too; every u is within one ulp of hc_pre_mix on its
    own operands and within the storage tolerance of the oracle's."""
    rng = np.random.default_rng(15)
    T, n, d, L = 512, 4, 4096, 12
    H, F, w, W, ws, g = case(rng, T, n, d, "bf16", False)
    Ws = [dev(storage((0.02 * rng.standard_normal((24, d))).astype(np.float32), "bf16"))
          for _ in range(L)]
    Fs = [dev(storage(rng.standard_normal((T, d)).astype(np.float32), "bf16")) for _ in range(L)]
    gd, wsd = dev(g), dev(ws)
    Ha, Hb = dev(H), dev(H)
    wa = hc.weights(Ha, Ws[0], wsd, 0.01)
    wb = wa.clone()
    ua = hc.pre_mix(Ha, wa, gd)
    for l in range(L - 1):
        if l > 0:
            # ua is the read-mix of (Ha, wa), formed by the previous boundary
            assert ulps(host(ua), host(hc.pre_mix(Ha, wa, gd))) <= 1, f"layer {l}: u"
            check(host(ua), oracle.pre_mix(host(Ha), host(wa).astype(np.float64), g, 1e-6),
                  f"layer {l}: u")
        Hb, wb = hc.post_mix_weights(Hb, Fs[l], wb, Ws[l + 1], wsd, 0.01)
        Ha, wa, ua = hc.post_weights_pre_mix(Ha, Fs[l], wa, Ws[l + 1], wsd, 0.01, gd)
        assert torch.equal(Ha.view(torch.int16), Hb.view(torch.int16)), f"layer {l}: H'"
        assert torch.equal(wa[:, n:], wb[:, n:]), f"layer {l}: records past alpha"
        assert rel_err(host(wa), host(wb).astype(np.float64)) <= TOL_RECORD, f"layer {l}: alpha"
    assert ulps(host(ua), host(hc.pre_mix(Ha, wa, gd))) <= 1


@pytest.mark.parametrize("name", ["dynamic-bf16", "dynamic-fp8"])
def test_boundary_dynamic_workload_full_size(name):
    """The dynamic workload at full size in the benchmark's launch
    configuration: H' bitwise hc_post_mix's, the records past alpha bitwise
    hc_post_mix_weights', every u within one ulp of hc_pre_mix on the same
    operands, and a sample of 1024 tokens against the oracle."""
    wl = workload(name)
    inp = make_inputs(wl)
    Hd, Fd, Wd, wsd, gd = (dev(inp["H"]), dev(inp["F"]), dev(inp["W"]), dev(inp["w_static"]),
                           dev(inp["gamma"]))
    w0 = hc.weights(Hd, Wd, wsd, wl.scale, wl.eps, 0)
    Ho, w1, u = hc.post_weights_pre_mix(Hd, Fd, w0, Wd, wsd, wl.scale, gd, wl.eps, wl.eps, 0)
    bits = (lambda t: t.view(torch.uint8)) if Ho.dtype == torch.float8_e4m3fn else (lambda t: t.view(torch.int16))
    assert torch.equal(bits(Ho), bits(hc.post_mix(Hd, Fd, w0)))
    _, w2 = hc.post_mix_weights(Hd, Fd, w0, Wd, wsd, wl.scale, wl.eps, 0)
    n = wl.n
    assert torch.equal(w1[:, n:], w2[:, n:])
    assert ulps(host(u), host(hc.pre_mix(Ho, w1, gd, wl.eps))) <= 1
    idx = np.random.default_rng(5).choice(wl.T, 1024, replace=False)
    idx.sort()
    got_h = host(Ho[torch.from_numpy(idx).cuda()])
    got_w = host(w1)[idx]
    e = rel_err(got_w, oracle.weights(got_h, inp["W"], inp["w_static"].astype(np.float64),
                                      wl.scale, wl.eps, 0))
    assert e <= TOL_RECORD
    check(host(u)[idx], oracle.pre_mix(got_h, got_w.astype(np.float64), inp["gamma"], wl.eps), name)


def test_boundary_mhc_many_tokens():
    """mHC mode at 20 iterations over 2048 tokens with logits of about unit
    scale: records and u against the oracle, columns summing to 1."""
    rng = np.random.default_rng(405)
    T, n, d = 2048, 4, 4096
    H, F, w, W, ws, g = case(rng, T, n, d, "bf16", False, wsd=0.03)
    _, got_w, _ = run_boundary(H, F, w, W, ws, g, 1.0, 20, n, "mhc 2048 tokens")
    A = got_w[:, 2 * n:].reshape(T, n, n).astype(np.float64)
    assert np.max(np.abs(A.sum(axis=1) - 1.0)) <= 1e-6


def test_boundary_rejects():
    rng = np.random.default_rng(2)
    H, F, w, W, ws, g = case(rng, 4, 4, 4104, "bf16", True)
    with pytest.raises(hc.HCError) as e:
        hc.post_weights_pre_mix(dev(H), dev(F), dev(w), dev(W), dev(ws), 0.01, dev(g))
    assert e.value.status == 2          # HC_ERR_SHAPE: W would not fit the registers
