"""GPU parity of the streaming kernels (pre, post, fused post+pre, tanh block)
against the fp64 oracle, through the C ABI.

Cases span every launch shape of the row kernels (blocks of 64..1024 threads
with 1, 2, 3 and 4 vectors per thread), ragged rows (d not a multiple of the
block's vector count), small odd T, the three storage dtypes (fp32, bf16, FP8
E4M3), n = 1..4, shared and per-token weight records."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, need_gpu, rel_err, rounded
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import (f32_to_bf16_bits, f32_to_fp8_bits, identity_record,
                                             make_inputs, workload)

pytestmark = pytest.mark.gpu

# d values per dtype: covers every (block, vectors-per-thread) launch shape
D_BF16 = [8, 40, 520, 2048, 4096, 6144, 8192, 8200, 16384]
D_F32 = [4, 36, 516, 1024, 3072, 4096, 4100, 8196, 12288, 12296, 16384]
D_FP8 = [16, 48, 1040, 4096, 8192, 8208, 12288, 16384]
SHAPES = ([("bf16", d) for d in D_BF16] + [("f32", d) for d in D_F32] +
          [("fp8", d) for d in D_FP8])


def storage(x: np.ndarray, dt: str) -> np.ndarray:
    if dt == "fp8":
        return f32_to_fp8_bits(x)
    return f32_to_bf16_bits(x) if dt == "bf16" else x.astype(np.float32)


def case(rng, dt, T, n, d, per_token):
    K = 2 * n + n * n
    H = storage(rng.standard_normal((T, n, d)).astype(np.float32), dt)
    F = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    if per_token:
        w = (identity_record(n)[None, :] + 0.3 * rng.standard_normal((T, K))).astype(np.float32)
    else:
        w = (identity_record(n) + 0.3 * rng.standard_normal(K)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    return H, F, w, g


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("dt,d", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_pre_parity(dt, d, n):
    rng = np.random.default_rng(1000 * n + d)
    T = 3 if d >= 8192 else 7
    H, F, w, g = case(rng, dt, T, n, d, per_token=(d % 3 == 0))
    u = host(hc.pre_mix(dev(H), dev(w), dev(g), 1e-6))
    ref = oracle.pre_mix(H, w.astype(np.float64), g, 1e-6)
    check(u, ref, f"pre n={n} d={d} {dt}")


@pytest.mark.parametrize("dt,d", SHAPES)
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_post_parity(dt, d, n):
    rng = np.random.default_rng(2000 * n + d)
    T = 3 if d >= 8192 else 7
    H, F, w, g = case(rng, dt, T, n, d, per_token=(d % 3 != 0))
    out = host(hc.post_mix(dev(H), dev(F), dev(w)))
    ref = oracle.post_mix(H, F, w.astype(np.float64))
    check(out, ref, f"post n={n} d={d} {dt}")


@pytest.mark.parametrize("dt", ["bf16", "f32", "fp8"])
@pytest.mark.parametrize("n", [1, 4])
def test_post_in_place(dt, n):
    rng = np.random.default_rng(7)
    H, F, w, g = case(rng, dt, 33, n, 4096, per_token=True)
    Hd = dev(H)
    ptr = Hd.data_ptr()
    hc.post_mix(Hd, dev(F), dev(w), out=Hd)
    assert Hd.data_ptr() == ptr
    check(host(Hd), oracle.post_mix(H, F, w.astype(np.float64)), "post in place")


@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 4096), ("bf16", 6144), ("bf16", 16384),
                                  ("f32", 1024), ("f32", 16384), ("fp8", 16), ("fp8", 4096),
                                  ("fp8", 8208)])
@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_identity_post_is_plain_residual_bitwise(dt, d, n):
    """alpha = e_0, beta = 1, A = I on n copies of x: every stream is the
    stored x + F, bitwise, and equals the oracle's rounded value bitwise."""
    rng = np.random.default_rng(d + n)
    T = 9
    x = storage(rng.standard_normal((T, 1, d)).astype(np.float32), dt)
    F = storage(rng.standard_normal((T, d)).astype(np.float32), dt)
    H = np.repeat(x, n, axis=1)
    out = host(hc.post_mix(dev(H), dev(F), dev(identity_record(n))))
    plain = rounded(oracle.widen(x)[:, 0, :] + oracle.widen(F), out)
    for i in range(n):
        assert np.array_equal(out[:, i, :], plain)
    # the n = 1 layer is the ordinary residual (x + f(x)) stored once
    one = host(hc.post_mix(dev(x), dev(F), dev(identity_record(1))))
    assert np.array_equal(one[:, 0, :], plain)


@pytest.mark.parametrize("dt,d", [("bf16", 8), ("bf16", 4096), ("bf16", 6144), ("bf16", 16384),
                                  ("f32", 1024), ("f32", 4100), ("fp8", 48), ("fp8", 16384)])
@pytest.mark.parametrize("n", [2, 3, 4])
def test_identity_pre_bitwise_equals_single_stream(dt, d, n):
    """alpha = e_0: u is bitwise the n = 1 call on stream 0 (the reduction
    order over d does not depend on n), up to the sign of zero: a -0 in
    stream 0 plus 0 * (a positive value) of another stream is +0 (FP8 draws
    round small values to -0)."""
    rng = np.random.default_rng(d * n)
    H, F, w, g = case(rng, dt, 11, n, d, per_token=False)
    u_n = host(hc.pre_mix(dev(H), dev(identity_record(n)), dev(g)))
    u_1 = host(hc.pre_mix(dev(np.ascontiguousarray(H[:, :1, :])), dev(identity_record(1)), dev(g)))
    zn, z1 = oracle.widen(u_n) == 0, oracle.widen(u_1) == 0
    assert np.array_equal(zn, z1)
    assert np.array_equal(u_n[~zn], u_1[~z1])


@pytest.mark.parametrize("dt,d", [("bf16", 40), ("bf16", 4096), ("bf16", 6144), ("bf16", 8200),
                                  ("bf16", 16384), ("f32", 516), ("f32", 8196), ("f32", 12288),
                                  ("f32", 16384), ("fp8", 48), ("fp8", 4096), ("fp8", 8208)])
@pytest.mark.parametrize("n", [1, 3, 4])
def test_fused_post_pre_bitwise(dt, d, n):
    rng = np.random.default_rng(31 * d + n)
    T = 13
    H, F, w, g = case(rng, dt, T, n, d, per_token=True)
    w2 = (identity_record(n) + 0.3 * rng.standard_normal(2 * n + n * n)).astype(np.float32)
    Hd, Fd, wd, w2d, gd = dev(H), dev(F), dev(w), dev(w2), dev(g)
    Hp, u = hc.post_pre_mix(Hd, Fd, wd, w2d, gd, 1e-6)
    Hp_ref = hc.post_mix(Hd, Fd, wd)
    u_ref = hc.pre_mix(Hp_ref, w2d, gd, 1e-6)
    assert np.array_equal(host(Hp), host(Hp_ref))
    assert np.array_equal(host(u), host(u_ref))
    # and against the oracle, fed the stored H'
    check(host(u), oracle.pre_mix(host(Hp), w2.astype(np.float64), g, 1e-6), "fused u")
    # in place
    Hd2 = dev(H)
    hc.post_pre_mix(Hd2, Fd, wd, w2d, gd, 1e-6, out=Hd2)
    assert np.array_equal(host(Hd2), host(Hp_ref))


def test_deterministic():
    rng = np.random.default_rng(5)
    H, F, w, g = case(rng, "bf16", 257, 4, 4096, per_token=True)
    Hd, Fd, wd, gd = dev(H), dev(F), dev(w), dev(g)
    a = [host(hc.pre_mix(Hd, wd, gd)) for _ in range(3)]
    b = [host(hc.post_mix(Hd, Fd, wd)) for _ in range(3)]
    assert all(np.array_equal(a[0], x) for x in a[1:])
    assert all(np.array_equal(b[0], x) for x in b[1:])


def test_nan_and_inf_propagate_like_the_oracle():
    rng = np.random.default_rng(9)
    H, F, w, g = case(rng, "bf16", 6, 4, 64, per_token=False)
    Hn = oracle.widen(H)
    Hn[1, 2, 5] = np.nan
    Hn[3, 0, 7] = np.inf
    H2 = oracle.round_bf16(Hn)
    Fn = oracle.widen(F)
    Fn[4, 9] = -np.inf
    F2 = oracle.round_bf16(Fn)
    wd = w.astype(np.float64)
    check(host(hc.pre_mix(dev(H2), dev(w), dev(g))), oracle.pre_mix(H2, wd, g), "pre nan")
    check(host(hc.post_mix(dev(H2), dev(F2), dev(w))), oracle.post_mix(H2, F2, wd), "post nan")


def test_zero_tokens_is_a_noop():
    e = torch.empty((0, 4, 4096), dtype=torch.bfloat16, device="cuda")
    u = hc.pre_mix(e, dev(identity_record(4)), torch.ones(4096, device="cuda"))
    assert u.shape == (0, 4096)
    o = hc.post_mix(e, torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda"),
                    dev(identity_record(4)))
    assert o.shape == (0, 4, 4096)


@pytest.mark.parametrize("dt", ["bf16", "f32", "fp8"])
def test_block_tanh(dt):
    rng = np.random.default_rng(3)
    u = storage(3 * rng.standard_normal((17, 1024)).astype(np.float32), dt)
    F = host(hc.block_tanh(dev(u)))
    check(F, oracle.block_tanh(u), "tanh")


def test_tiny_f32_workload():
    """T=256, n=4, d=1024 fp32, identity + N(0, 0.02) weights; F is the host
    tanh of the oracle's block input, fed to both post paths."""
    wl = workload("tiny-f32")
    inp = make_inputs(wl)
    H, w, g = inp["H"], inp["w"], inp["gamma"]
    Hd, wd = dev(H), dev(w)
    u = host(hc.pre_mix(Hd, wd, dev(g), wl.eps))
    u_ref = oracle.pre_mix(H, w.astype(np.float64), g, wl.eps)
    check(u, u_ref, "tiny pre")
    F = oracle.round_f32(np.tanh(u_ref))
    out = host(hc.post_mix(Hd, dev(F), wd))
    check(out, oracle.post_mix(H, F, w.astype(np.float64)), "tiny post")
    # unperturbed identity run: the ordinary residual, bitwise
    out_id = host(hc.post_mix(dev(np.repeat(H[:, :1], 4, axis=1)), dev(F), dev(identity_record(4))))
    assert np.array_equal(out_id[:, 3, :], oracle.round_f32(oracle.widen(H[:, 0, :]) + F))


def sample_tokens(T: int, k: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, size=k, replace=False)]))


def test_static_bf16_full_size_sampled():
    """T=8192, n=4, d=4096 bf16, in the launch configuration the benchmark
    times; 256 sampled tokens (plus the first and last) checked by the oracle."""
    wl = workload("static-bf16")
    inp = make_inputs(wl)
    Hd, Fd, wd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["w"]), dev(inp["gamma"])
    u = hc.pre_mix(Hd, wd, gd, wl.eps)
    Hp = hc.post_mix(Hd, Fd, wd)
    torch.cuda.synchronize()
    idx = sample_tokens(wl.T, 256, 11)
    sub = make_inputs(wl, tokens=idx)
    assert np.array_equal(sub["H"], inp["H"][idx])
    w64 = inp["w"].astype(np.float64)
    check(host(u[torch.from_numpy(idx).cuda()]), oracle.pre_mix(sub["H"], w64, inp["gamma"], wl.eps),
          "static pre")
    check(host(Hp[torch.from_numpy(idx).cuda()]), oracle.post_mix(sub["H"], sub["F"], w64),
          "static post")


@pytest.mark.parametrize("name", ["static-bf16", "static-fp8"])
def test_static_full_size_every_token(name):
    """The static workloads (T=8192 bf16, the headline, and T=16384 FP8; n=4,
    d=4096) in the benchmark's launch configuration: every token of u and H',
    and of the fused post+pre (its H' bitwise post's, its u against the oracle
    on that H'), in chunks of 1024 tokens."""
    wl = workload(name)
    inp = make_inputs(wl)
    Hd, Fd, wd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["w"]), dev(inp["gamma"])
    u, Hp = host(hc.pre_mix(Hd, wd, gd, wl.eps)), host(hc.post_mix(Hd, Fd, wd))
    Hp2, u2 = hc.post_pre_mix(Hd, Fd, wd, wd, gd, wl.eps)
    Hp2, u2 = host(Hp2), host(u2)
    assert np.array_equal(Hp2, Hp)               # the fused write-back is the same store
    w64 = inp["w"].astype(np.float64)
    for t0 in range(0, wl.T, 1024):
        sl = slice(t0, t0 + 1024)
        check(u[sl], oracle.pre_mix(inp["H"][sl], w64, inp["gamma"], wl.eps), f"pre tokens {t0}+")
        check(Hp[sl], oracle.post_mix(inp["H"][sl], inp["F"][sl], w64), f"post tokens {t0}+")
        check(u2[sl], oracle.pre_mix(Hp[sl], w64, inp["gamma"], wl.eps), f"fused pre {t0}+")


def _fp8_finite_codes() -> np.ndarray:
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]


def test_fp8_store_rounding_exhaustive():
    """Every sum of two finite FP8 values, stored by the identity post with
    n = 1 (H' = H + F, exact in fp32): the stored code is the oracle's
    nearest-even saturating rounding, bitwise.  Covers ties, the subnormal
    range, carries into the next binade and overflow past 448."""
    codes = _fp8_finite_codes()                      # 254 codes
    d = 256
    x = np.zeros(d, np.uint8)
    x[:codes.size] = codes
    H = np.repeat(x[None, None, :], codes.size, axis=0)              # (254, 1, 256)
    F = np.repeat(codes[:, None], d, axis=1).astype(np.uint8)        # token t adds code t
    out = host(hc.post_mix(dev(H), dev(F), dev(identity_record(1))))
    want = oracle.round_fp8(oracle.widen(H)[:, 0, :] + oracle.widen(F))
    assert np.array_equal(out[:, 0, :], want)
    assert (want == 0x7E).any() and (want == 0x01).any()             # saturation and subnormals hit


def test_fp8_nan_propagates_and_large_values_saturate():
    rng = np.random.default_rng(19)
    n, d, T = 4, 64, 5
    H = f32_to_fp8_bits(rng.standard_normal((T, n, d)).astype(np.float32) * 100)
    F = f32_to_fp8_bits(rng.standard_normal((T, d)).astype(np.float32) * 300)
    H[1, 2, 5] = 0x7F                                                   # NaN
    H[2, :, :8] = 0x7E                                                  # 448 in every stream
    w = (identity_record(n) + 0.3 * rng.standard_normal(2 * n + n * n)).astype(np.float32)
    w[n:2 * n] = 2.0                                                    # beta = 2 pushes past 448
    g = np.ones(d, np.float32)
    wd = w.astype(np.float64)
    out = host(hc.post_mix(dev(H), dev(F), dev(w)))
    ref = oracle.post_mix(H, F, wd)
    check(out, ref, "post fp8 nan/sat")
    assert (np.abs(ref) > 448).any() and ((out & 0x7F) == 0x7E).any()
    assert np.array_equal(np.isnan(oracle.widen(out)), np.isnan(ref))
    check(host(hc.pre_mix(dev(H), dev(w), dev(g))), oracle.pre_mix(H, wd, g), "pre fp8 nan")


def test_static_fp8_full_size_sampled():
    """T=16384, n=4, d=4096 FP8 E4M3, in the launch configuration the
    benchmark times; 256 sampled tokens (plus the first and last) checked by
    the oracle."""
    wl = workload("static-fp8")
    inp = make_inputs(wl)
    Hd, Fd, wd, gd = dev(inp["H"]), dev(inp["F"]), dev(inp["w"]), dev(inp["gamma"])
    u = hc.pre_mix(Hd, wd, gd, wl.eps)
    Hp = hc.post_mix(Hd, Fd, wd)
    Hp2, u2 = hc.post_pre_mix(Hd, Fd, wd, wd, gd, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(Hp2.view(torch.uint8), Hp.view(torch.uint8))
    idx = sample_tokens(wl.T, 256, 13)
    sub = make_inputs(wl, tokens=idx)
    assert np.array_equal(sub["H"], inp["H"][idx])
    w64 = inp["w"].astype(np.float64)
    ti = torch.from_numpy(idx).cuda()
    check(host(u[ti]), oracle.pre_mix(sub["H"], w64, inp["gamma"], wl.eps), "static fp8 pre")
    check(host(Hp[ti]), oracle.post_mix(sub["H"], sub["F"], w64), "static fp8 post")
    check(host(u2[ti]), oracle.pre_mix(host(Hp[ti]), w64, inp["gamma"], wl.eps), "static fp8 fused u")


@pytest.mark.parametrize("dt", ["bf16", "f32", "fp8"])
def test_degenerate_weights_give_exact_results(dt):
    """Zero read weights give u = 0 exactly (x = 0, r = 1/sqrt(eps)); zero
    write weights give H' = A H with no trace of F (bitwise the same with F =
    0); A = 0, beta = 0 gives zeros; a zero stream state gives u = 0."""
    n, d, T = 4, 4096, 5
    rng = np.random.default_rng(23)
    H, F, w, g = case(rng, dt, T, n, d, per_token=False)
    z = w.copy()
    z[:n] = 0.0                                           # alpha = 0
    u = host(hc.pre_mix(dev(H), dev(z), dev(g)))
    assert not oracle.widen(u).any()
    u0 = host(hc.pre_mix(dev(np.zeros_like(H)), dev(w), dev(g)))
    assert not oracle.widen(u0).any()
    nb = w.copy()
    nb[n:2 * n] = 0.0                                     # beta = 0: F has no effect
    a = host(hc.post_mix(dev(H), dev(F), dev(nb)))
    b = host(hc.post_mix(dev(H), dev(np.zeros_like(F)), dev(nb)))
    assert np.array_equal(a, b)
    check(a, oracle.post_mix(H, F, nb.astype(np.float64)), "beta = 0")
    zz = np.zeros_like(w)
    o = host(hc.post_mix(dev(H), dev(F), dev(zz)))
    assert not oracle.widen(o).any()
