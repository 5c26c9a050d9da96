"""The C ABI: the built library loads and exports every function include/hc.h
declares, and argument validation rejects bad calls before anything is
launched (these calls never reach the GPU, so they run on any host)."""
import ctypes
import os
import re
import subprocess

import pytest

from hyper_connections_amd import hc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hc.h")

OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, ARG = 0, 1, 2, 3, 4, 5, 6
BF16, F32, FP8 = hc.HC_BF16, hc.HC_F32, hc.HC_FP8

# fake, never dereferenced device addresses (16-byte aligned, far apart)
P = [0x10000000 * (i + 1) for i in range(14)]
MiB = 1 << 20


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(hc.LIB_PATH):
        from hyper_connections_amd import build
        build.build()
    return hc.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hc_status|const char\*|int32_t|int64_t)\s+(hc_\w+)\s*\(",
                                 text, re.M)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(hc.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", hc.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(hc_\w+)$", out, re.M))
    for n in names:
        assert n in exported, n
        assert getattr(L, n) is not None


def test_status_strings(L):
    for code in range(8):
        s = hc.status_str(code)
        assert s.startswith("HC_")
    assert hc.status_str(99).startswith("HC_ERR_UNKNOWN")
    assert hc.abi_version() == 8


def pre(L, H=P[0], w=P[1], ws=0, g=P[2], eps=1e-6, u=P[3], T=16, n=4, d=4096, dt=BF16):
    return L.hc_pre_mix(H, w, ws, g, eps, u, T, n, d, dt, None)


def post(L, H=P[0], F=P[1], w=P[2], ws=0, O=P[3], T=16, n=4, d=4096, dt=BF16):
    return L.hc_post_mix(H, F, w, ws, O, T, n, d, dt, None)


def test_pre_validation(L):
    assert pre(L, T=0) == OK                       # empty: no-op, nothing launched
    assert pre(L, T=0, H=None, u=None) == OK       # empty tensors have no storage
    assert pre(L, T=0, eps=0.0) == ARG and pre(L, T=0, ws=3) == SHAPE
    assert pre(L, H=None) == NULL and pre(L, u=None) == NULL and pre(L, g=None) == NULL
    assert pre(L, n=0) == SHAPE and pre(L, n=5) == SHAPE
    assert pre(L, d=4092) == SHAPE                 # bf16 needs d % 8 == 0
    assert pre(L, d=4092, dt=F32, T=0) == OK       # fp32 needs d % 4 == 0
    assert pre(L, d=0) == SHAPE and pre(L, d=hc.MAX_HIDDEN + 8) == SHAPE
    assert pre(L, dt=3) == DTYPE
    assert pre(L, dt=FP8, T=0) == OK
    assert pre(L, dt=FP8, d=4088) == SHAPE and pre(L, dt=FP8, d=4088, T=0) == SHAPE   # d % 16
    assert pre(L, dt=FP8, u=P[3] + 8) == ALIGN
    assert pre(L, dt=FP8, u=P[0] + 16 * 4096) == ALIAS   # u inside the fp8 H (16 x 4 x 4096 B)
    assert pre(L, T=-1) == ARG
    assert pre(L, eps=0.0) == ARG and pre(L, eps=-1.0) == ARG and pre(L, eps=float("inf")) == ARG
    assert pre(L, ws=5) == SHAPE                   # stride must be 0 or >= K = 24
    assert pre(L, H=P[0] + 8) == ALIGN and pre(L, u=P[3] + 4) == ALIGN
    assert pre(L, g=P[2] + 4) == ALIGN and pre(L, w=P[1] + 2) == ALIGN
    assert pre(L, u=P[0] + 16 * 4096) == ALIAS     # u inside H
    assert pre(L, u=P[1] - 64) == ALIAS            # u runs into w


def test_post_validation(L):
    assert post(L, T=0) == OK
    assert post(L, F=None) == NULL and post(L, O=None) == NULL
    assert post(L, n=7) == SHAPE and post(L, d=12) == SHAPE
    assert post(L, T=-3) == ARG and post(L, dt=9) == DTYPE
    assert post(L, O=P[3] + 8) == ALIGN
    assert post(L, O=P[0] + 16) == ALIAS           # partial overlap with H
    assert post(L, O=P[1]) == ALIAS                # H_out on F
    assert post(L, O=P[2] - 16) == ALIAS           # H_out runs into w
    assert post(L, T=0, O=P[0]) == OK              # exact in-place is allowed
    assert post(L, ws=23) == SHAPE


def test_fused_validation(L):
    f = lambda **k: L.hc_post_pre_mix(  # noqa: E731
        k.get("H", P[0]), k.get("F", P[1]), k.get("w", P[2]), k.get("ws", 0), k.get("w2", P[3]),
        k.get("ws2", 0), k.get("g", P[4]), k.get("eps", 1e-6), k.get("O", P[5]), k.get("u", P[6]),
        k.get("T", 4), 4, 4096, BF16, None)
    assert f(T=0) == OK
    assert f(w2=None) == NULL and f(u=None) == NULL
    assert f(ws2=3) == SHAPE and f(eps=0.0) == ARG
    assert f(u=P[5]) == ALIAS                      # u_next on H_out
    assert f(u=P[0]) == ALIAS                      # u_next on H
    assert f(O=P[0], T=0) == OK


def test_weights_validation(L):
    f = lambda **k: L.hc_weights(  # noqa: E731
        k.get("H", P[0]), k.get("W", P[1]), k.get("ws", P[2]), k.get("scale", 0.01),
        k.get("eps", 1e-6), k.get("it", 0), k.get("o", P[3]), k.get("T", 64), k.get("n", 4),
        k.get("d", 4096), k.get("dt", BF16), None)
    assert f(T=0) == OK
    assert f(W=None) == NULL
    assert f(it=-1) == ARG and f(it=hc.MAX_SINKHORN_ITERS + 1) == ARG
    assert f(scale=float("nan")) == ARG and f(eps=0.0) == ARG
    assert f(W=P[1] + 8) == ALIGN and f(o=P[3] + 2) == ALIGN
    assert f(o=P[0] + 64) == ALIAS and f(o=P[1]) == ALIAS
    assert f(n=0) == SHAPE and f(d=100) == SHAPE and f(dt=5) == DTYPE
    assert f(dt=FP8, T=0) == OK and f(dt=FP8, d=4104) == SHAPE   # fp8 needs d % 16 == 0


def test_backward_validation(L):
    ws_need = L.hc_backward_workspace(8, 4, 4096)
    assert ws_need > 0 and L.hc_backward_workspace(0, 4, 4096) == 0
    assert L.hc_backward_workspace(8, 5, 4096) == 0
    pb = lambda **k: L.hc_post_mix_backward(  # noqa: E731
        k.get("g", P[0]), k.get("H", P[1]), k.get("F", P[2]), k.get("w", P[3]), k.get("ws", 0),
        k.get("dH", P[4]), k.get("dF", P[5]), k.get("dw", P[6]), k.get("wk", P[7]),
        k.get("wkb", ws_need), k.get("T", 8), 4, 4096, k.get("dt", BF16), None)
    assert pb(dt=FP8) == DTYPE and pb(dt=FP8, T=0) == DTYPE
    assert pb(T=0) == OK and pb(T=0, dH=None) == OK
    assert pb(dF=None) == NULL and pb(ws=2) == SHAPE and pb(dH=P[4] + 8) == ALIGN
    # dH may be NULL (the pre gradient then forms it); the rest is still checked
    assert pb(dH=None, dF=None) == NULL and pb(dH=None, dF=P[0] + 16) == ALIAS
    assert pb(wk=None) == NULL and pb(wkb=ws_need - 1) == ARG and pb(wk=P[7] + 4) == ALIGN
    assert pb(dH=P[1]) == ALIAS and pb(dw=P[4] + 64) == ALIAS and pb(dF=P[0] + 16) == ALIAS
    assert pb(wk=P[6]) == ALIAS
    qb = lambda **k: L.hc_pre_mix_backward(  # noqa: E731
        k.get("du", P[0]), k.get("H", P[1]), k.get("w", P[2]), k.get("ws", 0), k.get("g", P[3]),
        k.get("eps", 1e-6), k.get("din", None), k.get("dout", None), k.get("dH", P[4]), k.get("dw", P[5]),
        k.get("dg", P[6]), k.get("wk", P[7]), k.get("wkb", ws_need), k.get("T", 8), 4, 4096,
        k.get("dt", BF16), None)
    assert qb(dt=FP8) == DTYPE and qb(dt=FP8, T=0) == DTYPE
    assert qb(T=0) == OK and qb(eps=0.0) == ARG and qb(wkb=ws_need - 4) == ARG
    assert qb(wk=None) == NULL and qb(dg=P[6] + 2) == ALIGN and qb(wk=P[7] + 8) == ALIGN
    assert qb(din=P[4] + 16) == ALIAS and qb(dH=P[1]) == ALIAS and qb(wk=P[5]) == ALIAS
    # dH_out: an input like H (at most one of dH_in and dH_out, checked first)
    assert qb(din=P[0], dout=P[1]) == ARG and qb(din=P[0], dout=P[1], T=0) == ARG
    assert qb(dout=P[0] + 8) == ALIGN and qb(dout=P[4]) == ALIAS and qb(dout=P[5] + 64) == ALIAS
    assert qb(dout=P[7]) == ALIAS
    # dH NULL: records and dgamma only, so no addend may be given
    assert qb(dH=None, din=P[0] + 64) == ARG and qb(dH=None, dout=P[1] + 64) == ARG
    assert qb(dH=None, T=0) == OK and qb(dg=None) == NULL   # dgamma left out only with dH
    assert qb(dH=None, dg=None, wk=None) == NULL
    assert L.hc_sum_records(P[0], 10, 0, P[1], None) == SHAPE
    assert L.hc_sum_records(P[0], -1, 24, P[1], None) == ARG
    assert L.hc_sum_records(P[0], 10, 24, P[0] + 8, None) == ALIAS
    # the empty sum: no pointer is needed and nothing is launched
    assert L.hc_sum_records(None, 0, 24, None, None) == OK
    assert L.hc_sum_records(P[0], 0, 24, None, None) == OK
    assert L.hc_sum_records(None, 0, 0, None, None) == SHAPE
    assert L.hc_sum_records(None, 10, 24, P[1], None) == NULL


@pytest.mark.gpu
def test_sum_records_binding_checks_out(L):
    """The binding passes only a pointer for `out`: one of the wrong dtype or
    size would let the kernel write past its end, so it is rejected first."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rec = torch.zeros((4, 24), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        hc.sum_records(rec, out=torch.zeros(23, dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        hc.sum_records(rec, out=torch.zeros(24, dtype=torch.float64, device="cuda"))
    # the empty sum writes zeros
    o = torch.full((24,), 7.0, dtype=torch.float32, device="cuda")
    hc.sum_records(torch.zeros((0, 24), dtype=torch.float32, device="cuda"), out=o)
    assert torch.count_nonzero(o).item() == 0


def test_post_mix_weights_validation(L):
    """The fused write-back + next-layer weights call: its own limits (bf16 or
    FP8, d <= 4096), the post_mix and weights checks, the optional saved
    state, and every aliasing rule.  Every call here fails validation or has
    T = 0, so nothing is launched (the pointers are fake)."""
    K = 24
    need = int(L.hc_weights_saved_bytes(16, 4))

    def f(**k):
        return L.hc_post_mix_weights(
            k.get("H", P[0]), k.get("F", P[1]), k.get("w", P[2]), k.get("ws", 0), k.get("W", P[3]),
            k.get("wst", P[4]), k.get("scale", 0.01), k.get("eps", 1e-6), k.get("it", 0),
            k.get("O", P[5]), k.get("wo", P[6]), k.get("sv", None), k.get("svb", 0), k.get("T", 16),
            k.get("n", 4), k.get("d", 4096), k.get("dt", BF16), None)
    assert f(T=0) == OK and f(T=0, H=None) == OK and f(T=0, dt=FP8) == OK and f(T=0, ws=K) == OK
    assert f(dt=F32) == DTYPE and f(dt=9) == DTYPE and f(dt=F32, T=0) == DTYPE
    assert f(d=4104) == SHAPE and f(d=8192, dt=FP8) == SHAPE and f(d=12) == SHAPE and f(n=5) == SHAPE
    assert f(ws=K - 1) == SHAPE
    assert f(T=-1) == ARG and f(eps=0.0) == ARG and f(it=-1) == ARG and f(scale=float("inf")) == ARG
    for name in ("H", "F", "w", "W", "wst", "O", "wo"):
        assert f(**{name: None}) == NULL, name
    assert f(H=P[0] + 8) == ALIGN and f(W=P[3] + 4) == ALIGN and f(wo=P[6] + 2) == ALIGN
    # in place is allowed (checked on the GPU); any other overlap of an output is not
    assert f(O=P[0] + 16) == ALIAS and f(O=P[1]) == ALIAS and f(O=P[3]) == ALIAS
    assert f(wo=P[0] + 64) == ALIAS and f(wo=P[5] + 64) == ALIAS and f(wo=P[3]) == ALIAS
    assert f(wo=P[2]) == ALIAS and f(wo=P[4]) == ALIAS
    # the kept state: big enough, aligned, overlapping nothing
    assert f(sv=P[7], svb=need - 4) == ARG
    assert f(sv=P[7] + 4, svb=need) == ALIGN and f(sv=P[6], svb=need) == ALIAS
    assert f(sv=P[5] + 16, svb=need) == ALIAS and f(sv=P[0], svb=need) == ALIAS


def test_post_weights_pre_mix_validation(L):
    """The whole layer boundary: every check of hc_post_mix_weights, plus the
    read-mix's gain and output (present, aligned, overlapping nothing) and
    its epsilon.  Nothing is launched (fake pointers, or T = 0)."""
    K = 24
    need = int(L.hc_weights_saved_bytes(16, 4))

    def f(**k):
        return L.hc_post_weights_pre_mix(
            k.get("H", P[0]), k.get("F", P[1]), k.get("w", P[2]), k.get("ws", 0), k.get("W", P[3]),
            k.get("wst", P[4]), k.get("scale", 0.01), k.get("eps", 1e-6), k.get("it", 0),
            k.get("g", P[8]), k.get("peps", 1e-6), k.get("O", P[5]), k.get("wo", P[6]),
            k.get("u", P[9]), k.get("sv", None), k.get("svb", 0), k.get("T", 16), k.get("n", 4),
            k.get("d", 4096), k.get("dt", BF16), None)
    assert f(T=0) == OK and f(T=0, g=None, u=None) == OK and f(T=0, dt=FP8) == OK
    assert f(dt=F32) == DTYPE and f(d=4104) == SHAPE and f(ws=K - 1) == SHAPE
    assert f(peps=0.0) == ARG and f(peps=float("nan")) == ARG and f(eps=0.0) == ARG
    for name in ("H", "F", "w", "W", "wst", "O", "wo", "g", "u"):
        assert f(**{name: None}) == NULL, name
    assert f(g=P[8] + 4) == ALIGN and f(u=P[9] + 8) == ALIGN
    # u overlaps nothing; gamma is not overwritten by any output
    assert f(u=P[0]) == ALIAS and f(u=P[1] + 16) == ALIAS and f(u=P[5]) == ALIAS
    assert f(u=P[6]) == ALIAS and f(u=P[8]) == ALIAS and f(u=P[2]) == ALIAS
    assert f(O=P[8]) == ALIAS and f(wo=P[8]) == ALIAS
    assert f(sv=P[9], svb=need) == ALIAS and f(sv=P[7], svb=need - 4) == ARG


def test_sinkhorn_validation(L):
    f = lambda **k: L.hc_sinkhorn(k.get("l", P[0]), k.get("o", P[1]), k.get("it", 20),  # noqa: E731
                                  k.get("T", 100), k.get("n", 4), None)
    assert f(T=0) == OK
    assert f(l=None) == NULL and f(n=5) == SHAPE and f(it=-2) == ARG and f(T=-1) == ARG
    assert f(o=P[0] + 4) == ALIAS and f(o=P[0] + 2) == ALIGN


def test_block_tanh_validation(L):
    f = lambda **k: L.hc_block_tanh(k.get("u", P[0]), k.get("F", P[1]), k.get("c", 4096),  # noqa: E731
                                    k.get("dt", BF16), None)
    assert f(c=0) == OK and f(c=-8) == ARG and f(c=12) == SHAPE and f(c=12, dt=F32, F=P[0] + 16) == ALIAS
    assert f(u=None) == NULL and f(dt=4) == DTYPE and f(F=P[1] + 4) == ALIGN
    assert f(dt=FP8, c=4104) == SHAPE and f(dt=FP8, F=P[0] + 4000) == ALIAS   # 4104 % 16 = 8


def test_binding_rejects_host_tensors():
    import torch
    H = torch.zeros(2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        hc.pre_mix(H, torch.zeros(24), torch.ones(64))


def test_post_pre_mix_backward_validation(L):
    """The layer boundary's gradient: dtype, shapes, strides (both shared or
    both per token), workspace size, NULLs, alignment, and overlaps (dH may
    be dH_out itself, nothing else may overlap).  Nothing is launched."""
    need = L.hc_backward_workspace(8, 4, 4096)

    def f(**k):
        return L.hc_post_pre_mix_backward(
            k.get("go", P[0]), k.get("du", P[1]), k.get("H", P[2]), k.get("F", P[3]),
            k.get("w", P[4]), k.get("ws", 0), k.get("wn", P[5]), k.get("wns", 0), k.get("g", P[6]),
            k.get("eps", 1e-6), k.get("dH", P[7]), k.get("dF", P[8]), k.get("dw", P[9]),
            k.get("dwn", P[10]), k.get("dg", P[11]), k.get("wk", P[12]), k.get("wkb", need),
            k.get("T", 8), k.get("n", 4), k.get("d", 4096), k.get("dt", BF16), None)
    assert f(T=0) == OK and f(T=0, go=None, dH=None) == OK
    assert f(dt=FP8) == DTYPE and f(dt=FP8, T=0) == DTYPE and f(dt=5) == DTYPE
    assert f(n=5) == SHAPE and f(d=4100) == SHAPE and f(ws=3) == SHAPE and f(wns=23) == SHAPE
    # equal per-token strides pass that check (and stop at the next one here)
    assert f(ws=24, wns=0) == ARG and f(ws=0, wns=24) == ARG and f(ws=24, wns=24, dg=None) == NULL
    assert f(eps=0.0) == ARG and f(T=-2) == ARG and f(wkb=need - 1) == ARG
    for name in ("go", "du", "H", "F", "w", "wn", "g", "dH", "dF", "dw", "dwn", "dg", "wk"):
        assert f(**{name: None}) == NULL, name
    for name in ("go", "du", "H", "F", "g", "dH", "dF", "wk"):
        assert f(**{name: P[13] + 8}) == ALIGN, name
    for name in ("w", "wn", "dw", "dwn", "dg"):
        assert f(**{name: P[13] + 2}) == ALIGN, name
    # (dH == dH_out, in place, is allowed: the GPU tests run it) a partial
    # overlap with dH_out is not
    assert f(dH=P[0] + 16) == ALIAS
    assert f(dH=P[2]) == ALIAS and f(dH=P[1]) == ALIAS and f(dF=P[3]) == ALIAS
    assert f(dF=P[0] + 64) == ALIAS and f(dw=P[5]) == ALIAS and f(dwn=P[9]) == ALIAS
    assert f(dg=P[6]) == ALIAS and f(wk=P[7]) == ALIAS and f(dF=P[7] + 16) == ALIAS


def test_weights_backward_validation(L):
    need = L.hc_weights_backward_workspace(64, 4, 4096, 0)
    assert need > 0 and L.hc_weights_backward_workspace(0, 4, 4096, 0) == 0
    assert L.hc_weights_backward_workspace(64, 5, 4096, 0) == 0
    assert L.hc_weights_backward_workspace(64, 4, 4096, -1) == 0
    assert L.hc_weights_backward_workspace(64, 4, 4096, 20) > need      # Sinkhorn scratch
    f = lambda **k: L.hc_weights_backward(  # noqa: E731
        k.get("H", P[0]), k.get("W", P[1]), k.get("ws", P[2]), k.get("scale", 0.01),
        k.get("eps", 1e-6), k.get("it", 0), k.get("g", P[3]), k.get("g2", None), k.get("sv", None),
        k.get("din", None), k.get("dH", P[4]),
        k.get("dW", P[5]), k.get("dws", P[6]), k.get("wk", P[7]), k.get("wkb", need),
        k.get("T", 64), k.get("n", 4), k.get("d", 4096), k.get("dt", BF16), None)
    assert f(T=0) == OK and f(T=0, dH=None) == OK
    assert f(dt=FP8) == DTYPE and f(dt=7) == DTYPE
    assert f(n=0) == SHAPE and f(d=100) == SHAPE
    assert f(eps=0.0) == ARG and f(scale=float("inf")) == ARG and f(it=-1) == ARG
    assert f(T=-1) == ARG and f(wkb=need - 1) == ARG
    assert f(dW=None) == NULL and f(wk=None) == NULL and f(g=None) == NULL
    assert f(dH=P[4] + 8) == ALIGN and f(wk=P[7] + 4) == ALIGN and f(dws=P[6] + 2) == ALIGN
    assert f(dH=P[0]) == ALIAS and f(dW=P[1] + 64) == ALIAS and f(wk=P[3]) == ALIAS
    assert f(din=P[4] + 16) == ALIAS and f(dws=P[5] + 64) == ALIAS
    assert f(g2=P[3] + 2) == ALIGN and f(g2=P[4]) == ALIAS             # dw2 under dH
    assert f(sv=P[3] + 4) == ALIGN and f(sv=P[4] + 64) == ALIAS and f(sv=P[7]) == ALIAS


def test_post_pre_mix_backward_terms_validation(L):
    """The boundary's gradient with the weight producer's factors: per-token
    records only, dhbar and coef required, aligned, and overlapping no
    output; the rest as the plain call.  Nothing is launched."""
    need = L.hc_backward_workspace(8, 4, 4096)

    def f(**k):
        return L.hc_post_pre_mix_backward_terms(
            k.get("go", P[0]), k.get("du", P[1]), k.get("H", P[2]), k.get("F", P[3]),
            k.get("w", P[4]), k.get("ws", 24), k.get("wn", P[5]), k.get("wns", 24), k.get("g", P[6]),
            k.get("eps", 1e-6), k.get("db", P[12] + 4 * MiB), k.get("co", P[13]), k.get("dH", P[7]),
            k.get("dF", P[8]), k.get("dw", P[9]), k.get("dwn", P[10]), k.get("dg", P[11]),
            k.get("wk", P[12]), k.get("wkb", need), k.get("T", 8), k.get("n", 4), k.get("d", 4096),
            k.get("dt", BF16), None)
    assert f(T=0) == OK and f(T=0, db=None, co=None) == OK
    assert f(ws=0, wns=0) == ARG                       # shared records take no terms
    assert f(dt=FP8) == DTYPE and f(n=5) == SHAPE
    assert f(db=None) == NULL and f(co=None) == NULL and f(dg=None) == NULL
    assert f(db=P[12] + 4 * MiB + 8) == ALIGN and f(co=P[13] + 2) == ALIGN
    assert f(dH=P[12] + 4 * MiB) == ALIAS and f(dF=P[13]) == ALIAS and f(wk=P[13]) == ALIAS
    assert f(dw=P[12] + 4 * MiB + 64) == ALIAS


def test_weights_backward_terms_validation(L):
    need = L.hc_weights_backward_workspace(64, 4, 4096, 0)
    f = lambda **k: L.hc_weights_backward_terms(  # noqa: E731
        k.get("H", P[0]), k.get("W", P[1]), k.get("ws", P[2]), k.get("scale", 0.01),
        k.get("eps", 1e-6), k.get("it", 0), k.get("g", P[3]), k.get("g2", None), k.get("sv", None),
        k.get("db", P[4]), k.get("co", P[8]), k.get("dW", P[5]), k.get("dws", P[6]),
        k.get("wk", P[7]), k.get("wkb", need), k.get("T", 64), k.get("n", 4), k.get("d", 4096),
        k.get("dt", BF16), None)
    assert f(T=0) == OK and f(T=0, db=None, co=None) == OK
    assert f(dt=FP8) == DTYPE and f(n=0) == SHAPE and f(d=100) == SHAPE
    assert f(eps=0.0) == ARG and f(it=-1) == ARG and f(wkb=need - 1) == ARG
    assert f(db=None) == NULL and f(co=None) == NULL and f(dW=None) == NULL
    assert f(db=P[4] + 8) == ALIGN and f(co=P[8] + 2) == ALIGN
    # dhbar over an input, coef over dhbar, coef over the workspace or an output
    assert f(db=P[0]) == ALIAS and f(co=P[4] + 64) == ALIAS and f(co=P[7]) == ALIAS
    assert f(co=P[5]) == ALIAS and f(co=P[3]) == ALIAS and f(dW=P[4] + 64) == ALIAS


def test_weights_save_validation(L):
    need = L.hc_weights_saved_bytes(64, 4)
    assert need == (64 * 4 * 24 + 64 * 4) * 4 and L.hc_weights_saved_bytes(0, 4) == 0
    assert L.hc_weights_saved_bytes(64, 5) == 0 and L.hc_weights_saved_bytes(63, 3) == (63 * 3 * 15 + 1 + 63 * 3 + 3) * 4
    f = lambda **k: L.hc_weights_save(  # noqa: E731
        k.get("H", P[0]), k.get("W", P[1]), k.get("ws", P[2]), k.get("scale", 0.01),
        k.get("eps", 1e-6), k.get("it", 0), k.get("o", P[3]), k.get("sv", P[4]), k.get("svb", need),
        k.get("T", 64), k.get("n", 4), k.get("d", 4096), k.get("dt", BF16), None)
    assert f(T=0) == OK and f(T=0, sv=None, o=None) == OK
    assert f(dt=7) == DTYPE and f(n=0) == SHAPE and f(d=100) == SHAPE
    assert f(eps=0.0) == ARG and f(it=-1) == ARG and f(T=-1) == ARG and f(svb=need - 4) == ARG
    assert f(sv=None) == NULL and f(o=None) == NULL
    assert f(sv=P[4] + 4) == ALIGN and f(o=P[3] + 2) == ALIGN
    assert f(sv=P[0]) == ALIAS and f(o=P[4] + 64) == ALIAS and f(sv=P[1] + 16) == ALIAS


def test_sinkhorn_backward_validation(L):
    need = L.hc_sinkhorn_backward_workspace(100, 20)
    assert need == 100 * 20 * 64 and L.hc_sinkhorn_backward_workspace(100, 0) == 0
    f = lambda **k: L.hc_sinkhorn_backward(  # noqa: E731
        k.get("l", P[0]), k.get("g", P[1]), k.get("g2", None), k.get("o", P[2]), k.get("it", 20),
        k.get("wk", P[3]), k.get("wkb", need), k.get("T", 100), k.get("n", 4), None)
    assert f(T=0) == OK
    assert f(n=5) == SHAPE and f(it=-1) == ARG and f(T=-2) == ARG and f(wkb=need - 4) == ARG
    assert f(l=None) == NULL and f(wk=None) == NULL
    assert f(o=P[0] + 4) == ALIAS and f(wk=P[1]) == ALIAS and f(o=P[2] + 2) == ALIGN
    # dw2: optional, an input like dw
    assert f(g2=P[4] + 2) == ALIGN and f(g2=P[2] + 64) == ALIAS and f(g2=P[3]) == ALIAS
