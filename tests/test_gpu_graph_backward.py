"""The backward calls inside a HIP graph (torch.cuda.CUDAGraph around the
library's launches): a layer's gradients -- post, pre accumulating into the
same dH (or, folded, pre forming the whole dH from post's dH'), and the
weight producer's -- captured once and replayed, with the
outputs and workspaces overwritten by eager work before every replay, so each
replay must rewrite everything it produces.  Every replay equals the eager
calls bitwise (the library enqueues kernels only: no memsets, no host work)."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, need_gpu
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import f32_to_bf16_bits, identity_record

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def bf16(rng, shape, sd=1.0):
    return dev(f32_to_bf16_bits((sd * rng.standard_normal(shape)).astype(np.float32)))


@pytest.mark.parametrize("fold", [False, True])
@pytest.mark.parametrize("records", ["shared", "per-token"])
def test_backward_graph_replays_equal_eager(records, fold):
    rng = np.random.default_rng(5 if records == "shared" else 6)
    T, n, d = 300, 4, 1024
    K = 2 * n + n * n
    H, F = bf16(rng, (T, n, d)), bf16(rng, (T, d))
    dHo, du = bf16(rng, (T, n, d)), bf16(rng, (T, d))
    gamma = dev((1 + 0.1 * rng.standard_normal(d)).astype(np.float32))
    ws = dev((identity_record(n) + 0.05 * rng.standard_normal(K)).astype(np.float32))
    W = bf16(rng, (K, d), 0.02)
    per_token = records == "per-token"
    if per_token:
        w, saved = hc.weights_save(H, W, ws, 0.01, 1e-6, 0)
        dwp = torch.empty((T, K), dtype=torch.float32, device="cuda")
        dwq = torch.empty_like(dwp)
    else:
        w, saved = ws, None
        dwp = torch.empty(K, dtype=torch.float32, device="cuda")
        dwq = torch.empty_like(dwp)
    dH = torch.empty_like(H)
    dF = torch.empty_like(F)
    dg = torch.empty(d, dtype=torch.float32, device="cuda")
    dW = torch.empty((K, d), dtype=torch.float32, device="cuda")
    dws = torch.empty(K, dtype=torch.float32, device="cuda")
    wk = torch.empty(int(hc.lib().hc_backward_workspace(T, n, d)), dtype=torch.uint8, device="cuda")
    wwk = torch.empty(int(hc.lib().hc_weights_backward_workspace(T, n, d, 0)), dtype=torch.uint8,
                      device="cuda")
    outs = [dH, dF, dg, dwp, dwq, dW, dws]

    def step():
        if fold:
            hc.post_mix_backward(dHo, H, F, w, dF=dF, dw=dwp, workspace=wk, h_grad=False)
            hc.pre_mix_backward(du, H, w, gamma, 1e-6, dH_out=dHo, out=dH, dw=dwq, dgamma=dg,
                                workspace=wk)
        else:
            hc.post_mix_backward(dHo, H, F, w, dH=dH, dF=dF, dw=dwp, workspace=wk)
            hc.pre_mix_backward(du, H, w, gamma, 1e-6, dH_in=dH, out=dH, dw=dwq, dgamma=dg,
                                workspace=wk)
        if per_token:
            hc.weights_backward(H, W, ws, 0.01, dwp, 1e-6, 0, dH_in=dH, out=dH, dW=dW,
                                dw_static=dws, workspace=wwk, dw2=dwq, saved=saved)

    step()
    torch.cuda.synchronize()
    eager = [host(t) for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        wk.fill_(0xFF)
        wwk.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, t in zip(["dH", "dF", "dgamma", "dw post", "dw pre", "dW", "dw_static"],
                              eager, outs):
            if per_token or name not in ("dW", "dw_static"):
                assert np.array_equal(host(t), a, equal_nan=True), f"replay {rep}: {name} differs"
        _ = (H.float() * 2).sum().item()   # eager work between replays


@pytest.mark.parametrize("records", ["shared", "per-token", "per-token-terms"])
def test_boundary_backward_graph_replays_equal_eager(records):
    """One layer boundary's gradient in one pass, captured and replayed: with
    shared records the boundary call alone; with per-token records produced
    from the streams the whole schedule (the read-mix's dalpha alone, the
    weight producer's gradient onto the arriving gradient, or as its factors
    (dhbar, coefficients) that the boundary call adds, then the boundary
    call).  Outputs and workspaces are overwritten before every replay."""
    rng = np.random.default_rng({"shared": 7, "per-token": 8, "per-token-terms": 9}[records])
    terms = records == "per-token-terms"
    T, n, d = 300, 4, 1024
    K = 2 * n + n * n
    H, F, H2 = bf16(rng, (T, n, d)), bf16(rng, (T, d)), bf16(rng, (T, n, d))
    G, du = bf16(rng, (T, n, d)), bf16(rng, (T, d))
    gamma = dev((1 + 0.1 * rng.standard_normal(d)).astype(np.float32))
    ws = dev((identity_record(n) + 0.05 * rng.standard_normal(K)).astype(np.float32))
    W = bf16(rng, (K, d), 0.02)
    per_token = records != "shared"
    if per_token:
        w, _ = hc.weights_save(H, W, ws, 0.01, 1e-6, 0)
        w2, saved2 = hc.weights_save(H2, W, ws, 0.01, 1e-6, 0)
        shape = (T, K)
    else:
        w, w2, saved2 = ws, ws, None
        shape = (K,)
    dwp = torch.empty(shape, dtype=torch.float32, device="cuda")
    dwn = torch.empty(shape, dtype=torch.float32, device="cuda")
    dalpha = torch.empty((T, K), dtype=torch.float32, device="cuda")
    post_part = dev(rng.standard_normal((T, K)).astype(np.float32))   # from the next boundary
    Gw = torch.empty_like(G)
    dH, dF = torch.empty_like(H), torch.empty_like(F)
    dg = torch.empty(d, dtype=torch.float32, device="cuda")
    dW = torch.empty((K, d), dtype=torch.float32, device="cuda")
    dws = torch.empty(K, dtype=torch.float32, device="cuda")
    wk = torch.empty(int(hc.lib().hc_backward_workspace(T, n, d)), dtype=torch.uint8, device="cuda")
    wk2 = torch.empty_like(wk)
    wwk = torch.empty(int(hc.lib().hc_weights_backward_workspace(T, n, d, 0)), dtype=torch.uint8,
                      device="cuda")
    dhb = torch.empty((T, d), dtype=torch.float32, device="cuda")
    coef = torch.empty((T, 2 * n), dtype=torch.float32, device="cuda")
    outs = [dH, dF, dwp, dwn, dg] + ([dalpha, dW, dws] if per_token else [])
    outs += [dhb, coef] if terms else ([Gw] if per_token else [])

    def step():
        arriving = G
        if per_token:
            hc.pre_mix_backward(du, H2, w2, gamma, 1e-6, h_grad=False, g_grad=False, dw=dalpha,
                                workspace=wk2)
        if terms:
            hc.weights_backward_terms(H2, W, ws, 0.01, dalpha, 1e-6, 0, dhbar=dhb, coef=coef,
                                      dW=dW, dw_static=dws, workspace=wwk, dw2=post_part,
                                      saved=saved2)
        elif per_token:
            hc.weights_backward(H2, W, ws, 0.01, dalpha, 1e-6, 0, dH_in=G, out=Gw, dW=dW,
                                dw_static=dws, workspace=wwk, dw2=post_part, saved=saved2)
            arriving = Gw
        hc.post_pre_mix_backward(arriving, du, H, F, w, w2, gamma, 1e-6, out=dH, dF=dF, dw=dwp,
                                 dw_next=dwn, dgamma_next=dg, workspace=wk,
                                 terms=(dhb, coef) if terms else None)

    step()
    torch.cuda.synchronize()
    eager = [host(t) for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        for t in (wk, wk2, wwk):
            t.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, t) in enumerate(zip(eager, outs)):
            assert np.array_equal(host(t), a, equal_nan=True), f"replay {rep}: output {i} differs"
        _ = (H.float() * 2).sum().item()   # eager work between replays
