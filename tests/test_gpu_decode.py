"""Decode regime: 64 tokens in flight, 78 layers (the explainer's worked shape:
hidden width 8192, four streams, about 4 MB of state).  The layer loop is
captured in a HIP graph (torch.cuda.CUDAGraph around the library's launches);
every replay must equal the eager loop bitwise, with eager work and
synchronisations between replays.  The input is never written, so every
replay starts from the same state."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, need_gpu
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import layer_record, make_inputs, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def chain(H_in, X, Y, u, F, recs, gd, fused):
    """78 layers: layer 0 reads H_in, then X and Y alternate; returns the final buffer."""
    src = H_in
    outs = (X, Y)
    if fused:
        hc.pre_mix(src, recs[0], gd, out=u)
        for l in range(len(recs) - 1):
            hc.block_tanh(u, out=F)
            dst = outs[l % 2]
            hc.post_pre_mix(src, F, recs[l], recs[l + 1], gd, out=dst, u_out=u)
            src = dst
    else:
        for l in range(len(recs) - 1):
            hc.pre_mix(src, recs[l], gd, out=u)
            hc.block_tanh(u, out=F)
            dst = outs[l % 2]
            hc.post_mix(src, F, recs[l], out=dst)
            src = dst
    return src


@pytest.mark.parametrize("fused", [False, True])
def test_decode_graph_replays_equal_eager(fused):
    wl = workload("decode-bf16")
    inp = make_inputs(wl)
    gd = dev(inp["gamma"])
    recs = [dev(layer_record(wl, l)) for l in range(wl.layers + 1)]
    H_in = dev(inp["H"])
    X, Y = torch.empty_like(H_in), torch.empty_like(H_in)
    u = torch.empty((wl.T, wl.d), dtype=H_in.dtype, device="cuda")
    F = torch.empty_like(u)
    out = chain(H_in, X, Y, u, F, recs, gd, fused)
    torch.cuda.synchronize()
    eager = host(out)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gout = chain(H_in, X, Y, u, F, recs, gd, fused)
    for rep in range(3):
        X.zero_()
        Y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(gout), eager), f"replay {rep} differs from eager"
        _ = (H_in.float() * 2).sum().item()   # eager work between replays


def test_decode_layer_parity():
    """One decode layer (d = 8192, a 1024-thread row) against the oracle."""
    wl = workload("decode-bf16")
    inp = make_inputs(wl)
    w = layer_record(wl, 0)
    Hd, gd, wd = dev(inp["H"]), dev(inp["gamma"]), dev(w)
    u = hc.pre_mix(Hd, wd, gd)
    F = hc.block_tanh(u)
    Hp = hc.post_mix(Hd, F, wd)
    w64 = w.astype(np.float64)
    check(host(u), oracle.pre_mix(inp["H"], w64, inp["gamma"]), "decode pre")
    check(host(F), oracle.block_tanh(host(u)), "decode block")
    check(host(Hp), oracle.post_mix(inp["H"], host(F), w64), "decode post")
