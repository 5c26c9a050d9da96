"""The 78-layer chain (T=4096, n=4, d=6144 bf16, per-layer weights identity +
N(0, 0.02), block F = tanh of the block input).

Pass criterion per layer: single-layer parity on 256 sampled tokens, with the
oracle fed the GPU's own layer input (pre, block and post each checked).
Tokens are independent, so a sample is an exact check of those tokens.

Drift is reported per layer against two oracle chains run on the same
sample from the same start: one in fp64 that stores u, F and H' to bf16
after every step as the GPU does, and one in pure fp64 with no store
rounding at all.  The first differs from the GPU only where fp32 and fp64
arithmetic round to different bf16 neighbours; 78 layers compound that, so
it is held to a bound a little above what was measured (below).  The second
also carries the rounding of every store and is reported only.  With
HC_DRIFT_OUT set to a path, the 78 rows are written there as JSON.

Identity weights are checked bitwise: the four streams stay copies and equal
the one-stream chain (explainer "Tencent open-sources Hy4 Preview at 770B --
Identity Hyper-Connections", "Jargon": identity initialization)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import check, dev, host, need_gpu, rel_err
from hyper_connections_amd import hc
from hyper_connections_amd.workloads import identity_record, layer_record, make_inputs, workload

pytestmark = pytest.mark.gpu

SAMPLE = 256
# Drift against the bf16-storing fp64 chain (single-layer parity is the pass
# criterion; the end-to-end drift, which compounds fp32-against-fp64
# rounding over 78 layers, is bounded and reported).  Measured on MI355X
# over the 78 layers on this sample: rising from 0 at layer 1 to 0.020
# (0.033 against pure fp64), per layer in profiles/chain-bf16_drift.md;
# the bound is twice that maximum.
DRIFT_BOUND = 0.04


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_chain_per_layer_parity_and_drift():
    wl = workload("chain-bf16")
    inp = make_inputs(wl)
    g = inp["gamma"]
    gd = dev(g)
    Ha = dev(inp["H"])
    Hb = torch.empty_like(Ha)
    u = torch.empty((wl.T, wl.d), dtype=torch.bfloat16, device="cuda")
    F = torch.empty_like(u)
    rng = np.random.default_rng(505)
    idx = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(np.arange(1, wl.T - 1), SAMPLE - 2,
                                                                replace=False)]))
    assert idx.size == SAMPLE
    ti = torch.from_numpy(idx).cuda()
    H_b16 = inp["H"][idx]                       # fp64 arithmetic, bf16 stores
    H_f64 = oracle.widen(inp["H"][idx])         # fp64 arithmetic, no store rounding
    rows = []
    for layer in range(wl.layers):
        w = layer_record(wl, layer)
        w64 = w.astype(np.float64)
        wd = dev(w)
        hc.pre_mix(Ha, wd, gd, wl.eps, out=u)
        hc.block_tanh(u, out=F)
        hc.post_mix(Ha, F, wd, out=Hb)
        H_in, u_s, F_s, H_out = host(Ha[ti]), host(u[ti]), host(F[ti]), host(Hb[ti])
        e_pre = check(u_s, oracle.pre_mix(H_in, w64, g, wl.eps), f"layer {layer} pre")
        e_blk = check(F_s, oracle.block_tanh(u_s), f"layer {layer} block")
        e_post = check(H_out, oracle.post_mix(H_in, F_s, w64), f"layer {layer} post")
        u_o = oracle.round_bf16(oracle.pre_mix(H_b16, w64, g, wl.eps))
        F_o = oracle.round_bf16(oracle.block_tanh(u_o))
        H_b16 = oracle.round_bf16(oracle.post_mix(H_b16, F_o, w64))
        u_64 = oracle.pre_mix(H_f64, w64, g, wl.eps)
        H_f64 = oracle.post_mix(H_f64, oracle.block_tanh(u_64), w64)
        rows.append({"layer": layer + 1, "parity_pre": e_pre, "parity_block": e_blk,
                     "parity_post": e_post,
                     "drift_vs_bf16_storing_fp64": rel_err(H_out, oracle.widen(H_b16)),
                     "drift_vs_pure_fp64": rel_err(H_out, H_f64)})
        Ha, Hb = Hb, Ha
    out = os.environ.get("HC_DRIFT_OUT")
    if out:
        with open(out, "w") as fh:
            json.dump({"workload": wl.name, "T": wl.T, "n": wl.n, "d": wl.d, "layers": wl.layers,
                       "sample_tokens": int(idx.size), "drift_bound": DRIFT_BOUND,
                       "rows": rows}, fh, indent=1)
    drift = [r["drift_vs_bf16_storing_fp64"] for r in rows]
    print("per-layer drift vs bf16-storing fp64 chain:", " ".join(f"{e:.2e}" for e in drift))
    assert max(drift) <= DRIFT_BOUND


def test_identity_chain_bitwise():
    """78 identity layers on n copies: the streams stay bitwise equal to each
    other and to the one-stream chain x_{l+1} = x_l + tanh(RMSNorm(x_l))."""
    wl = workload("chain-bf16", T=64)
    x = make_inputs(wl)["H"][:, :1, :].copy()
    gd = dev(np.ones(wl.d, np.float32))
    H4, H1 = dev(np.repeat(x, 4, axis=1)), dev(x)
    id4, id1 = dev(identity_record(4)), dev(identity_record(1))
    for _ in range(wl.layers):
        F4 = hc.block_tanh(hc.pre_mix(H4, id4, gd))
        F1 = hc.block_tanh(hc.pre_mix(H1, id1, gd))
        H4 = hc.post_mix(H4, F4, id4)
        H1 = hc.post_mix(H1, F1, id1)
    h4, h1 = host(H4), host(H1)
    for i in range(4):
        assert np.array_equal(h4[:, i, :], h1[:, 0, :])


def test_fused_chain_matches_unfused_bitwise():
    """Cross-layer fusion (write-back of layer l with the read-mix of layer
    l+1) over 12 layers equals the unfused chain bitwise."""
    wl = workload("chain-bf16", T=512)
    inp = make_inputs(wl)
    gd = dev(inp["gamma"])
    recs = [dev(layer_record(wl, l)) for l in range(13)]
    # unfused
    H = dev(inp["H"])
    for l in range(12):
        F = hc.block_tanh(hc.pre_mix(H, recs[l], gd))
        H = hc.post_mix(H, F, recs[l])
    ref = host(H)
    # fused: pre of layer 0, then post(l)+pre(l+1)
    H = dev(inp["H"])
    u = hc.pre_mix(H, recs[0], gd)
    for l in range(12):
        F = hc.block_tanh(u)
        H, u = hc.post_pre_mix(H, F, recs[l], recs[l + 1], gd)
    assert np.array_equal(host(H), ref)
