"""The binding on a side stream: every wrapper allocates its outputs and
workspaces on the stream its kernels run on, so that torch's caching
allocator cannot hand that memory to other work while the kernels still run.
Each gradient (post, pre, the weight producer, also as its factors, the
layer boundary's, also adding them) and the fused write-backs are run on a
side stream, with other work queued on the current stream that
reuses freed memory meanwhile, and compared bitwise with the same call on
the current stream."""
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


def inputs(T=2048, n=4, d=4096, seed=3):
    rng = np.random.default_rng(seed)
    K = 2 * n + n * n
    bf = lambda *s: dev(f32_to_bf16_bits(rng.standard_normal(s).astype(np.float32)))  # noqa: E731
    H, F, G, du = bf(T, n, d), bf(T, d), bf(T, n, d), bf(T, d)
    w = dev((identity_record(n) + 0.05 * rng.standard_normal(K)).astype(np.float32))
    wt = dev((identity_record(n) + 0.05 * rng.standard_normal((T, K))).astype(np.float32))
    g = dev((1 + 0.1 * rng.standard_normal(d)).astype(np.float32))
    W = bf(K, d) * 0.02
    ws = dev(identity_record(n))
    dw = dev(rng.standard_normal((T, K)).astype(np.float32))
    return H, F, G, du, w, wt, g, W, ws, dw


def churn():
    """Work on the current stream that allocates and frees device memory."""
    for _ in range(8):
        x = torch.empty(32 << 20, dtype=torch.uint8, device="cuda")
        x.fill_(0xAB)
        del x


@pytest.mark.parametrize("which", ["post", "pre", "weights", "post_weights", "boundary",
                                   "boundary_per_token", "post_weights_pre", "weights_terms",
                                   "boundary_terms"])
def test_side_stream_equals_current_stream(which):
    H, F, G, du, w, wt, g, W, ws, dw = inputs()
    terms = hc.weights_backward_terms(H, W, ws, 0.01, dw)[:2] if which == "boundary_terms" else None

    def run(stream):
        if which == "post":
            return hc.post_mix_backward(G, H, F, w, stream=stream)
        if which == "pre":
            return hc.pre_mix_backward(du, H, w, g, 1e-6, stream=stream)
        if which == "weights":
            return hc.weights_backward(H, W, ws, 0.01, dw, 1e-6, 0, stream=stream)
        if which == "boundary":
            return hc.post_pre_mix_backward(G, du, H, F, w, w, g, 1e-6, stream=stream)
        if which == "boundary_per_token":
            return hc.post_pre_mix_backward(G, du, H, F, wt, wt, g, 1e-6, stream=stream)
        if which == "post_weights_pre":
            return hc.post_weights_pre_mix(H, F, wt, W, ws, 0.01, g, stream=stream)
        if which == "weights_terms":
            return hc.weights_backward_terms(H, W, ws, 0.01, dw, 1e-6, 0, stream=stream)
        if which == "boundary_terms":
            # the factors come from the current stream's call; the side stream
            # waits for them before it starts (below)
            return hc.post_pre_mix_backward(G, du, H, F, wt, wt, g, 1e-6, stream=stream,
                                            terms=terms)
        return hc.post_mix_weights(H, F, wt, W, ws, 0.01, 1e-6, 0, stream=stream)

    ref = [host(x) for x in run(None)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = run(side)
    churn()                                  # competes for freed blocks meanwhile
    # the raw handle form is accepted too
    out2 = run(side.cuda_stream)
    churn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b, r in zip(out, out2, ref):
        assert np.array_equal(host(a), r)
        assert np.array_equal(host(b), r)
