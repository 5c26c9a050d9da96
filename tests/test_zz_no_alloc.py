"""hc_post_mix_backward_noalloc, the post gradient that allocates nothing
(its scratch is the library's own per-GPU array), called through the C ABI:
its outputs are bitwise those of hc_post_mix_backward with a caller
workspace, on two calls in a row, the second with a smaller input (the
array keeps the first call's contents), for a shared record (which uses the
scratch) and per-token records (which do not)."""
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


def noalloc():
    # the C entry point itself (its argument types are set by the binding)
    return hc.lib().hc_post_mix_backward_noalloc


def inputs(rng, T, n, d, shared):
    K = 2 * n + n * n
    G = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    H = f32_to_bf16_bits(rng.standard_normal((T, n, d)).astype(np.float32))
    F = f32_to_bf16_bits(rng.standard_normal((T, d)).astype(np.float32))
    w = (identity_record(n) + 0.05 * rng.standard_normal((K,) if shared else (T, K))).astype(np.float32)
    return dev(G), dev(H), dev(F), dev(w)


def run_noalloc(f, G, H, F, w, h_grad):
    T, n, d = H.shape
    K = 2 * n + n * n
    shared = w.dim() == 1
    dH = torch.empty_like(H) if h_grad else None
    dF = torch.empty((T, d), dtype=H.dtype, device="cuda")
    dw = torch.empty((K,) if shared else (T, K), dtype=torch.float32, device="cuda")
    st = f(G.data_ptr(), H.data_ptr(), F.data_ptr(), w.data_ptr(), 0 if shared else K,
           dH.data_ptr() if dH is not None else None, dF.data_ptr(), dw.data_ptr(), T, n, d,
           hc.HC_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0, hc.status_str(st)
    return dH, dF, dw


@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("h_grad", [True, False])
def test_noalloc_equals_workspace_call_twice(shared, h_grad):
    f = noalloc()
    rng = np.random.default_rng(7 + shared + 2 * h_grad)
    # the first call the larger (16384 tokens at n = 4), the second smaller,
    # over the first's leftovers in the scratch array
    for T, n, d in [(16384, 4, 1024), (300, 3, 4096)]:
        G, H, F, w = inputs(rng, T, n, d, shared)
        a = run_noalloc(f, G, H, F, w, h_grad)
        b = hc.post_mix_backward(G, H, F, w, h_grad=h_grad)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            if x is None:
                assert y is None
                continue
            assert np.array_equal(host(x), host(y)), f"T={T} n={n} d={d}"


def test_noalloc_rejects_bad_calls_without_launching():
    f = noalloc()
    P = [0x10000000 * (i + 1) for i in range(8)]
    args = lambda **k: (k.get("G", P[0]), P[1], P[2], P[3], 0, P[4], P[5], P[6],  # noqa: E731
                        k.get("T", 16), k.get("n", 4), k.get("d", 4096), k.get("dt", hc.HC_BF16), None)
    assert f(*args(dt=hc.HC_FP8)) == 3
    assert f(*args(n=5)) == 2
    assert f(*args(T=-1)) == 6
    assert f(*args(G=None)) == 1
    assert f(*args(T=0)) == 0
