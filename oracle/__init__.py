"""CPU oracle for the identity Hyper-Connections residual path.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library.
"""
from .oracle import (  # noqa: F401
    block_tanh,
    build,
    get_threads,
    load,
    post_mix,
    post_mix_backward,
    pre_mix,
    pre_mix_backward,
    round_bf16,
    round_f32,
    round_fp8,
    set_threads,
    sinkhorn,
    sinkhorn_backward,
    weights,
    weights_backward,
    widen,
)
