"""Algorithmic byte counts of the Hyper-Connections residual path.

These are the bytes the method itself must move through HBM, independent of
how a kernel is written: every stored input read once, every output written
once.  s is the storage size of one element (4 for fp32, 2 for bf16); a weight
record is K = 2n + n^2 fp32 values.

The state a layer boundary carries is n * d * s bytes per token in flight: one
hidden-width vector per stream (explainer "Tencent open-sources Hy4 Preview at
770B -- Identity Hyper-Connections", section "What four streams cost per
token", worked with hidden width 8192 in bf16).
"""
from __future__ import annotations

RECORD_BYTES_PER_ENTRY = 4


def state_bytes(n: int, d: int, s: int, tokens: int = 1) -> int:
    """Residual state handed across one layer boundary."""
    return n * d * s * tokens


def record_bytes(n: int) -> int:
    return (2 * n + n * n) * RECORD_BYTES_PER_ENTRY


def pre_bytes(n: int, d: int, s: int, per_token_record: bool = False) -> int:
    """Read H (n*d), write u (d); per-token alpha read when records are per token."""
    return (n + 1) * d * s + (n * RECORD_BYTES_PER_ENTRY if per_token_record else 0)


def post_bytes(n: int, d: int, s: int, per_token_record: bool = False) -> int:
    """Read H (n*d) and F (d), write H' (n*d); per-token beta and A read."""
    return (2 * n + 1) * d * s + ((n + n * n) * RECORD_BYTES_PER_ENTRY if per_token_record else 0)


def weights_bytes(n: int, d: int, s: int) -> int:
    """Read H (n*d) and write one record; the K x d projection matrix is
    shared by all tokens and not counted per token."""
    return n * d * s + record_bytes(n)


def sinkhorn_bytes(n: int) -> int:
    """Read one logit record, write one weight record."""
    return 2 * record_bytes(n)


def post_pre_bytes(n: int, d: int, s: int, per_token_record: bool = False) -> int:
    """Fused write-back of layer l and read-mix of layer l+1: read H and F,
    write H' and the next block input u."""
    rec = (n + n * n + n) * RECORD_BYTES_PER_ENTRY if per_token_record else 0
    return (2 * n + 2) * d * s + rec


def post_bwd_bytes(n: int, d: int, s: int, h_grad: bool = True) -> int:
    """Gradient of post: read dH', H and F, write dH (unless the pre gradient
    forms it: h_grad False) and dF and one gradient record."""
    return ((3 if h_grad else 2) * n + 2) * d * s + record_bytes(n)


def pre_bwd_bytes(n: int, d: int, s: int, accumulate: bool = True) -> int:
    """Gradient of pre: read du and H (and the incoming dH when it is
    accumulated), write dH and one gradient record (the dgamma partials,
    d floats per group of tokens, are not counted)."""
    return (2 * n + 1 + (n if accumulate else 0)) * d * s + record_bytes(n)


def weights_bwd_bytes(n: int, d: int, s: int) -> int:
    """Gradient of the per-token weights: read H, read the incoming dH and
    write dH once each, plus two gradient records read (from pre and post).
    Not counted: the projections P_i = W H_i and norms r_i, read from what
    the forward kept (n (K + 1) floats per token), or recomputed with a second
    read of H when it kept nothing."""
    return 3 * n * d * s + 2 * record_bytes(n)


def weights_bwd_stream_bytes(n: int, d: int, s: int) -> int:
    """The streaming pass of the weights gradient alone: read H and the
    incoming dH, write dH (the per-token coefficients it reads, K + 2n floats,
    are not counted)."""
    return 3 * n * d * s
