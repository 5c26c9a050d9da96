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
    """The separate weights kernel's own bytes: read H (n*d) and write one
    record; the K x d projection matrix is shared by all tokens and not
    counted per token.  This read of H is a second pass over the state that
    the method does not need (see method_bytes), so it counts for the
    kernel's own roofline, never towards a layer's."""
    return n * d * s + record_bytes(n)


def method_bytes(kind: str, n: int, d: int, s: int) -> int:
    """The bytes one layer of the method itself must move per token, the
    figure a layer's time is graded on however its kernels are split:
    pre reads H and writes u, post reads H and F and writes H'
    ((3n + 2) d s), plus the weight records that leave the chip:
      static   one shared record, not counted per token;
      dynamic  the per-token record is formed while H is on chip; its mix
               and write weights (n + n^2 fp32) are written once and read
               once by the write-back;
      mhc      the per-token logit record (K fp32) is read once.
    A kernel split that moves more (a separate weights pass re-reading H,
    a weight record written and read back) is charged against this."""
    base = (3 * n + 2) * d * s
    if kind == "dynamic":
        return base + 2 * (n + n * n) * RECORD_BYTES_PER_ENTRY
    if kind == "mhc":
        return base + record_bytes(n)
    return base


def post_weights_bytes(n: int, d: int, s: int) -> int:
    """Write-back fused with the next layer's weights: post's bytes with a
    per-token record read, plus the next record written (H' is projected
    from registers, not read back)."""
    return post_bytes(n, d, s, True) + record_bytes(n)


def post_weights_pre_bytes(n: int, d: int, s: int) -> int:
    """The whole layer boundary with per-token weights in one pass: read H
    and F, write H' and the next block input u; the per-token [beta | A]
    read and the next record written (alpha is used from the chip)."""
    return (2 * n + 2) * d * s + (n + n * n) * RECORD_BYTES_PER_ENTRY + record_bytes(n)


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


def post_pre_bwd_bytes(n: int, d: int, s: int, per_token_record: bool = False) -> int:
    """Gradient of one layer boundary (write-back and next read-mix) in one
    pass: read dH', du, H and F, write dH and dF ((3n + 3) d s; H' is
    recomputed, not read), and the two gradient records (as in the separate
    calls, whose rows total (5n + 3) d s); per-token records also read the
    two weight records."""
    return (3 * n + 3) * d * s + (4 if per_token_record else 2) * record_bytes(n)


def sinkhorn_bwd_bytes(n: int, two_gradients: bool = True) -> int:
    """Gradient of the mHC transform per token: read the logit record and the
    record gradient (two of them when they come from two calls), write the
    logit gradient.  Not counted: the workspace that keeps the matrix entering
    every iteration (64 B per iteration, written and read back)."""
    return (4 if two_gradients else 3) * record_bytes(n)


def pre_records_bytes(n: int, d: int, s: int) -> int:
    """The read-mix's record gradient alone (dH and dgamma not formed): read
    du and H, write one gradient record."""
    return (n + 1) * d * s + record_bytes(n)


def weights_bwd_bytes(n: int, d: int, s: int) -> int:
    """Gradient of the per-token weights: read H, read the incoming dH and
    write dH once each, plus two gradient records read (from pre and post).
    Not counted: the projections P_i = W H_i and norms r_i, read from what
    the forward kept (n (K + 1) floats per token), or recomputed with a second
    read of H when it kept nothing."""
    return 3 * n * d * s + 2 * record_bytes(n)


def weights_bwd_terms_bytes(n: int, d: int, s: int) -> int:
    """Gradient of the per-token weights returned as its factors: read H once,
    write dhbar (d fp32) and the coefficients (2n fp32), plus the two gradient
    records read.  The projections and norms kept by the forward are not
    counted, as in weights_bwd_bytes."""
    return n * d * s + 4 * d + 4 * 2 * n + 2 * record_bytes(n)


def post_pre_bwd_terms_bytes(n: int, d: int, s: int) -> int:
    """The layer boundary's gradient with the weight producer's factors added
    at H': post_pre_bwd_bytes with per-token records, plus dhbar (d fp32) and
    the coefficients (2n fp32) read."""
    return post_pre_bwd_bytes(n, d, s, True) + 4 * d + 4 * 2 * n


def weights_bwd_stream_bytes(n: int, d: int, s: int) -> int:
    """The streaming pass of the weights gradient alone: read H and the
    incoming dH, write dH (the per-token coefficients it reads, K + 2n floats,
    are not counted)."""
    return 3 * n * d * s
