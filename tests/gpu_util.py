"""Helpers for the GPU parity tests: host <-> device transfer of storage
arrays and the error metric.

Error metric: for every element, |gpu - ref| / max(|ref|, rms(ref row)), where
the row is the d-vector (or weight record) the element belongs to; the
maximum over elements is compared with the tolerance.  Dividing by the row
RMS stops cancellation near zero from failing a correct result.

Tolerances: 1e-5 for fp32 storage; 2e-2 for bf16 storage with fp32
arithmetic.  For bf16 the tests also require one bf16 unit in the last place
(2^-8 of the row scale), which a correctly rounded store plus fp32 arithmetic
meets with margin.  For FP8 E4M3 storage (3 mantissa bits) the bound is one
FP8 unit in the last place, 2^-3 of the value (or of the row scale), and the
stored codes must equal the oracle's rounding of its fp64 value except for
at most 1 + 0.1% of them: fp32 arithmetic moves a value across an FP8
rounding boundary only when it lies within about 1e-6 (relative) of one.
FP8 stores saturate, so FP8 results are compared with the reference clipped
to +-448."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle

TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_BF16_ULP = 2.0 ** -8
TOL_FP8 = 2.0 ** -3
TOL_RECORD = 1e-5      # fp32 weight records (any storage dtype of H)

# With HC_MARGIN_OUT set to a path, every gradient check's achieved error
# and its tolerance are collected and written there as JSON at the end of
# the session (tests/conftest.py), so the margin is visible and not only
# the pass or fail.
MARGINS: list = []


def record_margin(what: str, err: float, tol: float) -> None:
    import os
    if os.environ.get("HC_MARGIN_OUT"):
        MARGINS.append({"check": what, "error": float(err), "tolerance": float(tol)})


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def dev(a: np.ndarray) -> torch.Tensor:
    """Storage array (float32, uint16 bf16 bits or uint8 fp8 codes) -> device tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    if a.dtype == np.uint8:
        return torch.from_numpy(a).view(torch.float8_e4m3fn).cuda()
    if a.dtype in (np.float32, np.float64):
        return torch.from_numpy(a.astype(np.float32)).cuda()
    raise TypeError(a.dtype)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage array (uint16 bits for bf16, uint8 codes for fp8)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().copy()
    return t.numpy().copy()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max over elements of |got - ref| / max(|ref|, rms(ref row)); rows are
    the last axis.  NaNs must match position for position."""
    g = (oracle.widen(got) if got.dtype in (np.uint8, np.uint16, np.float32)
         else np.asarray(got, np.float64))
    r = np.asarray(ref, np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), "NaN positions differ"
    g, r = np.where(gn, 0.0, g), np.where(rn, 0.0, r)
    inf = np.isinf(r) | np.isinf(g)
    if inf.any():
        assert np.array_equal(g[inf], r[inf]), "infinities differ"
        g, r = np.where(inf, 0.0, g), np.where(inf, 0.0, r)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    scale = np.maximum(np.abs(r), rms)
    scale = np.where(scale == 0, 1.0, scale)
    return float(np.max(np.abs(g - r) / scale))


def check(got: np.ndarray, ref: np.ndarray, what: str = "", one_ulp: bool = True) -> float:
    """Assert the storage-dtype tolerance; returns the error.  `one_ulp=False`
    drops the one-ulp bound for results stored twice (an accumulation into a
    rounded buffer), which only the 2e-2 tolerance covers."""
    if got.dtype == np.uint8:
        # FP8 stores saturate at +-448: compare with the reference so clipped
        ref = np.asarray(ref, np.float64)
        ref = np.where(np.abs(ref) > 448.0, np.copysign(448.0, ref), ref)
    e = rel_err(got, ref)
    if got.dtype == np.uint8:
        assert e <= TOL_FP8, f"{what}: max rel err {e:.3g} > one fp8 ulp"
        want = oracle.round_fp8(np.asarray(ref, np.float64))
        fin = ~np.isnan(np.asarray(ref, np.float64))
        bad = int(np.count_nonzero(want[fin] != got[fin]))
        assert bad <= 1 + fin.sum() // 1000, f"{what}: {bad} of {fin.sum()} fp8 codes differ"
    elif got.dtype == np.uint16:
        assert e <= TOL_BF16, f"{what}: max rel err {e:.3g} > {TOL_BF16}"
        if one_ulp:
            assert e <= TOL_BF16_ULP, f"{what}: max rel err {e:.3g} > one bf16 ulp"
    else:
        assert e <= TOL_F32, f"{what}: max rel err {e:.3g} > {TOL_F32}"
    return e


def rounded(ref64: np.ndarray, like: np.ndarray) -> np.ndarray:
    """The oracle's value stored in the storage dtype of `like`."""
    if like.dtype == np.uint8:
        return oracle.round_fp8(ref64)
    return oracle.round_bf16(ref64) if like.dtype == np.uint16 else oracle.round_f32(ref64)
