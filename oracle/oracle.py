"""ctypes front end of the fp64 CPU oracle (``hc_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Loaded by the test suite, the smoke check and the
benchmark's CPU-baseline leg; the GPU library never imports it and it never
imports the GPU library.

Arrays are numpy arrays on the host.  Storage tensors (H, F, W, u) are passed
in their storage type: ``np.float32`` for fp32, ``np.uint16`` holding bf16 bit
patterns or ``np.uint8`` holding FP8 E4M3 codes; ``np.float64`` passes values
that were never rounded to a storage format (the pure fp64 chain).  Weight
records, gains and logits are ``np.float64`` (callers widen fp32 values
exactly).  Every result is returned unrounded in float64;
``round_bf16`` / ``round_f32`` model a store to the storage type.

Which passage each function follows is stated in ``hc_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hc_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

F32, BF16, FP8, F64 = 0, 1, 2, 3

_lib = None


def build() -> str:
    """Compile ``liboracle.so`` with gcc (no HIP headers, no GPU code)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
         "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def load():
    """Load the built library, building it first only if nothing is built."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("HC_ORACLE_SO")   # the mutation tests load planted-bug builds
    if path is None:
        path = _SO
        if not os.path.exists(path):
            build()
    lib = ctypes.CDLL(path)
    vp, dp, i64, i32, dbl = (ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                             ctypes.c_int64, ctypes.c_int, ctypes.c_double)
    lib.orc_pre_mix.argtypes = [vp, i32, dp, i64, dp, dbl, dp, i64, i32, i32]
    lib.orc_post_mix.argtypes = [vp, vp, i32, dp, i64, dp, i64, i32, i32]
    lib.orc_weights.argtypes = [vp, vp, i32, dp, dbl, dbl, i32, dp, i64, i32, i32]
    lib.orc_sinkhorn.argtypes = [dp, dp, i32, i64, i32]
    lib.orc_block_tanh.argtypes = [vp, i32, dp, i64]
    lib.orc_round_bf16_array.argtypes = [dp, ctypes.POINTER(ctypes.c_uint16), i64]
    lib.orc_round_f32_array.argtypes = [dp, ctypes.POINTER(ctypes.c_float), i64]
    lib.orc_round_fp8_array.argtypes = [dp, ctypes.POINTER(ctypes.c_uint8), i64]
    lib.orc_widen_array.argtypes = [vp, i32, dp, i64]
    lib.orc_post_mix_backward.argtypes = [vp, vp, vp, i32, dp, i64, dp, dp, dp, i64, i32, i32]
    lib.orc_pre_mix_backward.argtypes = [vp, vp, i32, dp, i64, dp, dbl, dp, dp, dp, dp, i64, i32, i32]
    lib.orc_sinkhorn_backward.argtypes = [dp, dp, dp, i32, i64, i32]
    lib.orc_weights_backward.argtypes = [vp, vp, i32, dp, dbl, dbl, i32, dp, dp, dp, dp, i64, i32, i32]
    lib.orc_round_bf16.argtypes = [dbl]
    lib.orc_round_bf16.restype = ctypes.c_uint16
    lib.orc_set_threads.argtypes = [i32]
    lib.orc_get_threads.restype = i32
    for f in ("orc_pre_mix", "orc_post_mix", "orc_weights", "orc_sinkhorn",
              "orc_post_mix_backward", "orc_pre_mix_backward", "orc_sinkhorn_backward",
              "orc_weights_backward",
              "orc_block_tanh", "orc_round_bf16_array", "orc_round_f32_array", "orc_round_fp8_array",
              "orc_widen_array", "orc_set_threads"):
        getattr(lib, f).restype = None
    _lib = lib
    return lib


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return FP8
    if a.dtype == np.float64:
        return F64     # unrounded values (the pure fp64 chain)
    raise TypeError(f"storage arrays must be float32, uint16 (bf16 bits), uint8 (fp8 e4m3 "
                    f"codes) or float64 (unrounded), got {a.dtype}")


def _c(a: np.ndarray, dtype=None) -> np.ndarray:
    if dtype is not None:
        a = np.asarray(a, dtype=dtype)
    return np.ascontiguousarray(a)


def _dp(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _record(w: np.ndarray, T: int, K: int):
    """Weight records: shape (K,) is shared by all tokens (stride 0),
    shape (T, K) is one record per token (stride K)."""
    w = _c(w, np.float64)
    if w.shape == (K,):
        return w, 0
    if w.shape == (T, K):
        return w, K
    raise ValueError(f"weight record must be ({K},) or ({T}, {K}), got {w.shape}")


def set_threads(n: int) -> None:
    load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(load().orc_get_threads())


def pre_mix(H: np.ndarray, w: np.ndarray, gamma: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """u = RMSNorm_gamma(sum_i alpha_i H_i); H (T, n, d) -> u (T, d) float64."""
    lib = load()
    H = _c(H)
    T, n, d = H.shape
    K = 2 * n + n * n
    w, ws = _record(w, T, K)
    gamma = _c(gamma, np.float64)
    assert gamma.shape == (d,)
    u = np.empty((T, d), np.float64)
    lib.orc_pre_mix(H.ctypes.data, _dt(H), _dp(w), ws, _dp(gamma), float(eps), _dp(u), T, n, d)
    return u


def post_mix(H: np.ndarray, F: np.ndarray, w: np.ndarray) -> np.ndarray:
    """H'_i = sum_j A[i][j] H_j + beta_i F; H (T, n, d), F (T, d) -> (T, n, d) float64."""
    lib = load()
    H, F = _c(H), _c(F)
    T, n, d = H.shape
    assert F.shape == (T, d) and F.dtype == H.dtype
    K = 2 * n + n * n
    w, ws = _record(w, T, K)
    out = np.empty((T, n, d), np.float64)
    lib.orc_post_mix(H.ctypes.data, F.ctypes.data, _dt(H), _dp(w), ws, _dp(out), T, n, d)
    return out


def weights(H: np.ndarray, W: np.ndarray, w_static: np.ndarray, scale: float,
            eps: float = 1e-6, iters: int = 0) -> np.ndarray:
    """Per-token weight records from the streams; W has shape (K, d)."""
    lib = load()
    H, W = _c(H), _c(W)
    T, n, d = H.shape
    K = 2 * n + n * n
    assert W.shape == (K, d) and W.dtype == H.dtype
    ws = _c(w_static, np.float64)
    assert ws.shape == (K,)
    out = np.empty((T, K), np.float64)
    lib.orc_weights(H.ctypes.data, W.ctypes.data, _dt(H), _dp(ws), float(scale), float(eps),
                    int(iters), _dp(out), T, n, d)
    return out


def sinkhorn(logits: np.ndarray, n: int, iters: int) -> np.ndarray:
    """mHC transform of per-token logit records (T, K) -> weight records (T, K)."""
    lib = load()
    lg = _c(logits, np.float64)
    K = 2 * n + n * n
    T = lg.shape[0]
    assert lg.shape == (T, K)
    out = np.empty((T, K), np.float64)
    lib.orc_sinkhorn(_dp(lg), _dp(out), int(iters), T, n)
    return out


def block_tanh(u: np.ndarray) -> np.ndarray:
    """Stand-in block F = tanh(u), unrounded float64, same shape as u."""
    lib = load()
    u = _c(u)
    out = np.empty(u.shape, np.float64)
    lib.orc_block_tanh(u.ctypes.data, _dt(u), _dp(out), u.size)
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); returns uint16 bits."""
    lib = load()
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib.orc_round_bf16_array(_dp(x), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), x.size)
    return out


def round_fp8(x: np.ndarray) -> np.ndarray:
    """Round float64 values to FP8 E4M3 (nearest even, saturating at +-448);
    returns uint8 codes."""
    lib = load()
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint8)
    lib.orc_round_fp8_array(_dp(x), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), x.size)
    return out


def round_f32(x: np.ndarray) -> np.ndarray:
    lib = load()
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.float32)
    lib.orc_round_f32_array(_dp(x), out.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), x.size)
    return out


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a storage array (float32, bf16 bits or fp8 codes)."""
    lib = load()
    x = _c(x)
    out = np.empty(x.shape, np.float64)
    lib.orc_widen_array(x.ctypes.data, _dt(x), _dp(out), x.size)
    return out


def post_mix_backward(dHo: np.ndarray, H: np.ndarray, F: np.ndarray, w: np.ndarray):
    """Gradients of post given dL/dH': returns (dH, dF, dw) in float64; dw is
    one gradient record per token [dalpha (0) | dbeta | dA]."""
    lib = load()
    dHo, H, F = _c(dHo), _c(H), _c(F)
    T, n, d = H.shape
    assert dHo.shape == H.shape and F.shape == (T, d) and dHo.dtype == H.dtype == F.dtype
    K = 2 * n + n * n
    w, ws = _record(w, T, K)
    dH = np.empty((T, n, d), np.float64)
    dF = np.empty((T, d), np.float64)
    dw = np.empty((T, K), np.float64)
    lib.orc_post_mix_backward(dHo.ctypes.data, H.ctypes.data, F.ctypes.data, _dt(H), _dp(w), ws,
                              _dp(dH), _dp(dF), _dp(dw), T, n, d)
    return dH, dF, dw


def pre_mix_backward(du: np.ndarray, H: np.ndarray, w: np.ndarray, gamma: np.ndarray,
                     eps: float = 1e-6, dH_in: np.ndarray | None = None):
    """Gradients of pre given dL/du: returns (dH, dw, dgamma) in float64; dH
    includes dH_in when given; dw is one record per token [dalpha | 0 | 0];
    dgamma is summed over tokens."""
    lib = load()
    du, H = _c(du), _c(H)
    T, n, d = H.shape
    assert du.shape == (T, d) and du.dtype == H.dtype
    K = 2 * n + n * n
    w, ws = _record(w, T, K)
    gamma = _c(gamma, np.float64)
    dH = np.empty((T, n, d), np.float64)
    dw = np.empty((T, K), np.float64)
    dg = np.empty(d, np.float64)
    acc = None
    if dH_in is not None:
        acc = _c(dH_in, np.float64)
        assert acc.shape == (T, n, d)
    lib.orc_pre_mix_backward(du.ctypes.data, H.ctypes.data, _dt(H), _dp(w), ws, _dp(gamma),
                             float(eps), _dp(acc) if acc is not None else None, _dp(dH), _dp(dw),
                             _dp(dg), T, n, d)
    return dH, dw, dg


def sinkhorn_backward(logits: np.ndarray, dw: np.ndarray, n: int, iters: int) -> np.ndarray:
    """Gradient of the mHC transform: dL/dlogits (T, K) from dL/dw (T, K)."""
    lib = load()
    lg, g = _c(logits, np.float64), _c(dw, np.float64)
    K = 2 * n + n * n
    T = lg.shape[0]
    assert lg.shape == (T, K) and g.shape == (T, K)
    out = np.empty((T, K), np.float64)
    lib.orc_sinkhorn_backward(_dp(lg), _dp(g), _dp(out), int(iters), T, n)
    return out


def weights_backward(H: np.ndarray, W: np.ndarray, w_static: np.ndarray, scale: float,
                     dw: np.ndarray, eps: float = 1e-6, iters: int = 0):
    """Gradients of `weights` given dL/dw (T, K): returns (dH (T, n, d),
    dW (K, d), dw_static (K,)) in float64; dH is this path's part only."""
    lib = load()
    H, W = _c(H), _c(W)
    T, n, d = H.shape
    K = 2 * n + n * n
    assert W.shape == (K, d) and W.dtype == H.dtype
    ws = _c(w_static, np.float64)
    g = _c(dw, np.float64)
    assert ws.shape == (K,) and g.shape == (T, K)
    dH = np.empty((T, n, d), np.float64)
    dW = np.empty((K, d), np.float64)
    dws = np.empty(K, np.float64)
    lib.orc_weights_backward(H.ctypes.data, W.ctypes.data, _dt(H), _dp(ws), float(scale), float(eps),
                             int(iters), _dp(g), _dp(dH), _dp(dW), _dp(dws), T, n, d)
    return dH, dW, dws
