"""Seeded synthetic workloads for the Hyper-Connections residual path.

This module only draws random inputs and packs them into storage types; it
holds none of the method's arithmetic.  Both the GPU path and the CPU oracle
are fed from it, so that they see the same values.

Recipe.  Every random tensor is drawn from numpy's PCG64 with
``SeedSequence([seed, tensor_id, chunk])``, one chunk per 256 tokens, as
``standard_normal(dtype=float32)`` and then scaled.  A token's values depend
only on (seed, tensor, token), so any subset of tokens can be regenerated on
its own (the sampled checks at full size rely on that).  bf16 tensors are the
fp32 draw rounded to nearest-even bf16 and are held as ``uint16`` bit patterns
on the host; fp8 tensors (E4M3, the OCP 8-bit float with 3 mantissa bits) are
the draw rounded to the nearest code, ties to even, held as ``uint8``.

The weight record of a token has K = 2n + n^2 fp32 entries laid out as
``[alpha_0..alpha_{n-1} | beta_0..beta_{n-1} | A row-major]``; the identity
record is alpha = e_0, beta = 1, A = I (the streams start as copies of one and
the layer reduces to an ordinary residual, per the explainer
"Tencent open-sources Hy4 Preview at 770B -- Identity Hyper-Connections",
section "Jargon", identity initialization).

Workloads (hidden width, token counts and distributions are synthetic; the
pages publish no hidden width and no dataset):

==================  =====  =  ====  =====  =====================================
name                T      n  d     dtype  weights
==================  =====  =  ====  =====  =====================================
tiny-f32            256    4  1024  f32    static identity + N(0, 0.02)
static-bf16         8192   4  4096  bf16   static identity + N(0, 0.05)
dynamic-bf16        16384  4  4096  bf16   per token: W ~ N(0, 0.02), scale 0.01
mhc-bf16            32768  4  4096  bf16   per token logits ~ N(0, 1), 20 iters
chain-bf16 (x78)    4096   4  6144  bf16   per layer identity + N(0, 0.02)
decode-bf16 (x78)   64     4  8192  bf16   per layer identity + N(0, 0.02)
static-fp8          16384  4  4096  fp8    static identity + N(0, 0.05)
dynamic-fp8         16384  4  4096  fp8    as dynamic-bf16, H, F and W in FP8
==================  =====  =  ====  =====  =====================================

The decode workload is the explainer's worked shape (section "What four
streams cost per token"): 64 tokens in flight, hidden width 8192, four
streams, about 4 MB of residual state.
"""
from __future__ import annotations

import dataclasses

import numpy as np

CHUNK = 256

# tensor ids inside SeedSequence([seed, tensor_id, chunk])
TID_H, TID_F, TID_W, TID_GAMMA, TID_PROJ, TID_LOGITS, TID_X = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    n: int
    d: int
    dtype: str            # "f32" | "bf16" | "fp8"
    seed: int
    kind: str             # "static" | "dynamic" | "mhc" | "chain"
    weight_sd: float = 0.0
    gamma_sd: float = 0.0  # 0 -> gamma = 1
    proj_sd: float = 0.0
    scale: float = 0.0
    iters: int = 0
    layers: int = 1
    eps: float = 1e-6
    F_kind: str = "normal"  # "normal" (given) | "tanh" (block = tanh of its input)

    @property
    def K(self) -> int:
        return 2 * self.n + self.n * self.n

    @property
    def elem_bytes(self) -> int:
        return {"f32": 4, "bf16": 2, "fp8": 1}[self.dtype]


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny-f32", 256, 4, 1024, "f32", 101, "static", weight_sd=0.02, F_kind="tanh"),
        Workload("static-bf16", 8192, 4, 4096, "bf16", 202, "static", weight_sd=0.05, gamma_sd=0.1),
        Workload("dynamic-bf16", 16384, 4, 4096, "bf16", 303, "dynamic", gamma_sd=0.1,
                 proj_sd=0.02, scale=0.01),
        Workload("mhc-bf16", 32768, 4, 4096, "bf16", 404, "mhc", gamma_sd=0.1, iters=20),
        Workload("chain-bf16", 4096, 4, 6144, "bf16", 505, "chain", weight_sd=0.02, layers=78,
                 F_kind="tanh"),
        Workload("decode-bf16", 64, 4, 8192, "bf16", 606, "chain", weight_sd=0.02, layers=78,
                 F_kind="tanh"),
        Workload("static-fp8", 16384, 4, 4096, "fp8", 707, "static", weight_sd=0.05, gamma_sd=0.1),
        Workload("dynamic-fp8", 16384, 4, 4096, "fp8", 808, "dynamic", gamma_sd=0.1,
                 proj_sd=0.02, scale=0.01),
    ]
}


def workload(name: str, **overrides) -> Workload:
    """A named workload, optionally with fields replaced (e.g. a smaller T)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


# ------------------------------------------------------------------ storage

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _fp8_table() -> np.ndarray:
    """Values of the FP8 E4M3 codes 0..126 (the non-negative finite ones), in
    increasing order: subnormals m * 2^-9, normals (1 + m/8) * 2^(e-7)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, np.ldexp(m, -9), np.ldexp(8 + m, e - 10)).astype(np.float64)


_FP8_VALUES = _fp8_table()


def f32_to_fp8_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to FP8 E4M3 (nearest, ties to the even code), saturating
    at +-448; NaN -> 0x7F.  Returns uint8 codes."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    a = np.minimum(np.abs(x.astype(np.float64)), 448.0)
    a = np.where(np.isnan(a), 0.0, a)
    hi = np.clip(np.searchsorted(_FP8_VALUES, a), 1, 126)
    lo = hi - 1
    dlo, dhi = a - _FP8_VALUES[lo], _FP8_VALUES[hi] - a
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    code[np.isnan(x)] = 0x7F
    return code


def fp8_bits_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    v = _FP8_VALUES[np.minimum(b & 0x7F, 126)].astype(np.float32)
    v[(b & 0x7F) == 0x7F] = np.nan
    return np.where(b & 0x80, -v, v).astype(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp8":
        return f32_to_fp8_bits(x)
    return np.ascontiguousarray(x, np.float32)


def identity_record(n: int) -> np.ndarray:
    """alpha = e_0, beta = 1, A = I as one fp32 weight record."""
    rec = np.zeros(2 * n + n * n, np.float32)
    rec[0] = 1.0
    rec[n:2 * n] = 1.0
    rec[2 * n:] = np.eye(n, dtype=np.float32).reshape(-1)
    return rec


# --------------------------------------------------------------- generators

def _rng(seed: int, tensor_id: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, chunk])))


def normal_rows(seed: int, tensor_id: int, T: int, row_shape: tuple, sd: float = 1.0,
                tokens: np.ndarray | None = None) -> np.ndarray:
    """float32 N(0, sd^2) values, one row of ``row_shape`` per token.

    ``tokens`` (optional, any order) selects a subset; row t is identical to
    row t of the full draw."""
    row = int(np.prod(row_shape)) if row_shape else 1
    idx = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    out = np.empty((len(idx), row), np.float32)
    if len(idx) == 0:
        return out.reshape((0,) + tuple(row_shape))
    chunks = idx // CHUNK
    for c in np.unique(chunks):
        nt = min(CHUNK, T - c * CHUNK)
        draw = _rng(seed, tensor_id, int(c)).standard_normal(nt * row, dtype=np.float32)
        draw = draw.reshape(nt, row)
        sel = np.nonzero(chunks == c)[0]
        out[sel] = draw[idx[sel] - c * CHUNK]
    if sd != 1.0:
        out *= np.float32(sd)
    return out.reshape((len(idx),) + tuple(row_shape))


def static_record(wl: Workload, layer: int | None = None) -> np.ndarray:
    """Identity record plus N(0, weight_sd) on every entry (fp32)."""
    seed = wl.seed if layer is None else wl.seed * 1000 + layer
    noise = _rng(seed, TID_W, 0).standard_normal(wl.K, dtype=np.float32) * np.float32(wl.weight_sd)
    return identity_record(wl.n) + noise


def gamma(wl: Workload) -> np.ndarray:
    if wl.gamma_sd == 0.0:
        return np.ones(wl.d, np.float32)
    g = _rng(wl.seed, TID_GAMMA, 0).standard_normal(wl.d, dtype=np.float32)
    return np.float32(1.0) + g * np.float32(wl.gamma_sd)


def make_inputs(wl: Workload, tokens: np.ndarray | None = None) -> dict:
    """Host inputs of one workload (all tokens, or the given subset).

    Returns storage arrays (float32 or uint16 bf16 bits) and fp32 parameters:
      H (T, n, d); F (T, d) when given; w (K,) static record or (T, K) logits
      for mHC; W (K, d) projection and w_static (K,) for dynamic weights;
      gamma (d,).  For the chain workload H is n copies of one x."""
    T, n, d = wl.T, wl.n, wl.d
    out = {"gamma": gamma(wl)}
    if wl.kind == "chain":
        x = normal_rows(wl.seed, TID_X, T, (d,), tokens=tokens)
        out["H"] = to_storage(np.repeat(x[:, None, :], n, axis=1), wl.dtype)
        return out
    out["H"] = to_storage(normal_rows(wl.seed, TID_H, T, (n, d), tokens=tokens), wl.dtype)
    if wl.F_kind == "normal":
        out["F"] = to_storage(normal_rows(wl.seed, TID_F, T, (d,), tokens=tokens), wl.dtype)
    if wl.kind == "static":
        out["w"] = static_record(wl)
    elif wl.kind == "dynamic":
        out["W"] = to_storage(normal_rows(wl.seed, TID_PROJ, wl.K, (d,), sd=wl.proj_sd), wl.dtype)
        out["w_static"] = identity_record(n)
    elif wl.kind == "mhc":
        out["logits"] = normal_rows(wl.seed, TID_LOGITS, T, (wl.K,), tokens=tokens)
    return out


def layer_record(wl: Workload, layer: int) -> np.ndarray:
    """Per-layer static record of the chain workload (seeded per layer)."""
    return static_record(wl, layer)
