"""Thin ctypes binding of libhc.so (declared in include/hc.h).

Argument marshalling only: every function checks the torch tensors it is
given (device, dtype, contiguity, shape), passes raw device pointers and the
current HIP stream to the C entry point of the same name, and raises
``HCError`` with the library's status text when the call is rejected.  All
work runs in the library's kernels; there is no CPU fallback, and the module
raises on first use if the library is not built.

Tensor conventions (storage dtype torch.float32, torch.bfloat16 or
torch.float8_e4m3fn; the last for pre_mix, post_mix, post_pre_mix and
block_tanh only):
  H      (T, n, d)      residual streams
  u, F   (T, d)         block input / block output
  w      (K,) float32   one weight record shared by all tokens, or
         (T, K) float32 one record per token; K = 2n + n^2 laid out as
                        [alpha (n) | beta (n) | A (n x n, row-major)]
  gamma  (d,) float32   RMSNorm gain
  W      (K, d)         projection for per-token weights
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HC_LIB names another build of the same library (the sanitizer test loads
# one whose host code is built with AddressSanitizer); there is no fallback
LIB_PATH = os.environ.get("HC_LIB") or os.path.join(_PKG, "libhc.so")

HC_F32, HC_BF16, HC_FP8 = 0, 1, 2
MAX_STREAMS = 4
MAX_HIDDEN = 16384
MAX_SINKHORN_ITERS = 10000

# (name, argtypes); every entry point returns hc_status (int)
_vp, _fp = ctypes.c_void_p, ctypes.c_void_p
_i64, _i32, _f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
_SIGS = {
    "hc_pre_mix": [_vp, _fp, _i64, _fp, _f32, _vp, _i64, _i32, _i32, _i32, _vp],
    "hc_post_mix": [_vp, _vp, _fp, _i64, _vp, _i64, _i32, _i32, _i32, _vp],
    "hc_post_pre_mix": [_vp, _vp, _fp, _i64, _fp, _i64, _fp, _f32, _vp, _vp, _i64, _i32, _i32,
                        _i32, _vp],
    "hc_weights": [_vp, _vp, _fp, _f32, _f32, _i32, _fp, _i64, _i32, _i32, _i32, _vp],
    "hc_sinkhorn": [_fp, _fp, _i32, _i64, _i32, _vp],
    "hc_block_tanh": [_vp, _vp, _i64, _i32, _vp],
    "hc_post_mix_backward": [_vp, _vp, _vp, _fp, _i64, _vp, _vp, _fp, _vp, _i64, _i64, _i32, _i32,
                             _i32, _vp],
    "hc_pre_mix_backward": [_vp, _vp, _fp, _i64, _fp, _f32, _vp, _vp, _vp, _fp, _fp, _vp, _i64,
                            _i64, _i32, _i32, _i32, _vp],
    "hc_post_pre_mix_backward": [_vp, _vp, _vp, _vp, _fp, _i64, _fp, _i64, _fp, _f32, _vp, _vp,
                                 _fp, _fp, _fp, _vp, _i64, _i64, _i32, _i32, _i32, _vp],
    "hc_post_pre_mix_backward_terms": [_vp, _vp, _vp, _vp, _fp, _i64, _fp, _i64, _fp, _f32, _fp,
                                       _fp, _vp, _vp, _fp, _fp, _fp, _vp, _i64, _i64, _i32, _i32,
                                       _i32, _vp],
    "hc_weights_backward_terms": [_vp, _vp, _fp, _f32, _f32, _i32, _fp, _fp, _fp, _fp, _fp, _fp,
                                  _fp, _vp, _i64, _i64, _i32, _i32, _i32, _vp],
    "hc_sum_records": [_fp, _i64, _i32, _fp, _vp],
    "hc_weights_save": [_vp, _vp, _fp, _f32, _f32, _i32, _fp, _fp, _i64, _i64, _i32, _i32, _i32,
                        _vp],
    "hc_weights_backward": [_vp, _vp, _fp, _f32, _f32, _i32, _fp, _fp, _fp, _vp, _vp, _fp, _fp,
                            _vp, _i64, _i64, _i32, _i32, _i32, _vp],
    "hc_sinkhorn_backward": [_fp, _fp, _fp, _fp, _i32, _vp, _i64, _i64, _i32, _vp],
    "hc_post_mix_weights": [_vp, _vp, _fp, _i64, _vp, _fp, _f32, _f32, _i32, _vp, _fp, _fp, _i64,
                            _i64, _i32, _i32, _i32, _vp],
    "hc_post_mix_backward_noalloc": [_vp, _vp, _vp, _fp, _i64, _vp, _vp, _fp, _i64, _i32, _i32,
                                     _i32, _vp],
    "hc_post_weights_pre_mix": [_vp, _vp, _fp, _i64, _vp, _fp, _f32, _f32, _i32, _fp, _f32, _vp,
                                _fp, _vp, _fp, _i64, _i64, _i32, _i32, _i32, _vp],
}
EXPORTS = tuple(_SIGS) + ("hc_status_str", "hc_abi_version", "hc_backward_workspace",
                          "hc_weights_backward_workspace", "hc_sinkhorn_backward_workspace",
                          "hc_weights_saved_bytes")

_lib = None


class HCError(RuntimeError):
    def __init__(self, func: str, status: int, text: str):
        super().__init__(f"{func}: {text}")
        self.func, self.status = func, status


def lib() -> ctypes.CDLL:
    """Load libhc.so once; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built: run `python -m hyper_connections_amd.build`; "
                "there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.hc_status_str.argtypes = [ctypes.c_int]
        L.hc_status_str.restype = ctypes.c_char_p
        L.hc_abi_version.argtypes = []
        L.hc_abi_version.restype = ctypes.c_int32
        L.hc_backward_workspace.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
        L.hc_backward_workspace.restype = ctypes.c_int64
        L.hc_weights_backward_workspace.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                                    ctypes.c_int32]
        L.hc_weights_backward_workspace.restype = ctypes.c_int64
        L.hc_sinkhorn_backward_workspace.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.hc_sinkhorn_backward_workspace.restype = ctypes.c_int64
        L.hc_weights_saved_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32]
        L.hc_weights_saved_bytes.restype = ctypes.c_int64
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().hc_status_str(int(status)).decode()


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise HCError(name, st, status_str(st))


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on_launch_stream(fn):
    """Give `fn` its launch stream as the current stream.  Everything the
    wrapper allocates (outputs, workspaces) then belongs to the stream its
    kernels run on, so torch's caching allocator cannot hand that memory to
    other work before those kernels are done.  `stream` may be a
    torch.cuda.Stream or a raw hipStream_t handle; None means the current
    stream."""
    pos = list(inspect.signature(fn).parameters).index("stream")

    @functools.wraps(fn)
    def wrapper(*args, **kwargs):
        if len(args) > pos:
            stream, args = args[pos], args[:pos] + (None,) + args[pos + 1:]
        else:
            stream = kwargs.pop("stream", None)
        if stream is None:
            return fn(*args, **kwargs)
        s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(s):
            return fn(*args, **kwargs)
    return wrapper


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HC_BF16
    if t.dtype == torch.float8_e4m3fn:
        return HC_FP8
    if t.dtype == torch.float32:
        return HC_F32
    raise TypeError(f"storage dtype must be float8_e4m3fn, bfloat16 or float32, got {t.dtype}")


def _dev(t: torch.Tensor, what: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on a GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _record(w: torch.Tensor, T: int, K: int, what: str = "w") -> int:
    """Validate a weight-record tensor; returns its token stride."""
    _dev(w, what)
    if w.dtype != torch.float32:
        raise TypeError(f"{what} must be float32")
    if tuple(w.shape) == (K,):
        return 0
    if tuple(w.shape) == (T, K):
        return K
    raise ValueError(f"{what} must have shape ({K},) or ({T}, {K}), got {tuple(w.shape)}")


def _H(H: torch.Tensor):
    _dev(H, "H")
    if H.dim() != 3:
        raise ValueError(f"H must be (T, n, d), got {tuple(H.shape)}")
    T, n, d = H.shape
    return T, n, d, 2 * n + n * n


@_on_launch_stream
def pre_mix(H, w, gamma, eps: float = 1e-6, out=None, stream=None) -> torch.Tensor:
    """Block input u = RMSNorm_gamma(sum_i alpha_i H_i), shape (T, d)."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    _dev(gamma, "gamma")
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (d,):
        raise ValueError("gamma must be float32 of shape (d,)")
    u = torch.empty((T, d), dtype=H.dtype, device=H.device) if out is None else _dev(out, "out")
    if u.dtype != H.dtype or tuple(u.shape) != (T, d):
        raise ValueError("out must match H's dtype and have shape (T, d)")
    _call("hc_pre_mix", H.data_ptr(), w.data_ptr(), ws, gamma.data_ptr(), float(eps), u.data_ptr(),
          T, n, d, _dt(H), _stream(stream))
    return u


@_on_launch_stream
def post_mix(H, F, w, out=None, stream=None) -> torch.Tensor:
    """H'_i = sum_j A[i][j] H_j + beta_i F, shape (T, n, d).  ``out=H`` runs in place."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    _dev(F, "F")
    if F.dtype != H.dtype or tuple(F.shape) != (T, d):
        raise ValueError("F must match H's dtype and have shape (T, d)")
    o = torch.empty_like(H) if out is None else _dev(out, "out")
    if o.dtype != H.dtype or o.shape != H.shape:
        raise ValueError("out must match H")
    _call("hc_post_mix", H.data_ptr(), F.data_ptr(), w.data_ptr(), ws, o.data_ptr(), T, n, d,
          _dt(H), _stream(stream))
    return o


@_on_launch_stream
def post_pre_mix(H, F, w, w_next, gamma_next, eps: float = 1e-6, out=None, u_out=None,
                 stream=None):
    """Fused write-back of one layer and read-mix + RMSNorm of the next.
    Returns (H', u_next); bitwise equal to post_mix followed by pre_mix."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    ws2 = _record(w_next, T, K, "w_next")
    _dev(F, "F")
    _dev(gamma_next, "gamma_next")
    if F.dtype != H.dtype or tuple(F.shape) != (T, d):
        raise ValueError("F must match H's dtype and have shape (T, d)")
    if gamma_next.dtype != torch.float32 or tuple(gamma_next.shape) != (d,):
        raise ValueError("gamma_next must be float32 of shape (d,)")
    o = torch.empty_like(H) if out is None else _dev(out, "out")
    u = torch.empty((T, d), dtype=H.dtype, device=H.device) if u_out is None else _dev(u_out, "u_out")
    if o.dtype != H.dtype or o.shape != H.shape or u.dtype != H.dtype or tuple(u.shape) != (T, d):
        raise ValueError("out / u_out do not match H")
    _call("hc_post_pre_mix", H.data_ptr(), F.data_ptr(), w.data_ptr(), ws, w_next.data_ptr(), ws2,
          gamma_next.data_ptr(), float(eps), o.data_ptr(), u.data_ptr(), T, n, d, _dt(H),
          _stream(stream))
    return o, u


def _weights_args(H, W, w_static, out):
    T, n, d, K = _H(H)
    _dev(W, "W")
    if W.dtype != H.dtype or tuple(W.shape) != (K, d):
        raise ValueError(f"W must match H's dtype and have shape ({K}, {d})")
    _dev(w_static, "w_static")
    if w_static.dtype != torch.float32 or tuple(w_static.shape) != (K,):
        raise ValueError(f"w_static must be float32 of shape ({K},)")
    o = torch.empty((T, K), dtype=torch.float32, device=H.device) if out is None else _dev(out, "out")
    if o.dtype != torch.float32 or tuple(o.shape) != (T, K):
        raise ValueError(f"out must be float32 of shape ({T}, {K})")
    return T, n, d, K, o


@_on_launch_stream
def weights(H, W, w_static, scale: float, eps: float = 1e-6, sinkhorn_iters: int = 0,
            out=None, stream=None) -> torch.Tensor:
    """Per-token weight records (T, K) float32 from the streams (see include/hc.h)."""
    T, n, d, K, o = _weights_args(H, W, w_static, out)
    _call("hc_weights", H.data_ptr(), W.data_ptr(), w_static.data_ptr(), float(scale), float(eps),
          int(sinkhorn_iters), o.data_ptr(), T, n, d, _dt(H), _stream(stream))
    return o


@_on_launch_stream
def weights_save(H, W, w_static, scale: float, eps: float = 1e-6, sinkhorn_iters: int = 0,
                 out=None, saved=None, stream=None):
    """weights() for a training forward: returns (records, saved), where saved
    (a float32 device buffer of hc_weights_saved_bytes) holds what
    weights_backward(..., saved=saved) would otherwise recompute."""
    T, n, d, K, o = _weights_args(H, W, w_static, out)
    need = int(lib().hc_weights_saved_bytes(T, n))
    if saved is None:
        saved = torch.empty(max(need, 16) // 4, dtype=torch.float32, device=H.device)
    _dev(saved, "saved")
    if saved.dtype != torch.float32:
        raise ValueError("saved must be float32")
    _call("hc_weights_save", H.data_ptr(), W.data_ptr(), w_static.data_ptr(), float(scale),
          float(eps), int(sinkhorn_iters), o.data_ptr(), saved.data_ptr(),
          saved.numel() * 4, T, n, d, _dt(H), _stream(stream))
    return o, saved


@_on_launch_stream
def post_mix_weights(H, F, w, W, w_static, scale: float, eps: float = 1e-6,
                     sinkhorn_iters: int = 0, out=None, w_out=None, saved=None, stream=None):
    """The write-back of one layer fused with the next layer's per-token
    weights: returns (H', w_next), H' = post_mix(H, F, w) (bitwise) and
    w_next = weights(H', W, w_static, scale, eps, sinkhorn_iters) formed from
    H' while it is on chip.  ``out=H`` runs in place.  ``saved`` (True, or a
    float32 buffer of hc_weights_saved_bytes) also keeps the projections and
    norms for weights_backward, and the result is (H', w_next, saved).
    bf16 and FP8 storage, d <= 4096."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    _dev(F, "F")
    if F.dtype != H.dtype or tuple(F.shape) != (T, d):
        raise ValueError("F must match H's dtype and have shape (T, d)")
    o = torch.empty_like(H) if out is None else _dev(out, "out")
    if o.dtype != H.dtype or o.shape != H.shape:
        raise ValueError("out must match H")
    W_, ro = W, w_out
    T2, n2, d2, K2, ro = _weights_args(H, W_, w_static, ro)
    keep = saved is not None and saved is not False
    if saved is True:
        saved = torch.empty(max(int(lib().hc_weights_saved_bytes(T, n)), 16) // 4,
                            dtype=torch.float32, device=H.device)
    if keep:
        _dev(saved, "saved")
        if saved.dtype != torch.float32:
            raise ValueError("saved must be float32")
    _call("hc_post_mix_weights", H.data_ptr(), F.data_ptr(), w.data_ptr(), ws, W.data_ptr(),
          w_static.data_ptr(), float(scale), float(eps), int(sinkhorn_iters), o.data_ptr(),
          ro.data_ptr(), saved.data_ptr() if keep else None, saved.numel() * 4 if keep else 0,
          T, n, d, _dt(H), _stream(stream))
    return (o, ro, saved) if keep else (o, ro)


@_on_launch_stream
def post_weights_pre_mix(H, F, w, W, w_static, scale: float, gamma_next, eps: float = 1e-6,
                         pre_eps: float = 1e-6, sinkhorn_iters: int = 0, out=None, w_out=None,
                         u_out=None, saved=None, stream=None):
    """The whole layer boundary in one pass: returns (H', w_next, u_next),
    H' = post_mix(H, F, w) (bitwise), w_next = the next layer's per-token
    weights from H' (as post_mix_weights), u_next = pre_mix(H', w_next,
    gamma_next, pre_eps) to one unit in the last place.  ``out=H`` runs in
    place; ``saved`` as post_mix_weights (the result then ends with it).
    bf16 and FP8 storage, d <= 4096."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    _dev(F, "F")
    if F.dtype != H.dtype or tuple(F.shape) != (T, d):
        raise ValueError("F must match H's dtype and have shape (T, d)")
    _dev(gamma_next, "gamma_next")
    if gamma_next.dtype != torch.float32 or tuple(gamma_next.shape) != (d,):
        raise ValueError("gamma_next must be float32 of shape (d,)")
    o = torch.empty_like(H) if out is None else _dev(out, "out")
    if o.dtype != H.dtype or o.shape != H.shape:
        raise ValueError("out must match H")
    u = torch.empty((T, d), dtype=H.dtype, device=H.device) if u_out is None else _dev(u_out, "u_out")
    if u.dtype != H.dtype or tuple(u.shape) != (T, d):
        raise ValueError("u_out must match H's dtype and have shape (T, d)")
    _, _, _, _, ro = _weights_args(H, W, w_static, w_out)
    keep = saved is not None and saved is not False
    if saved is True:
        saved = torch.empty(max(int(lib().hc_weights_saved_bytes(T, n)), 16) // 4,
                            dtype=torch.float32, device=H.device)
    if keep:
        _dev(saved, "saved")
        if saved.dtype != torch.float32:
            raise ValueError("saved must be float32")
    _call("hc_post_weights_pre_mix", H.data_ptr(), F.data_ptr(), w.data_ptr(), ws, W.data_ptr(),
          w_static.data_ptr(), float(scale), float(eps), int(sinkhorn_iters),
          gamma_next.data_ptr(), float(pre_eps), o.data_ptr(), ro.data_ptr(), u.data_ptr(),
          saved.data_ptr() if keep else None, saved.numel() * 4 if keep else 0, T, n, d, _dt(H),
          _stream(stream))
    return (o, ro, u, saved) if keep else (o, ro, u)


@_on_launch_stream
def sinkhorn(logits, n: int, iters: int, out=None, stream=None) -> torch.Tensor:
    """mHC transform of per-token logit records (T, K) -> weight records (T, K)."""
    _dev(logits, "logits")
    K = 2 * n + n * n
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.shape[1] != K:
        raise ValueError(f"logits must be float32 of shape (T, {K})")
    T = logits.shape[0]
    o = torch.empty_like(logits) if out is None else _dev(out, "out")
    if o.dtype != torch.float32 or o.shape != logits.shape:
        raise ValueError("out must match logits")
    _call("hc_sinkhorn", logits.data_ptr(), o.data_ptr(), int(iters), T, int(n), _stream(stream))
    return o


@_on_launch_stream
def block_tanh(u, out=None, stream=None) -> torch.Tensor:
    """Stand-in block F = tanh(u) (not part of the method)."""
    _dev(u, "u")
    F = torch.empty_like(u) if out is None else _dev(out, "out")
    if F.dtype != u.dtype or F.shape != u.shape:
        raise ValueError("out must match u")
    _call("hc_block_tanh", u.data_ptr(), F.data_ptr(), u.numel(), _dt(u), _stream(stream))
    return F


def abi_version() -> int:
    return int(lib().hc_abi_version())


def backward_workspace(T: int, n: int, d: int) -> int:
    """Bytes of workspace the backward calls need (hc_backward_workspace)."""
    return int(lib().hc_backward_workspace(int(T), int(n), int(d)))


def _workspace(ws, T, n, d, device):
    need = backward_workspace(T, n, d)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _dev(ws, "workspace")
    return ws, ws.numel() * ws.element_size()


def _grad_record(dw, T, K, ws_stride, device, what="dw"):
    shape = (K,) if ws_stride == 0 else (T, K)
    if dw is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    _dev(dw, what)
    if dw.dtype != torch.float32 or tuple(dw.shape) != shape:
        raise ValueError(f"{what} must be float32 of shape {shape} (the shape of the weights)")
    return dw


@_on_launch_stream
def post_mix_backward(dH_out, H, F, w, dH=None, dF=None, dw=None, workspace=None, stream=None,
                      h_grad=True):
    """Gradients of post_mix: returns (dH, dF, dw).  dw has the shape of the
    weights: (K,) for a shared record (summed over tokens), (T, K) for
    per-token records; entries [dalpha (0) | dbeta | dA].  With
    ``h_grad=False`` dH is not formed (None is returned for it): pass dH_out
    to pre_mix_backward(dH_out=...) instead, which adds it there."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    _dev(dH_out, "dH_out")
    _dev(F, "F")
    if dH_out.dtype != H.dtype or dH_out.shape != H.shape:
        raise ValueError("dH_out must match H")
    if F.dtype != H.dtype or tuple(F.shape) != (T, d):
        raise ValueError("F must match H's dtype and have shape (T, d)")
    if not h_grad:
        if dH is not None:
            raise ValueError("dH given with h_grad=False")
    else:
        dH = torch.empty_like(H) if dH is None else _dev(dH, "dH")
        if dH.shape != H.shape or dH.dtype != H.dtype:
            raise ValueError("dH does not match H")
    dF = torch.empty_like(F) if dF is None else _dev(dF, "dF")
    if dF.shape != F.shape or dF.dtype != F.dtype:
        raise ValueError("dF does not match F")
    dw = _grad_record(dw, T, K, ws, H.device)
    wk, wkb = (None, 0) if ws != 0 else _workspace(workspace, T, n, d, H.device)
    _call("hc_post_mix_backward", dH_out.data_ptr(), H.data_ptr(), F.data_ptr(), w.data_ptr(), ws,
          dH.data_ptr() if dH is not None else None, dF.data_ptr(), dw.data_ptr(),
          wk.data_ptr() if wk is not None else None,
          wkb, T, n, d, _dt(H), _stream(stream))
    return dH, dF, dw


@_on_launch_stream
def post_mix_backward_noalloc(dH_out, H, F, w, dH=None, dF=None, dw=None, stream=None,
                              h_grad=True):
    """post_mix_backward without a workspace: the library's own per-GPU
    scratch array holds a shared record's partial sums, so the call allocates
    nothing when the outputs are given.  Calls that overlap on one GPU race
    for that array."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    _dev(dH_out, "dH_out")
    _dev(F, "F")
    if dH_out.dtype != H.dtype or dH_out.shape != H.shape:
        raise ValueError("dH_out must match H")
    if F.dtype != H.dtype or tuple(F.shape) != (T, d):
        raise ValueError("F must match H's dtype and have shape (T, d)")
    if not h_grad:
        if dH is not None:
            raise ValueError("dH given with h_grad=False")
    else:
        dH = torch.empty_like(H) if dH is None else _dev(dH, "dH")
        if dH.shape != H.shape or dH.dtype != H.dtype:
            raise ValueError("dH does not match H")
    dF = torch.empty_like(F) if dF is None else _dev(dF, "dF")
    if dF.shape != F.shape or dF.dtype != F.dtype:
        raise ValueError("dF does not match F")
    dw = _grad_record(dw, T, K, ws, H.device)
    _call("hc_post_mix_backward_noalloc", dH_out.data_ptr(), H.data_ptr(), F.data_ptr(),
          w.data_ptr(), ws, dH.data_ptr() if dH is not None else None, dF.data_ptr(),
          dw.data_ptr(), T, n, d, _dt(H), _stream(stream))
    return dH, dF, dw


@_on_launch_stream
def pre_mix_backward(du, H, w, gamma, eps: float = 1e-6, dH_in=None, out=None, dw=None,
                     dgamma=None, workspace=None, stream=None, dH_out=None, h_grad=True,
                     g_grad=True):
    """Gradients of pre_mix: returns (dH, dw, dgamma).  dH includes dH_in when
    given (``out=dH_in`` accumulates in place), or, given dH_out (the
    gradient at post_mix's output, after post_mix_backward(h_grad=False)),
    the write-back's H gradient formed from it and the same records; dw has
    the shape of the weights ([dalpha | 0 | 0]); dgamma is summed over
    tokens.  h_grad=False computes dw and dgamma only (dH is None; no
    addend); with g_grad=False as well, dw alone (dgamma is None).  Output
    buffers and the workspace may be passed in."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    _dev(du, "du")
    _dev(gamma, "gamma")
    if du.dtype != H.dtype or tuple(du.shape) != (T, d):
        raise ValueError("du must match H's dtype and have shape (T, d)")
    if gamma.dtype != torch.float32 or tuple(gamma.shape) != (d,):
        raise ValueError("gamma must be float32 of shape (d,)")
    if dH_in is not None and dH_out is not None:
        raise ValueError("give at most one of dH_in and dH_out")
    for name, x in (("dH_in", dH_in), ("dH_out", dH_out)):
        if x is not None:
            _dev(x, name)
            if x.dtype != H.dtype or x.shape != H.shape:
                raise ValueError(f"{name} must match H")
    if h_grad:
        dH = torch.empty_like(H) if out is None else _dev(out, "out")
        if dH.dtype != H.dtype or dH.shape != H.shape:
            raise ValueError("out must match H")
    else:
        if dH_in is not None or dH_out is not None or out is not None:
            raise ValueError("h_grad=False takes no dH_in, dH_out or out")
        dH = None
    dw = _grad_record(dw, T, K, ws, H.device)
    if not g_grad and h_grad:
        raise ValueError("g_grad=False needs h_grad=False")
    if g_grad:
        dg = torch.empty(d, dtype=torch.float32, device=H.device) if dgamma is None else _dev(dgamma, "dgamma")
        if dg.dtype != torch.float32 or tuple(dg.shape) != (d,):
            raise ValueError(f"dgamma must be float32 of shape ({d},)")
    else:
        dg = None
    wk, wkb = _workspace(workspace, T, n, d, H.device)
    _call("hc_pre_mix_backward", du.data_ptr(), H.data_ptr(), w.data_ptr(), ws, gamma.data_ptr(),
          float(eps), dH_in.data_ptr() if dH_in is not None else None,
          dH_out.data_ptr() if dH_out is not None else None,
          dH.data_ptr() if dH is not None else None,
          dw.data_ptr(), dg.data_ptr() if dg is not None else None, wk.data_ptr(), wkb, T, n, d,
          _dt(H), _stream(stream))
    return dH, dw, dg


@_on_launch_stream
def post_pre_mix_backward(dH_out, du_next, H, F, w, w_next, gamma_next, eps: float = 1e-6,
                          out=None, dF=None, dw=None, dw_next=None, dgamma_next=None,
                          workspace=None, stream=None, terms=None):
    """Gradients of post_pre_mix (one layer boundary): returns (dH, dF, dw,
    dw_next, dgamma_next).  dH_out is the gradient at H' from the next layer's
    write-back (not from the read-mix, whose share is formed here from
    du_next); H' is recomputed from H, F and w.  dw ([0 | dbeta | dA]) and
    dw_next ([dalpha | 0 | 0]) have the shape of w and w_next, which must be
    both shared or both per token.  ``out=dH_out`` writes dH in place.
    ``terms=(dhbar, coef)`` from weights_backward_terms (per-token records
    only) adds the weight producer's gradient a_i dhbar + b_i H'_i at H'."""
    T, n, d, K = _H(H)
    ws = _record(w, T, K)
    ws2 = _record(w_next, T, K, "w_next")
    if ws != ws2:
        raise ValueError("w and w_next must be both shared (K,) or both per token (T, K)")
    if terms is not None:
        if ws == 0:
            raise ValueError("terms come with per-token records (T, K)")
        dhbar, coef = terms
        _dev(dhbar, "dhbar")
        _dev(coef, "coef")
        if dhbar.dtype != torch.float32 or tuple(dhbar.shape) != (T, d) or not dhbar.is_contiguous():
            raise ValueError(f"dhbar must be contiguous float32 of shape ({T}, {d})")
        if coef.dtype != torch.float32 or tuple(coef.shape) != (T, 2 * n) or not coef.is_contiguous():
            raise ValueError(f"coef must be contiguous float32 of shape ({T}, {2 * n})")
    for name, x, shape in (("dH_out", dH_out, tuple(H.shape)), ("du_next", du_next, (T, d)),
                           ("F", F, (T, d))):
        _dev(x, name)
        if x.dtype != H.dtype or tuple(x.shape) != shape:
            raise ValueError(f"{name} must match H's dtype and have shape {shape}")
    _dev(gamma_next, "gamma_next")
    if gamma_next.dtype != torch.float32 or tuple(gamma_next.shape) != (d,):
        raise ValueError("gamma_next must be float32 of shape (d,)")
    dH = torch.empty_like(H) if out is None else _dev(out, "out")
    f = torch.empty((T, d), dtype=H.dtype, device=H.device) if dF is None else _dev(dF, "dF")
    if dH.dtype != H.dtype or dH.shape != H.shape or f.dtype != H.dtype or tuple(f.shape) != (T, d):
        raise ValueError("out / dF do not match H")
    dw = _grad_record(dw, T, K, ws, H.device)
    dwn = _grad_record(dw_next, T, K, ws, H.device, "dw_next")
    dg = (torch.empty(d, dtype=torch.float32, device=H.device) if dgamma_next is None
          else _dev(dgamma_next, "dgamma_next"))
    if dg.dtype != torch.float32 or tuple(dg.shape) != (d,):
        raise ValueError(f"dgamma_next must be float32 of shape ({d},)")
    wk, wkb = _workspace(workspace, T, n, d, H.device)
    if terms is None:
        _call("hc_post_pre_mix_backward", dH_out.data_ptr(), du_next.data_ptr(), H.data_ptr(),
              F.data_ptr(), w.data_ptr(), ws, w_next.data_ptr(), ws2, gamma_next.data_ptr(),
              float(eps), dH.data_ptr(), f.data_ptr(), dw.data_ptr(), dwn.data_ptr(), dg.data_ptr(),
              wk.data_ptr(), wkb, T, n, d, _dt(H), _stream(stream))
    else:
        _call("hc_post_pre_mix_backward_terms", dH_out.data_ptr(), du_next.data_ptr(), H.data_ptr(),
              F.data_ptr(), w.data_ptr(), ws, w_next.data_ptr(), ws2, gamma_next.data_ptr(),
              float(eps), dhbar.data_ptr(), coef.data_ptr(), dH.data_ptr(), f.data_ptr(),
              dw.data_ptr(), dwn.data_ptr(), dg.data_ptr(), wk.data_ptr(), wkb, T, n, d, _dt(H),
              _stream(stream))
    return dH, f, dw, dwn, dg


@_on_launch_stream
def sum_records(rec, out=None, stream=None):
    """Sum of per-token records over tokens: (T, K) float32 -> (K,)."""
    _dev(rec, "rec")
    if rec.dtype != torch.float32 or rec.dim() != 2:
        raise ValueError("rec must be float32 of shape (T, K)")
    T, K = rec.shape
    o = torch.empty(K, dtype=torch.float32, device=rec.device) if out is None else _dev(out, "out")
    if o.dtype != torch.float32 or tuple(o.shape) != (K,):
        raise ValueError(f"out must be float32 of shape ({K},)")
    _call("hc_sum_records", rec.data_ptr(), T, K, o.data_ptr(), _stream(stream))
    return o


@_on_launch_stream
def weights_backward(H, W, w_static, scale: float, dw, eps: float = 1e-6, sinkhorn_iters: int = 0,
                     dH_in=None, out=None, dW=None, dw_static=None, workspace=None, dw2=None,
                     saved=None, stream=None):
    """Gradients of weights: returns (dH, dW, dw_static).  dw is dL/d(records)
    (T, K) float32 (plus dw2 when given, e.g. the pre and post gradients of the
    same records); dH includes dH_in when given (``out=dH_in`` accumulates in
    place); dW (K, d) and dw_static (K,) are float32.  ``saved`` is the buffer
    weights_save filled for the same H, W and eps (else recomputed)."""
    T, n, d, K = _H(H)
    _dev(W, "W")
    _dev(w_static, "w_static")
    _dev(dw, "dw")
    if W.dtype != H.dtype or tuple(W.shape) != (K, d):
        raise ValueError(f"W must match H's dtype and have shape ({K}, {d})")
    if w_static.dtype != torch.float32 or tuple(w_static.shape) != (K,):
        raise ValueError(f"w_static must be float32 of shape ({K},)")
    if dw.dtype != torch.float32 or tuple(dw.shape) != (T, K):
        raise ValueError(f"dw must be float32 of shape ({T}, {K})")
    if dw2 is not None:
        _dev(dw2, "dw2")
        if dw2.dtype != torch.float32 or tuple(dw2.shape) != (T, K):
            raise ValueError(f"dw2 must be float32 of shape ({T}, {K})")
    if dH_in is not None:
        _dev(dH_in, "dH_in")
        if dH_in.dtype != H.dtype or dH_in.shape != H.shape:
            raise ValueError("dH_in must match H")
    if saved is not None:
        _dev(saved, "saved")
        if saved.dtype != torch.float32 or saved.numel() * 4 < int(lib().hc_weights_saved_bytes(T, n)):
            raise ValueError("saved must be the float32 buffer weights_save filled")
    dH = torch.empty_like(H) if out is None else _dev(out, "out")
    if dH.dtype != H.dtype or dH.shape != H.shape:
        raise ValueError("out must match H")
    dW = torch.empty((K, d), dtype=torch.float32, device=H.device) if dW is None else _dev(dW, "dW")
    dws = (torch.empty(K, dtype=torch.float32, device=H.device) if dw_static is None
           else _dev(dw_static, "dw_static"))
    if dW.dtype != torch.float32 or tuple(dW.shape) != (K, d):
        raise ValueError(f"dW must be float32 of shape ({K}, {d})")
    if dws.dtype != torch.float32 or tuple(dws.shape) != (K,):
        raise ValueError(f"dw_static must be float32 of shape ({K},)")
    need = int(lib().hc_weights_backward_workspace(T, n, d, int(sinkhorn_iters)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=H.device)
    _dev(workspace, "workspace")
    _call("hc_weights_backward", H.data_ptr(), W.data_ptr(), w_static.data_ptr(), float(scale),
          float(eps), int(sinkhorn_iters), dw.data_ptr(),
          dw2.data_ptr() if dw2 is not None else None,
          saved.data_ptr() if saved is not None else None,
          dH_in.data_ptr() if dH_in is not None else None, dH.data_ptr(), dW.data_ptr(),
          dws.data_ptr(), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
          T, n, d, _dt(H), _stream(stream))
    return dH, dW, dws


@_on_launch_stream
def weights_backward_terms(H, W, w_static, scale: float, dw, eps: float = 1e-6,
                           sinkhorn_iters: int = 0, dhbar=None, coef=None, dW=None, dw_static=None,
                           workspace=None, dw2=None, saved=None, stream=None):
    """weights_backward without dH: returns (dhbar, coef, dW, dw_static) with
    dhbar (T, d) float32 = W^T dz per token and coef (T, 2n) float32 = (a | b),
    so that the gradient reaching stream i is a_i dhbar + b_i H_i (for
    post_pre_mix_backward(..., terms=(dhbar, coef)))."""
    T, n, d, K = _H(H)
    for name, x in (("W", W), ("w_static", w_static), ("dw", dw)):
        _dev(x, name)
    if W.dtype != H.dtype or tuple(W.shape) != (K, d):
        raise ValueError(f"W must match H's dtype and have shape ({K}, {d})")
    if w_static.dtype != torch.float32 or tuple(w_static.shape) != (K,):
        raise ValueError(f"w_static must be float32 of shape ({K},)")
    if dw.dtype != torch.float32 or tuple(dw.shape) != (T, K):
        raise ValueError(f"dw must be float32 of shape ({T}, {K})")
    if dw2 is not None:
        _dev(dw2, "dw2")
        if dw2.dtype != torch.float32 or tuple(dw2.shape) != (T, K):
            raise ValueError(f"dw2 must be float32 of shape ({T}, {K})")
    if saved is not None:
        _dev(saved, "saved")
        if saved.dtype != torch.float32 or saved.numel() * 4 < int(lib().hc_weights_saved_bytes(T, n)):
            raise ValueError("saved must be the float32 buffer weights_save filled")
    dhb = torch.empty((T, d), dtype=torch.float32, device=H.device) if dhbar is None else _dev(dhbar, "dhbar")
    co = torch.empty((T, 2 * n), dtype=torch.float32, device=H.device) if coef is None else _dev(coef, "coef")
    if dhb.dtype != torch.float32 or tuple(dhb.shape) != (T, d) or not dhb.is_contiguous():
        raise ValueError(f"dhbar must be contiguous float32 of shape ({T}, {d})")
    if co.dtype != torch.float32 or tuple(co.shape) != (T, 2 * n) or not co.is_contiguous():
        raise ValueError(f"coef must be contiguous float32 of shape ({T}, {2 * n})")
    dW = torch.empty((K, d), dtype=torch.float32, device=H.device) if dW is None else _dev(dW, "dW")
    dws = (torch.empty(K, dtype=torch.float32, device=H.device) if dw_static is None
           else _dev(dw_static, "dw_static"))
    if dW.dtype != torch.float32 or tuple(dW.shape) != (K, d):
        raise ValueError(f"dW must be float32 of shape ({K}, {d})")
    if dws.dtype != torch.float32 or tuple(dws.shape) != (K,):
        raise ValueError(f"dw_static must be float32 of shape ({K},)")
    need = int(lib().hc_weights_backward_workspace(T, n, d, int(sinkhorn_iters)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=H.device)
    _dev(workspace, "workspace")
    _call("hc_weights_backward_terms", H.data_ptr(), W.data_ptr(), w_static.data_ptr(), float(scale),
          float(eps), int(sinkhorn_iters), dw.data_ptr(),
          dw2.data_ptr() if dw2 is not None else None,
          saved.data_ptr() if saved is not None else None, dhb.data_ptr(), co.data_ptr(),
          dW.data_ptr(), dws.data_ptr(), workspace.data_ptr(),
          workspace.numel() * workspace.element_size(), T, n, d, _dt(H), _stream(stream))
    return dhb, co, dW, dws


@_on_launch_stream
def sinkhorn_backward(logits, dw, n: int, iters: int, out=None, workspace=None, stream=None,
                      dw2=None):
    """Gradient of sinkhorn: dL/dlogits (T, K) float32 from dL/dw (T, K),
    plus dw2 when given (the records' gradient from a second call, e.g. the
    read-mix's and the write-back's of one layer)."""
    _dev(logits, "logits")
    _dev(dw, "dw")
    K = 2 * n + n * n
    if logits.dtype != torch.float32 or logits.dim() != 2 or logits.shape[1] != K:
        raise ValueError(f"logits must be float32 of shape (T, {K})")
    if dw.dtype != torch.float32 or dw.shape != logits.shape:
        raise ValueError("dw must match logits")
    if dw2 is not None:
        _dev(dw2, "dw2")
        if dw2.dtype != torch.float32 or dw2.shape != logits.shape:
            raise ValueError("dw2 must match logits")
    T = logits.shape[0]
    o = torch.empty_like(logits) if out is None else _dev(out, "out")
    need = int(lib().hc_sinkhorn_backward_workspace(T, int(iters)))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=logits.device)
    _dev(workspace, "workspace")
    _call("hc_sinkhorn_backward", logits.data_ptr(), dw.data_ptr(),
          dw2.data_ptr() if dw2 is not None else None, o.data_ptr(), int(iters),
          workspace.data_ptr(), workspace.numel() * workspace.element_size(), T, n,
          _stream(stream))
    return o
