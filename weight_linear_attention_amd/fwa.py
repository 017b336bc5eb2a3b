"""Python binding of libfwa.so: argument marshalling only.

Every step of the layer runs in the HIP kernels behind the C ABI declared in include/fwa.h;
PyTorch is used only to allocate device memory and to name the stream.  The library must have
been built (weight_linear_attention_amd/build.py, or __graft_entry__.build()); loading fails
loudly otherwise -- there is no fallback.

Functions (same names as the C entry points, minus the prefix):
    dpfp(x, nu)                                   -> phi
    delta_forward(q, k, v, beta_logit, W0=None, chunk=64, out=None, W_final=None)
                                                  -> (y, W_final)
    delta_step(q, k, v, beta_logit, W, out=None)  -> y      (W is updated in place)
    delta_forward_info(B, H, T, d_k, d_v, nu, chunk, dtype)
                                                  -> ("chunked" | "fused" | "none", workspace bytes)
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfwa.so")

FWA_OK, FWA_ERR_INVALID_ARG, FWA_ERR_UNSUPPORTED, FWA_ERR_HIP = 0, 1, 2, 3
FWA_F32, FWA_BF16 = 0, 1
FWA_PATH_NONE, FWA_PATH_CHUNKED, FWA_PATH_FUSED, FWA_PATH_STREAM = 0, 1, 2, 3

EXPORTED = ("fwa_dpfp", "fwa_delta_forward", "fwa_delta_forward_info", "fwa_delta_step",
            "fwa_status_string", "fwa_last_error", "fwa_version")


class FwaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


_lib = None


def lib():
    """The loaded libfwa.so with argument types declared (raises if it was never built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m weight_linear_attention_amd.build` first")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    L.fwa_dpfp.argtypes = [P, P, i64, i32, i32, i32, P]
    L.fwa_dpfp.restype = i32
    L.fwa_delta_forward.argtypes = [P, P, P, P, P, P, P] + [i32] * 7 + [i32, P]
    L.fwa_delta_forward.restype = i32
    L.fwa_delta_forward_info.argtypes = [i32] * 8 + [ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.fwa_delta_forward_info.restype = i32
    L.fwa_delta_step.argtypes = [P, P, P, P, P, P] + [i32] * 5 + [i32, P]
    L.fwa_delta_step.restype = i32
    L.fwa_status_string.argtypes = [i32]
    L.fwa_status_string.restype = ctypes.c_char_p
    L.fwa_last_error.restype = ctypes.c_char_p
    L.fwa_version.restype = i32
    _lib = L
    return L


def _check(status):
    if status != FWA_OK:
        L = lib()
        raise FwaError(status, "%s: %s" % (L.fwa_status_string(status).decode(),
                                           L.fwa_last_error().decode()))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return FWA_F32
    if t.dtype == torch.bfloat16:
        return FWA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, device, dtype=None):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def dpfp(x, nu, out=None):
    """DPFP over the last axis: [..., d_k] -> [..., 2*d_k*nu], same dtype and device."""
    dev = x.device
    _need(x, "x", dev)
    d_k = x.shape[-1]
    n_vec = x.numel() // d_k if d_k else 0
    if out is None:
        out = torch.empty(*x.shape[:-1], 2 * d_k * nu, dtype=x.dtype, device=dev)
    _need(out, "out", dev, x.dtype)
    _check(lib().fwa_dpfp(_ptr(x), _ptr(out), n_vec, d_k, nu, _dtype_code(x), _stream(dev)))
    return out


def delta_forward(q, k, v, beta_logit, W0=None, chunk=64, nu=1, out=None, W_final=None,
                  return_final=True):
    """Causal chunked forward. q,k [B,H,T,d_k]; v [B,H,T,d_v]; beta_logit [B,H,T];
    W0 [B,H,d_v,D] fp32 or None.  Returns (y [B,H,T,d_v], W_final [B,H,d_v,D] fp32 or None)."""
    dev = q.device
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    D = 2 * d_k * nu
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta_logit, "beta_logit")):
        _need(t, n, dev, q.dtype)
    if k.shape != q.shape or v.shape[:3] != (B, H, T) or beta_logit.shape != (B, H, T):
        raise ValueError("shape mismatch between q, k, v and beta_logit")
    if W0 is not None:
        _need(W0, "W0", dev, torch.float32)
        if W0.shape != (B, H, d_v, D):
            raise ValueError(f"W0 must be {(B, H, d_v, D)}")
    if out is None:
        out = torch.empty(B, H, T, d_v, dtype=q.dtype, device=dev)
    _need(out, "out", dev, q.dtype)
    if W_final is None and return_final:
        W_final = torch.empty(B, H, d_v, D, dtype=torch.float32, device=dev)
    if W_final is not None:
        _need(W_final, "W_final", dev, torch.float32)
    _check(lib().fwa_delta_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta_logit), _ptr(W0),
                                   _ptr(out), _ptr(W_final), B, H, T, d_k, d_v, nu, chunk,
                                   _dtype_code(q), _stream(dev)))
    return out, W_final


def delta_forward_info(B, H, T, d_k, d_v, nu=1, chunk=64, dtype=torch.float32):
    """Implementation ("chunked", "fused" or "none") that delta_forward takes for these sizes
    under the current FWA_FORWARD_PATH, and the bytes of workspace it allocates."""
    code = {torch.float32: FWA_F32, torch.bfloat16: FWA_BF16}.get(dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {dtype}; expected float32 or bfloat16")
    path, ws = ctypes.c_int(0), ctypes.c_int64(0)
    _check(lib().fwa_delta_forward_info(B, H, T, d_k, d_v, nu, chunk, code, ctypes.byref(path),
                                        ctypes.byref(ws)))
    names = {FWA_PATH_NONE: "none", FWA_PATH_CHUNKED: "chunked", FWA_PATH_FUSED: "fused",
             FWA_PATH_STREAM: "stream"}
    return names[path.value], ws.value


def delta_step(q, k, v, beta_logit, W, nu=1, out=None):
    """One decode step; W [B,H,d_v,D] fp32 is updated in place.  Returns y [B,H,d_v]."""
    dev = q.device
    B, H, d_k = q.shape
    d_v = v.shape[-1]
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta_logit, "beta_logit")):
        _need(t, n, dev, q.dtype)
    _need(W, "W", dev, torch.float32)
    if W.shape != (B, H, d_v, 2 * d_k * nu):
        raise ValueError(f"W must be {(B, H, d_v, 2 * d_k * nu)}")
    if out is None:
        out = torch.empty(B, H, d_v, dtype=q.dtype, device=dev)
    _need(out, "out", dev, q.dtype)
    _check(lib().fwa_delta_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta_logit), _ptr(W), _ptr(out),
                                B, H, d_k, d_v, nu, _dtype_code(q), _stream(dev)))
    return out
