"""Python binding of libfwa.so: argument marshalling only.

Every step of the layer runs in the HIP kernels behind the C ABI declared in include/fwa.h;
PyTorch is used only to allocate device memory and to name the stream.  The library must have
been built (weight_linear_attention_amd/build.py, or __graft_entry__.build()); loading fails
loudly otherwise -- there is no fallback.

Functions (same names as the C entry points, minus the prefix):
    dpfp(x, nu, out=None)                         -> phi
    delta_forward(q, k, v, beta_logit, W0=None, chunk=64, nu=1, out=None, W_final=None,
                  path="auto", workspace=None)    -> (y, W_final)
    delta_step(q, k, v, beta_logit, W, nu=1, out=None)
                                                  -> y      (W is updated in place)
    delta_forward_info(B, H, T, d_k, d_v, nu, chunk, dtype, path="auto")
                                                  -> ("chunked" | "stream" | "fused" | "none",
                                                      workspace bytes)
    delta_backward(q, k, v, beta_logit, dy, W0=None, dW_final=None, nu=1)
                                                  -> (dq, dk, dv, dbeta_logit, dW0)
    sum_forward(q, k, v, W0=None, z0=None, nu=1)  -> (y, W_final, z_final)
    layer_project(x, W_qkvb, H, d_k, d_v)         -> (q, k, v, beta_logit)
    layer_output(y, W_o, b_o=None, residual=None) -> out
    decode_layers(x, layers, memories, H, d_k, d_v, nu=1)
                                                  -> x (one token through all layers, in place)

Shapes are checked before anything else, so a wrong shape raises ValueError without touching
the device.  The forward's workspace is allocated here with torch on the current stream (the
caching allocator keeps it in stream order) unless the caller passes one.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfwa.so")

FWA_OK, FWA_ERR_INVALID_ARG, FWA_ERR_UNSUPPORTED, FWA_ERR_HIP = 0, 1, 2, 3
FWA_F32, FWA_BF16 = 0, 1
FWA_PATH_AUTO, FWA_PATH_CHUNKED, FWA_PATH_FUSED, FWA_PATH_STREAM, FWA_PATH_NONE = 0, 1, 2, 3, 4
PATHS = {"auto": FWA_PATH_AUTO, "chunked": FWA_PATH_CHUNKED, "fused": FWA_PATH_FUSED,
         "stream": FWA_PATH_STREAM}
PATH_NAMES = {FWA_PATH_NONE: "none", FWA_PATH_CHUNKED: "chunked", FWA_PATH_FUSED: "fused",
              FWA_PATH_STREAM: "stream"}

EXPORTED = ("fwa_dpfp", "fwa_delta_forward", "fwa_delta_forward_path", "fwa_delta_forward_info",
            "fwa_delta_forward_noalloc", "fwa_delta_backward", "fwa_delta_backward_info",
            "fwa_sum_forward", "fwa_sum_forward_info", "fwa_layer_project", "fwa_layer_output",
            "fwa_decode_layers", "fwa_decode_layers_info", "fwa_delta_step", "fwa_status_string",
            "fwa_last_error", "fwa_version")


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
    fwd = [P, P, P, P, P, P, P] + [i32] * 7 + [i32, P, i64, P]
    L.fwa_delta_forward.argtypes = fwd
    L.fwa_delta_forward.restype = i32
    L.fwa_delta_forward_path.argtypes = [i32] + fwd
    L.fwa_delta_forward_path.restype = i32
    L.fwa_delta_forward_noalloc.argtypes = [P, P, P, P, P, P, P] + [i32] * 7 + [i32, P]
    L.fwa_delta_forward_noalloc.restype = i32
    L.fwa_delta_forward_info.argtypes = [i32] * 9 + [ctypes.POINTER(i32), ctypes.POINTER(i64)]
    L.fwa_delta_forward_info.restype = i32
    L.fwa_delta_backward.argtypes = [P] * 12 + [i32] * 6 + [i32, P, i64, P]
    L.fwa_delta_backward.restype = i32
    L.fwa_delta_backward_info.argtypes = [i32] * 7 + [ctypes.POINTER(i64)]
    L.fwa_delta_backward_info.restype = i32
    L.fwa_sum_forward.argtypes = [P] * 8 + [i32] * 6 + [i32, P, i64, P]
    L.fwa_sum_forward.restype = i32
    L.fwa_sum_forward_info.argtypes = [i32] * 7 + [ctypes.POINTER(i64)]
    L.fwa_sum_forward_info.restype = i32
    L.fwa_layer_project.argtypes = [P] * 6 + [i32] * 6 + [i32, P]
    L.fwa_layer_project.restype = i32
    L.fwa_layer_output.argtypes = [P] * 5 + [i32] * 5 + [i32, P]
    L.fwa_layer_output.restype = i32
    L.fwa_decode_layers.argtypes = [P, i32, P, P, P, P] + [i32] * 6 + [i32, P, i64, P]
    L.fwa_decode_layers.restype = i32
    L.fwa_decode_layers_info.argtypes = [i32] * 7 + [ctypes.POINTER(i64)]
    L.fwa_decode_layers_info.restype = i32
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


def _dtype_code(dtype):
    if dtype == torch.float32:
        return FWA_F32
    if dtype == torch.bfloat16:
        return FWA_BF16
    raise TypeError(f"unsupported dtype {dtype}; expected float32 or bfloat16")


def _path_code(path):
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}, got {path!r}")
    return PATHS[path]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _shape(t, name, shape):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need(t, name, device, dtype=None):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def dpfp(x, nu, out=None):
    """DPFP over the last axis: [..., d_k] -> [..., 2*d_k*nu], same dtype and device."""
    d_k = x.shape[-1]
    _shape(out, "out", (*x.shape[:-1], 2 * d_k * nu))
    dev = x.device
    _need(x, "x", dev)
    n_vec = x.numel() // d_k if d_k else 0
    if out is None:
        out = torch.empty(*x.shape[:-1], 2 * d_k * nu, dtype=x.dtype, device=dev)
    _need(out, "out", dev, x.dtype)
    _check(lib().fwa_dpfp(_ptr(x), _ptr(out), n_vec, d_k, nu, _dtype_code(x.dtype), _stream(dev)))
    return out


def check_forward_shapes(q, k, v, beta_logit, W0=None, nu=1, out=None, W_final=None):
    """Raises ValueError unless the forward's tensors have consistent shapes."""
    if q.dim() != 4:
        raise ValueError(f"q must be [B, H, T, d_k], got {tuple(q.shape)}")
    B, H, T, d_k = q.shape
    if v.dim() != 4:
        raise ValueError(f"v must be [B, H, T, d_v], got {tuple(v.shape)}")
    d_v = v.shape[-1]
    D = 2 * d_k * nu
    _shape(k, "k", q.shape)
    _shape(v, "v", (B, H, T, d_v))
    _shape(beta_logit, "beta_logit", (B, H, T))
    _shape(W0, "W0", (B, H, d_v, D))
    _shape(out, "out", (B, H, T, d_v))
    _shape(W_final, "W_final", (B, H, d_v, D))
    return B, H, T, d_k, d_v, D


def delta_forward_info(B, H, T, d_k, d_v, nu=1, chunk=64, dtype=torch.float32, path="auto"):
    """Implementation ("chunked", "stream", "fused" or "none") a forward with these sizes takes
    (path="auto": the planner's choice) and the bytes of workspace it needs."""
    got, ws = ctypes.c_int(0), ctypes.c_int64(0)
    _check(lib().fwa_delta_forward_info(B, H, T, d_k, d_v, nu, chunk, _dtype_code(dtype),
                                        _path_code(path), ctypes.byref(got), ctypes.byref(ws)))
    return PATH_NAMES[got.value], ws.value


def delta_forward(q, k, v, beta_logit, W0=None, chunk=64, nu=1, out=None, W_final=None,
                  return_final=True, path="auto", workspace=None):
    """Causal chunked forward. q,k [B,H,T,d_k]; v [B,H,T,d_v]; beta_logit [B,H,T];
    W0 [B,H,d_v,D] fp32 or None.  Returns (y [B,H,T,d_v], W_final [B,H,d_v,D] fp32 or None).
    `path` pins the implementation ("auto" = the planner's choice); `workspace` is an optional
    uint8 device tensor of at least delta_forward_info(...)[1] bytes."""
    B, H, T, d_k, d_v, D = check_forward_shapes(q, k, v, beta_logit, W0, nu, out, W_final)
    code = _path_code(path)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta_logit, "beta_logit")):
        _need(t, n, dev, q.dtype)
    if W0 is not None:
        _need(W0, "W0", dev, torch.float32)
    if out is None:
        out = torch.empty(B, H, T, d_v, dtype=q.dtype, device=dev)
    _need(out, "out", dev, q.dtype)
    if W_final is None and return_final:
        W_final = torch.empty(B, H, d_v, D, dtype=torch.float32, device=dev)
    if W_final is not None:
        _need(W_final, "W_final", dev, torch.float32)
    if workspace is None:
        _, nbytes = delta_forward_info(B, H, T, d_k, d_v, nu, chunk, q.dtype, path)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    else:
        _need(workspace, "workspace", dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().fwa_delta_forward_path(code, _ptr(q), _ptr(k), _ptr(v), _ptr(beta_logit),
                                        _ptr(W0), _ptr(out), _ptr(W_final), B, H, T, d_k, d_v,
                                        nu, chunk, _dtype_code(q.dtype), _ptr(workspace),
                                        ws_bytes, _stream(dev)))
    return out, W_final


def delta_backward_info(B, H, T, d_k, d_v, nu=1, dtype=torch.float32):
    """Bytes of workspace delta_backward needs for these sizes."""
    ws = ctypes.c_int64(0)
    _check(lib().fwa_delta_backward_info(B, H, T, d_k, d_v, nu, _dtype_code(dtype),
                                         ctypes.byref(ws)))
    return ws.value


def delta_backward(q, k, v, beta_logit, dy, W0=None, dW_final=None, nu=1, need_dW0=True,
                   workspace=None):
    """Gradient of delta_forward: returns (dq, dk, dv, dbeta_logit, dW0) for the loss whose
    gradients with respect to y and W_final are dy and dW_final (None: zero).  dW0 is None when
    need_dW0 is False."""
    B, H, T, d_k, d_v, D = check_forward_shapes(q, k, v, beta_logit, W0, nu)
    _shape(dy, "dy", (B, H, T, d_v))
    _shape(dW_final, "dW_final", (B, H, d_v, D))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta_logit, "beta_logit"), (dy, "dy")):
        _need(t, n, dev, q.dtype)
    for t, n in ((W0, "W0"), (dW_final, "dW_final")):
        if t is not None:
            _need(t, n, dev, torch.float32)
    dq, dk = torch.empty_like(q), torch.empty_like(k)
    dv, dl = torch.empty_like(v), torch.empty_like(beta_logit)
    dW0 = torch.empty(B, H, d_v, D, dtype=torch.float32, device=dev) if need_dW0 else None
    if workspace is None:
        nbytes = delta_backward_info(B, H, T, d_k, d_v, nu, q.dtype)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    else:
        _need(workspace, "workspace", dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().fwa_delta_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(beta_logit), _ptr(W0),
                                    _ptr(dy), _ptr(dW_final), _ptr(dq), _ptr(dk), _ptr(dv),
                                    _ptr(dl), _ptr(dW0), B, H, T, d_k, d_v, nu,
                                    _dtype_code(q.dtype), _ptr(workspace), ws_bytes,
                                    _stream(dev)))
    return dq, dk, dv, dl, dW0


def sum_forward_info(B, H, T, d_k, d_v, nu=1, dtype=torch.float32):
    """Bytes of workspace sum_forward needs for these sizes."""
    ws = ctypes.c_int64(0)
    _check(lib().fwa_sum_forward_info(B, H, T, d_k, d_v, nu, _dtype_code(dtype), ctypes.byref(ws)))
    return ws.value


def sum_forward(q, k, v, W0=None, z0=None, nu=1, out=None, W_final=None, z_final=None,
                return_final=True, workspace=None):
    """Sum-update linear attention with the z normaliser.  Returns (y, W_final, z_final)."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B, H, T, d_k] and v [B, H, T, d_v]")
    B, H, T, d_k = q.shape
    d_v = v.shape[-1]
    D = 2 * d_k * nu
    _shape(k, "k", q.shape)
    _shape(v, "v", (B, H, T, d_v))
    _shape(W0, "W0", (B, H, d_v, D))
    _shape(z0, "z0", (B, H, D))
    _shape(out, "out", (B, H, T, d_v))
    _shape(W_final, "W_final", (B, H, d_v, D))
    _shape(z_final, "z_final", (B, H, D))
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, dev, q.dtype)
    for t, n in ((W0, "W0"), (z0, "z0")):
        if t is not None:
            _need(t, n, dev, torch.float32)
    if out is None:
        out = torch.empty(B, H, T, d_v, dtype=q.dtype, device=dev)
    _need(out, "out", dev, q.dtype)
    if return_final and W_final is None:
        W_final = torch.empty(B, H, d_v, D, dtype=torch.float32, device=dev)
    if return_final and z_final is None:
        z_final = torch.empty(B, H, D, dtype=torch.float32, device=dev)
    for t, n in ((W_final, "W_final"), (z_final, "z_final")):
        if t is not None:
            _need(t, n, dev, torch.float32)
    if workspace is None:
        nbytes = sum_forward_info(B, H, T, d_k, d_v, nu, q.dtype)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    else:
        _need(workspace, "workspace", dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().fwa_sum_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(W0), _ptr(z0), _ptr(out),
                                 _ptr(W_final), _ptr(z_final), B, H, T, d_k, d_v, nu,
                                 _dtype_code(q.dtype), _ptr(workspace), ws_bytes, _stream(dev)))
    return out, W_final, z_final


def layer_project(x, W_qkvb, H, d_k, d_v):
    """x [B, T, d_model] -> (q, k [B,H,T,d_k], v [B,H,T,d_v], beta_logit [B,H,T])."""
    if x.dim() != 3:
        raise ValueError(f"x must be [B, T, d_model], got {tuple(x.shape)}")
    B, T, d_model = x.shape
    _shape(W_qkvb, "W_qkvb", (2 * H * d_k + H * d_v + H, d_model))
    dev = x.device
    _need(x, "x", dev)
    _need(W_qkvb, "W_qkvb", dev, x.dtype)
    q = torch.empty(B, H, T, d_k, dtype=x.dtype, device=dev)
    k = torch.empty_like(q)
    v = torch.empty(B, H, T, d_v, dtype=x.dtype, device=dev)
    bl = torch.empty(B, H, T, dtype=x.dtype, device=dev)
    _check(lib().fwa_layer_project(_ptr(x), _ptr(W_qkvb), _ptr(q), _ptr(k), _ptr(v), _ptr(bl),
                                   B, T, d_model, H, d_k, d_v, _dtype_code(x.dtype), _stream(dev)))
    return q, k, v, bl


def layer_output(y, W_o, b_o=None, residual=None, out=None):
    """residual + b_o + concat_heads(y) W_o^T for y [B, H, T, d_v]; returns [B, T, d_model]
    (out may be the residual tensor itself)."""
    if y.dim() != 4:
        raise ValueError(f"y must be [B, H, T, d_v], got {tuple(y.shape)}")
    B, H, T, d_v = y.shape
    d_model = W_o.shape[0]
    _shape(W_o, "W_o", (d_model, H * d_v))
    _shape(b_o, "b_o", (d_model,))
    _shape(residual, "residual", (B, T, d_model))
    _shape(out, "out", (B, T, d_model))
    dev = y.device
    _need(y, "y", dev)
    for t, n in ((W_o, "W_o"), (b_o, "b_o"), (residual, "residual")):
        if t is not None:
            _need(t, n, dev, y.dtype)
    if out is None:
        out = torch.empty(B, T, d_model, dtype=y.dtype, device=dev)
    _need(out, "out", dev, y.dtype)
    _check(lib().fwa_layer_output(_ptr(y), _ptr(W_o), _ptr(b_o), _ptr(residual), _ptr(out), B, T,
                                  H, d_v, d_model, _dtype_code(y.dtype), _stream(dev)))
    return out


def decode_layers(x, layers, memories, H, d_k, d_v, nu=1, workspace=None):
    """One token through len(layers) layers, in place: x [B, d_model]; layers a list of
    (W_qkvb, W_o, b_o or None); memories a list of fp32 [B, H, d_v, D] tensors (updated)."""
    if x.dim() != 2:
        raise ValueError(f"x must be [B, d_model], got {tuple(x.shape)}")
    B, d_model = x.shape
    L = len(layers)
    if len(memories) != L:
        raise ValueError("one memory per layer")
    D = 2 * d_k * nu
    dev = x.device
    _need(x, "x", dev)
    for l, ((Wp, Wo, bo), W) in enumerate(zip(layers, memories)):
        _shape(Wp, f"W_qkvb[{l}]", (2 * H * d_k + H * d_v + H, d_model))
        _shape(Wo, f"W_o[{l}]", (d_model, H * d_v))
        _shape(bo, f"b_o[{l}]", (d_model,))
        _shape(W, f"W[{l}]", (B, H, d_v, D))
        for t, n in ((Wp, "W_qkvb"), (Wo, "W_o"), (bo, "b_o")):
            if t is not None:
                _need(t, n, dev, x.dtype)
        _need(W, "W", dev, torch.float32)
    code = _dtype_code(x.dtype)
    if workspace is None:
        nbytes = ctypes.c_int64(0)
        _check(lib().fwa_decode_layers_info(B, d_model, H, d_k, d_v, nu, code, ctypes.byref(nbytes)))
        workspace = torch.empty(max(nbytes.value, 16), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", dev)
    arr = lambda ts: (ctypes.c_void_p * max(L, 1))(*[None if t is None else t.data_ptr() for t in ts])
    _check(lib().fwa_decode_layers(_ptr(x), L, arr([p[0] for p in layers]), arr([p[1] for p in layers]),
                                   arr([p[2] for p in layers]), arr(memories), B, d_model, H, d_k,
                                   d_v, nu, code, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(dev)))
    return x


def check_step_shapes(q, k, v, beta_logit, W, nu=1, out=None):
    """Raises ValueError unless the decode step's tensors have consistent shapes."""
    if q.dim() != 3:
        raise ValueError(f"q must be [B, H, d_k], got {tuple(q.shape)}")
    B, H, d_k = q.shape
    if v.dim() != 3:
        raise ValueError(f"v must be [B, H, d_v], got {tuple(v.shape)}")
    d_v = v.shape[-1]
    _shape(k, "k", q.shape)
    _shape(v, "v", (B, H, d_v))
    _shape(beta_logit, "beta_logit", (B, H))
    _shape(W, "W", (B, H, d_v, 2 * d_k * nu))
    _shape(out, "out", (B, H, d_v))
    return B, H, d_k, d_v


def delta_step(q, k, v, beta_logit, W, nu=1, out=None):
    """One decode step; W [B,H,d_v,D] fp32 is updated in place.  Returns y [B,H,d_v]."""
    B, H, d_k, d_v = check_step_shapes(q, k, v, beta_logit, W, nu, out)
    dev = q.device
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (beta_logit, "beta_logit")):
        _need(t, n, dev, q.dtype)
    _need(W, "W", dev, torch.float32)
    if out is None:
        out = torch.empty(B, H, d_v, dtype=q.dtype, device=dev)
    _need(out, "out", dev, q.dtype)
    _check(lib().fwa_delta_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta_logit), _ptr(W), _ptr(out),
                                B, H, d_k, d_v, nu, _dtype_code(q.dtype), _stream(dev)))
    return out
