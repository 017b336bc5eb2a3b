"""fp64 CPU oracle for the fast-weight delta-rule layer with DPFP projection.

TEST INFRASTRUCTURE ONLY.  Only tests/, the package's smoke() check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP library and never
imports it.

`dpfp`, `dpfp_mask`, `delta_forward`, `delta_step`, `delta_backward` (the gradient of
`delta_forward`), `sum_forward` (sum-update linear attention with the z normaliser),
`layer_project` and `layer_output` (the linear maps around the layer) wrap the plain-C fp64 implementation in
fwa_oracle.c (built by oracle/build.py); `twin` holds an independent NumPy transcription used to
cross-check it.  All arrays are float64, C-contiguous, in the [B, H, T, d] layout; W is
[B, H, d_v, D] with D = 2 * d_k * nu.  Inputs given in fp32 or bf16 are taken exactly (bf16 and
fp32 values are exactly representable in fp64).
"""
import ctypes
import os

import numpy as np

from . import build as _build


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """Bindings to one compiled copy of fwa_oracle.c (the real one, or a test's variant)."""

    def __init__(self, path):
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_dpfp.argtypes = [P, P, i64, i32, i32]
        L.oracle_dpfp_mask.argtypes = [P, P, i64, i32, i32]
        L.oracle_delta_forward.argtypes = [P, P, P, P, P, P, P] + [i32] * 6
        L.oracle_delta_step.argtypes = [P, P, P, P, P, P] + [i32] * 5
        L.oracle_delta_backward.argtypes = [P] * 12 + [i32] * 6
        L.oracle_sum_forward.argtypes = [P] * 8 + [i32] * 6
        L.oracle_layer_project.argtypes = [P] * 6 + [i32] * 6
        L.oracle_layer_output.argtypes = [P] * 5 + [i32] * 5
        L.oracle_sigmoid.argtypes = [ctypes.c_double]
        L.oracle_sigmoid.restype = ctypes.c_double
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        self.lib = L
        self.path = path

    def num_threads(self):
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n):
        self.lib.oracle_set_num_threads(int(n))

    def sigmoid(self, x):
        return self.lib.oracle_sigmoid(float(x))

    def dpfp(self, x, nu):
        """phi = DPFP(x) over the last axis; x [..., d_k] -> [..., 2*d_k*nu] (float64)."""
        x = _f64(x)
        d_k = x.shape[-1]
        n = int(np.prod(x.shape[:-1], dtype=np.int64))
        out = np.empty(x.shape[:-1] + (2 * d_k * nu,), dtype=np.float64)
        self.lib.oracle_dpfp(_p(x), _p(out), n, d_k, nu)
        return out

    def dpfp_mask(self, x, nu):
        """Boolean zero/nonzero pattern of DPFP(x), decided from signs alone."""
        x = _f64(x)
        d_k = x.shape[-1]
        n = int(np.prod(x.shape[:-1], dtype=np.int64))
        out = np.empty(x.shape[:-1] + (2 * d_k * nu,), dtype=np.uint8)
        self.lib.oracle_dpfp_mask(_p(x), _p(out), n, d_k, nu)
        return out.astype(bool)

    def delta_forward(self, q, k, v, beta_logit, W0=None, nu=1):
        """Literal per-step recurrence. Returns (y [B,H,T,d_v], W_final [B,H,d_v,D])."""
        q, k, v, beta_logit = _f64(q), _f64(k), _f64(v), _f64(beta_logit)
        B, H, T, d_k = q.shape
        d_v = v.shape[-1]
        D = 2 * d_k * nu
        assert k.shape == q.shape and v.shape == (B, H, T, d_v)
        assert beta_logit.shape == (B, H, T)
        if W0 is not None:
            W0 = _f64(W0)
            assert W0.shape == (B, H, d_v, D)
        y = np.zeros((B, H, T, d_v), dtype=np.float64)
        Wf = np.empty((B, H, d_v, D), dtype=np.float64)
        self.lib.oracle_delta_forward(_p(q), _p(k), _p(v), _p(beta_logit), _p(W0), _p(y),
                                      _p(Wf), B, H, T, d_k, d_v, nu)
        return y, Wf

    def delta_backward(self, q, k, v, beta_logit, W0, dy, dW_final=None, nu=1):
        """Gradients of <dy, y> + <dW_final, W_final> through delta_forward (reverse mode
        through the literal recurrence).  Returns (dq, dk, dv, dbeta_logit, dW0)."""
        q, k, v, beta_logit, dy = _f64(q), _f64(k), _f64(v), _f64(beta_logit), _f64(dy)
        B, H, T, d_k = q.shape
        d_v = v.shape[-1]
        D = 2 * d_k * nu
        assert k.shape == q.shape and v.shape == (B, H, T, d_v) and dy.shape == v.shape
        assert beta_logit.shape == (B, H, T)
        if W0 is not None:
            W0 = _f64(W0)
            assert W0.shape == (B, H, d_v, D)
        if dW_final is not None:
            dW_final = _f64(dW_final)
            assert dW_final.shape == (B, H, d_v, D)
        dq = np.empty_like(q)
        dk = np.empty_like(k)
        dv = np.empty_like(v)
        dl = np.empty_like(beta_logit)
        dW0 = np.empty((B, H, d_v, D), dtype=np.float64)
        self.lib.oracle_delta_backward(_p(q), _p(k), _p(v), _p(beta_logit), _p(W0), _p(dy),
                                       _p(dW_final), _p(dq), _p(dk), _p(dv), _p(dl), _p(dW0),
                                       B, H, T, d_k, d_v, nu)
        return dq, dk, dv, dl, dW0

    def sum_forward(self, q, k, v, W0=None, z0=None, nu=1):
        """Sum-update linear attention with the z normaliser.  Returns (y, W_final, z_final)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, T, d_k = q.shape
        d_v = v.shape[-1]
        D = 2 * d_k * nu
        assert k.shape == q.shape and v.shape == (B, H, T, d_v)
        if W0 is not None:
            W0 = _f64(W0)
            assert W0.shape == (B, H, d_v, D)
        if z0 is not None:
            z0 = _f64(z0)
            assert z0.shape == (B, H, D)
        y = np.zeros((B, H, T, d_v), dtype=np.float64)
        Wf = np.empty((B, H, d_v, D), dtype=np.float64)
        zf = np.empty((B, H, D), dtype=np.float64)
        self.lib.oracle_sum_forward(_p(q), _p(k), _p(v), _p(W0), _p(z0), _p(y), _p(Wf), _p(zf),
                                    B, H, T, d_k, d_v, nu)
        return y, Wf, zf

    def layer_project(self, x, Wqkvb, H, d_k, d_v):
        """x [B, T, d_model] through the stacked bias-free projections Wqkvb
        [2*H*d_k + H*d_v + H, d_model].  Returns (q, k, v, beta_logit) in [B, H, T, .]."""
        x, Wqkvb = _f64(x), _f64(Wqkvb)
        B, T, d_model = x.shape
        assert Wqkvb.shape == (2 * H * d_k + H * d_v + H, d_model)
        q = np.empty((B, H, T, d_k))
        k = np.empty((B, H, T, d_k))
        v = np.empty((B, H, T, d_v))
        bl = np.empty((B, H, T))
        self.lib.oracle_layer_project(_p(x), _p(Wqkvb), _p(q), _p(k), _p(v), _p(bl), B, T,
                                      d_model, H, d_k, d_v)
        return q, k, v, bl

    def layer_output(self, y, Wo, bo=None, residual=None):
        """residual + bo + concat_heads(y) Wo^T for y [B, H, T, d_v], Wo [d_model, H*d_v]."""
        y, Wo = _f64(y), _f64(Wo)
        B, H, T, d_v = y.shape
        d_model = Wo.shape[0]
        assert Wo.shape == (d_model, H * d_v)
        bo = None if bo is None else _f64(bo)
        residual = None if residual is None else _f64(residual)
        out = np.empty((B, T, d_model))
        self.lib.oracle_layer_output(_p(y), _p(Wo), _p(bo), _p(residual), _p(out), B, T, H, d_v,
                                     d_model)
        return out

    def delta_step(self, q, k, v, beta_logit, W, nu=1):
        """One decode step. q,k [B,H,d_k], v [B,H,d_v], beta_logit [B,H], W [B,H,d_v,D].
        Returns (y [B,H,d_v], W_new); the W passed in is not modified."""
        q, k, v, beta_logit = _f64(q), _f64(k), _f64(v), _f64(beta_logit)
        B, H, d_k = q.shape
        d_v = v.shape[-1]
        W = np.array(W, dtype=np.float64, copy=True, order="C")
        assert W.shape == (B, H, d_v, 2 * d_k * nu)
        y = np.empty((B, H, d_v), dtype=np.float64)
        self.lib.oracle_delta_step(_p(q), _p(k), _p(v), _p(beta_logit), _p(W), _p(y),
                                   B, H, d_k, d_v, nu)
        return y, W


_DEFAULT = None


def default():
    """The oracle built from oracle/fwa_oracle.c (rebuilt when the source is newer)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _DEFAULT = Oracle(_build.LIB)
    return _DEFAULT


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    default().set_num_threads(n)


def sigmoid(x):
    return default().sigmoid(x)


def dpfp(x, nu):
    return default().dpfp(x, nu)


def dpfp_mask(x, nu):
    return default().dpfp_mask(x, nu)


def delta_forward(q, k, v, beta_logit, W0=None, nu=1):
    return default().delta_forward(q, k, v, beta_logit, W0, nu)


def delta_step(q, k, v, beta_logit, W, nu=1):
    return default().delta_step(q, k, v, beta_logit, W, nu)


def layer_project(x, Wqkvb, H, d_k, d_v):
    return default().layer_project(x, Wqkvb, H, d_k, d_v)


def layer_output(y, Wo, bo=None, residual=None):
    return default().layer_output(y, Wo, bo, residual)


def sum_forward(q, k, v, W0=None, z0=None, nu=1):
    return default().sum_forward(q, k, v, W0, z0, nu)


def delta_backward(q, k, v, beta_logit, W0, dy, dW_final=None, nu=1):
    return default().delta_backward(q, k, v, beta_logit, W0, dy, dW_final, nu)
