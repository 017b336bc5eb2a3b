"""Helpers shared by the GPU parity tests: error metrics and oracle runs on exact copies of
the inputs the HIP path sees.  Imports the oracle (test infrastructure) and the input
generator; never the other way round."""
import sys

import numpy as np
import torch

import oracle
from weight_linear_attention_amd.synthetic import to_f64

# Tolerances: normwise per (b, h) slice, max|gpu - ref| / max|ref|.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def normwise(gpu, ref, slice_axes):
    """Max over slices of max|gpu - ref| / max|ref|, where a slice is everything but the
    leading `slice_axes` axes.  Slices whose reference is identically zero use max|gpu|."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    lead = int(np.prod(gpu.shape[:slice_axes])) if slice_axes else 1
    g = gpu.reshape(lead, -1)
    r = ref.reshape(lead, -1)
    err = np.abs(g - r).max(axis=1) if g.shape[1] else np.zeros(lead)
    scale = np.abs(r).max(axis=1) if r.shape[1] else np.ones(lead)
    rel = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)
    return float(rel.max()) if lead else 0.0


def oracle_forward(inp, nu, bh_index=None):
    """Oracle forward on the same (CPU) tensors; optionally only on the (b, h) slices listed
    in bh_index (a list of (b, h) pairs) -- returns arrays stacked in that order."""
    q, k, v, l, W0 = (to_f64(inp[n]) for n in ("q", "k", "v", "beta_logit", "W0"))
    if bh_index is not None:
        sel = tuple(np.array(ix) for ix in zip(*bh_index))
        q, k, v, l = (a[sel][None] for a in (q, k, v, l))
        W0 = None if W0 is None else W0[sel][None]
    return oracle.delta_forward(q, k, v, l, W0, nu=nu)


def oracle_forward_batched(inp, nu):
    """Oracle forward on every (b, h) slice, one batch row (H slices) per oracle call so that
    only one row's fp64 inputs exist at a time.  Returns (y, W_final) as fp64 arrays."""
    q, k, v, l, W0 = (inp[n] for n in ("q", "k", "v", "beta_logit", "W0"))
    B, H, T, _ = q.shape
    d_v = v.shape[-1]
    D = 2 * q.shape[-1] * nu
    y = np.empty((B, H, T, d_v), dtype=np.float64)
    Wf = np.empty((B, H, d_v, D), dtype=np.float64)
    for b in range(B):
        row = lambda t: None if t is None else to_f64(t[b:b + 1])
        y[b:b + 1], Wf[b:b + 1] = oracle.delta_forward(row(q), row(k), row(v), row(l), row(W0),
                                                        nu=nu)
    return y, Wf
