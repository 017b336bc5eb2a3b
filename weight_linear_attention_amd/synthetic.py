"""Seeded synthetic inputs for the fast-weight delta-rule layer.

This module holds no arithmetic of the method: it only draws random tensors.  Both the HIP
path's tests/benchmark and the fp64 oracle consume exactly the tensors made here.

Recipe (the same for every workload): a CPU `torch.Generator` seeded with the workload's seed
draws fp32 N(0, 1) samples in the fixed order q, k, v, beta_logit, then W0 (scaled by the
workload's w0_std, or W0 = None when the state starts at zero).  For bf16 workloads q, k, v and
beta_logit are then rounded to bf16 (round-to-nearest-even); W0 stays fp32 because the state is
always fp32.  The values stand in for projected activations of the layer at the shapes the pages
use (d_model 512 = 8 heads x d_k 64, chunk 64, sequence 64/1024); no dataset is used.
"""
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    d_k: int
    d_v: int
    nu: int
    dtype: str            # "f32" or "bf16": element type of q, k, v, beta_logit and y
    chunk: int
    w0_std: Optional[float]  # None: the state starts at zero
    seed: int
    steps: int = 0        # decode workloads: number of successive single-token steps

    @property
    def D(self):
        return 2 * self.d_k * self.nu

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


WORKLOADS = {
    w.name: w for w in [
        # single head, 64 steps, d 16: small enough for the oracle in milliseconds
        Workload("tiny_t64_d16_nu1_f32", 1, 1, 64, 16, 16, 1, "f32", 64, None, 1001),
        # the pages' layer shape: 8 heads x d_k 64 (d_model 512), nu 1, sequence 1024, chunk 64
        Workload("h8_t1024_d64_nu1_f32", 1, 8, 1024, 64, 64, 1, "f32", 64, None, 1002),
        # bf16 activations, nu 2, state carried in from a previous segment
        Workload("b4_h8_t4096_d64_nu2_bf16_carried", 4, 8, 4096, 64, 64, 2, "bf16", 64, 0.01,
                 1003),
        # long sequence, nu 3 (D 384), bf16 activations
        Workload("b8_h16_t16384_d64_nu3_bf16", 8, 16, 16384, 64, 64, 3, "bf16", 64, None, 1004),
        # decode: 256 sequences x 8 heads, persistent fp32 state [256, 8, 64, 128]
        Workload("decode_b256_h8_d64_nu1_f32", 256, 8, 1, 64, 64, 1, "f32", 1, None, 1005,
                 steps=1024),
    ]
}


def workload(name, **overrides):
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def make_inputs(w: Workload, seed: Optional[int] = None):
    """Forward inputs on the CPU: dict(q, k, v, beta_logit, W0)."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    q = torch.randn(w.B, w.H, w.T, w.d_k, generator=g)
    k = torch.randn(w.B, w.H, w.T, w.d_k, generator=g)
    v = torch.randn(w.B, w.H, w.T, w.d_v, generator=g)
    beta_logit = torch.randn(w.B, w.H, w.T, generator=g)
    W0 = None
    if w.w0_std is not None:
        W0 = torch.randn(w.B, w.H, w.d_v, w.D, generator=g) * w.w0_std
    cast = (lambda t: t.to(torch.bfloat16)) if w.dtype == "bf16" else (lambda t: t)
    return dict(q=cast(q), k=cast(k), v=cast(v), beta_logit=cast(beta_logit), W0=W0)


EDGE_CASES = ("beta_saturated", "tiny_keys", "repeated_key", "zero_keys")


def make_edge_inputs(w: Workload, case: str, seed: Optional[int] = None):
    """Forward inputs (as make_inputs) reshaped into one of the method's edge cases:
      beta_saturated  beta_logit = +-20 (sign drawn at random): beta within 2e-9 of 0 or 1;
      tiny_keys       k scaled by 1e-3, so DPFP's sum is of the order of its eps;
      repeated_key    rows [40, 104) of k (across a chunk boundary at 64) all equal row 40;
      zero_keys       every 7th row of k (from row 3) and rows [64, 80) are zero.
    The edits are made on the fp32 draw, before any rounding to bf16."""
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    q = torch.randn(w.B, w.H, w.T, w.d_k, generator=g)
    k = torch.randn(w.B, w.H, w.T, w.d_k, generator=g)
    v = torch.randn(w.B, w.H, w.T, w.d_v, generator=g)
    beta_logit = torch.randn(w.B, w.H, w.T, generator=g)
    W0 = None
    if w.w0_std is not None:
        W0 = torch.randn(w.B, w.H, w.d_v, w.D, generator=g) * w.w0_std
    if case == "beta_saturated":
        beta_logit = torch.where(beta_logit >= 0, 20.0, -20.0)
    elif case == "tiny_keys":
        k = k * 1e-3
    elif case == "repeated_key":
        lo, hi = min(40, w.T), min(104, w.T)
        k[:, :, lo:hi] = k[:, :, lo:lo + 1]
    elif case == "zero_keys":
        k[:, :, 3::7] = 0.0
        k[:, :, 64:80] = 0.0
    else:
        raise ValueError(f"unknown edge case {case!r}")
    cast = (lambda t: t.to(torch.bfloat16)) if w.dtype == "bf16" else (lambda t: t)
    return dict(q=cast(q), k=cast(k), v=cast(v), beta_logit=cast(beta_logit), W0=W0)


def make_cotangents(w: Workload, with_dW_final: bool = True, seed: Optional[int] = None):
    """Gradients of a loss with respect to the forward's outputs, for the backward: dy
    [B,H,T,d_v] ~ N(0, 1) in the workload's dtype and dW_final [B,H,d_v,D] ~ N(0, 1) fp32
    (None when with_dW_final is False), drawn from seed + 100 in that order."""
    g = torch.Generator("cpu").manual_seed((w.seed if seed is None else seed) + 100)
    dy = torch.randn(w.B, w.H, w.T, w.d_v, generator=g)
    dWf = torch.randn(w.B, w.H, w.d_v, w.D, generator=g) if with_dW_final else None
    if w.dtype == "bf16":
        dy = dy.to(torch.bfloat16)
    return dict(dy=dy, dW_final=dWf)


def make_decode_inputs(w: Workload, steps: Optional[int] = None, seed: Optional[int] = None):
    """Decode inputs on the CPU for `steps` successive tokens: q, k [S,B,H,d_k], v [S,B,H,d_v],
    beta_logit [S,B,H], and the initial state W0 (zeros unless w0_std is set)."""
    S = w.steps if steps is None else steps
    g = torch.Generator("cpu").manual_seed(w.seed if seed is None else seed)
    q = torch.randn(S, w.B, w.H, w.d_k, generator=g)
    k = torch.randn(S, w.B, w.H, w.d_k, generator=g)
    v = torch.randn(S, w.B, w.H, w.d_v, generator=g)
    beta_logit = torch.randn(S, w.B, w.H, generator=g)
    if w.w0_std is not None:
        W0 = torch.randn(w.B, w.H, w.d_v, w.D, generator=g) * w.w0_std
    else:
        W0 = torch.zeros(w.B, w.H, w.d_v, w.D)
    cast = (lambda t: t.to(torch.bfloat16)) if w.dtype == "bf16" else (lambda t: t)
    return dict(q=cast(q), k=cast(k), v=cast(v), beta_logit=cast(beta_logit), W0=W0)


def to_f64(t):
    """Exact float64 numpy copy of a CPU/GPU tensor (bf16 and fp32 embed exactly)."""
    return None if t is None else t.detach().to("cpu", torch.float32).double().numpy()
