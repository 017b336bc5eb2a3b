"""Parity of the HIP backward (fwa_delta_backward, through the C ABI) with the fp64 oracle's
gradient on the GPU.

Every gradient (dq, dk, dv, dbeta_logit, dW0) is compared normwise per (b, h) slice against
oracle.delta_backward on the same inputs and cotangents: fp32 inputs 1e-4, bf16 inputs 2e-2
(fp32 arithmetic, gradients rounded to bf16 on output).
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, log, normwise
from weight_linear_attention_amd import fwa
from weight_linear_attention_amd.synthetic import (EDGE_CASES, make_cotangents, make_edge_inputs,
                                                   make_inputs, to_f64, workload)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
NAMES = ("dq", "dk", "dv", "dbeta_logit", "dW0")


def _run(inp, cot, nu, need_dW0=True):
    d = {k: (None if v is None else v.to(DEV)) for k, v in {**inp, **cot}.items()}
    out = fwa.delta_backward(d["q"], d["k"], d["v"], d["beta_logit"], d["dy"], W0=d["W0"],
                             dW_final=d["dW_final"], nu=nu, need_dW0=need_dW0)
    torch.cuda.synchronize()
    return out


def _check(inp, cot, nu, dtype, label, need_dW0=True):
    got = _run(inp, cot, nu, need_dW0)
    f = lambda n: to_f64(inp[n]) if n in inp else None
    ref = oracle.delta_backward(f("q"), f("k"), f("v"), f("beta_logit"), to_f64(inp["W0"]),
                                to_f64(cot["dy"]), to_f64(cot["dW_final"]), nu=nu)
    errs = {}
    for name, g, r in zip(NAMES, got, ref):
        if g is None:
            continue
        errs[name] = normwise(to_f64(g), r, 2)
    log(f"  backward {label}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    tol = TOL[dtype]
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    return got


BWD_CASES = [
    ("tiny_t64_d16_nu1_f32", {}, True),
    ("tiny_t64_d16_nu1_f32", {"T": 77, "w0_std": 0.05}, False),
    ("h8_t1024_d64_nu1_f32", {}, True),
    ("h8_t1024_d64_nu1_f32", {"T": 333, "w0_std": 0.05, "nu": 2, "d_v": 40}, True),
    ("h8_t1024_d64_nu1_f32", {"B": 2, "H": 3, "T": 20, "d_k": 32, "nu": 3, "d_v": 16}, False),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {}, True),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 1000, "nu": 3}, True),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 2, "T": 45, "d_k": 16, "nu": 5, "d_v": 24}, False),
    # more chunks than resident workgroups, not a multiple of them, and a ragged last chunk
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"T": 2100}, False),
]


@pytest.mark.parametrize("name,ov,with_dwf", BWD_CASES,
                         ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(BWD_CASES)])
def test_backward_parity(name, ov, with_dwf):
    w = workload(name, **ov)
    log(f"backward {w} dW_final={'yes' if with_dwf else 'no'}")
    inp = make_inputs(w)
    cot = make_cotangents(w, with_dW_final=with_dwf)
    _check(inp, cot, w.nu, w.torch_dtype, w.name)


@pytest.mark.parametrize("case", EDGE_CASES)
@pytest.mark.parametrize("name,ov", [("tiny_t64_d16_nu1_f32", {"T": 150, "w0_std": 0.05}),
                                     ("h8_t1024_d64_nu1_f32", {"T": 200}),
                                     ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 2, "T": 300})])
def test_backward_edge_cases(name, ov, case):
    w = workload(name, **ov)
    inp = make_edge_inputs(w, case)
    cot = make_cotangents(w)
    got = _check(inp, cot, w.nu, w.torch_dtype, f"{name} {case}")
    for g in got:
        assert torch.isfinite(g.float()).all()


def test_backward_without_dW0_and_deterministic():
    w = workload("h8_t1024_d64_nu1_f32", T=300, w0_std=0.05)
    inp, cot = make_inputs(w), make_cotangents(w)
    a = _run(inp, cot, w.nu)
    b = _run(inp, cot, w.nu, need_dW0=False)
    assert b[4] is None
    for x, y in zip(a[:4], b[:4]):
        assert torch.equal(x, y)
    c = _run(inp, cot, w.nu)
    for x, y in zip(a, c):
        assert torch.equal(x, y)


def test_backward_T0_and_empty():
    w = workload("h8_t1024_d64_nu1_f32", T=0, w0_std=0.1)
    inp, cot = make_inputs(w), make_cotangents(w)
    out = _run(inp, cot, w.nu)
    assert torch.equal(out[4], cot["dW_final"].to(DEV))
    cot["dW_final"] = None
    out = _run(inp, cot, w.nu)
    assert torch.count_nonzero(out[4]) == 0
    w = workload("h8_t1024_d64_nu1_f32", B=0)
    out = _run(make_inputs(w), make_cotangents(w), w.nu)
    assert out[0].numel() == 0


def test_backward_matches_forward_differences():
    """A directional derivative of the GPU forward (central difference in fp32 along a random
    direction of every input at once) matches the inner product of that direction with the GPU
    gradients, for L = <dy, y> + <dW_final, W_final>."""
    w = workload("h8_t1024_d64_nu1_f32", T=200, w0_std=0.05)
    inp, cot = make_inputs(w), make_cotangents(w)
    for n in ("q", "k"):          # |entries| >= 0.2: no ReLU kink within the step below
        inp[n] = torch.sign(inp[n]) * (inp[n].abs() + 0.2)
    d = {k: v.to(DEV).double() for k, v in inp.items()}
    g = torch.Generator().manual_seed(5)
    dirs = {k: torch.randn(v.shape, generator=g).to(DEV).double() for k, v in inp.items()}
    dy, dWf = cot["dy"].to(DEV).double(), cot["dW_final"].to(DEV).double()

    def loss(eps):
        x = {k: (d[k] + eps * dirs[k]).float().contiguous() for k in d}
        y, Wf = fwa.delta_forward(x["q"], x["k"], x["v"], x["beta_logit"], x["W0"], nu=w.nu,
                                  path="fused")
        return float((dy * y.double()).sum() + (dWf * Wf.double()).sum())

    h = 1e-2                      # the step moves q, k by at most ~0.05
    num = (loss(h) - loss(-h)) / (2 * h)
    grads = _run(inp, cot, w.nu)
    ana = sum(float((gr.double() * dirs[n]).sum())
              for gr, n in zip(grads, ("q", "k", "v", "beta_logit", "W0")))
    log(f"  directional derivative: finite difference {num:.6e}, gradients {ana:.6e}")
    assert abs(num - ana) <= 2e-3 * max(1.0, abs(ana))
