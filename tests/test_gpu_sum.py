"""Parity of the sum-update linear attention with the z normaliser (fwa_sum_forward, through
the C ABI) with the fp64 oracle on the GPU: y, W_final and z_final normwise per (b, h) slice,
fp32 inputs 1e-4, bf16 inputs 2e-2."""
import pytest
import torch

import oracle
from parity_util import TOL, log, normwise
from weight_linear_attention_amd import fwa
from weight_linear_attention_amd.synthetic import make_edge_inputs, make_inputs, to_f64, workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _z0(w, seed=3):
    g = torch.Generator().manual_seed(w.seed + seed)
    return torch.rand(w.B, w.H, w.D, generator=g) * 0.5


def _check(inp, nu, dtype, z0=None, label=""):
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    y, Wf, zf = fwa.sum_forward(d["q"], d["k"], d["v"], d["W0"],
                                None if z0 is None else z0.to(DEV), nu=nu)
    torch.cuda.synchronize()
    yr, Wr, zr = oracle.sum_forward(to_f64(inp["q"]), to_f64(inp["k"]), to_f64(inp["v"]),
                                    to_f64(inp["W0"]), to_f64(z0), nu=nu)
    e = (normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2), normwise(to_f64(zf), zr, 2))
    log(f"  sum {label}: y {e[0]:.2e}  W_final {e[1]:.2e}  z_final {e[2]:.2e}")
    assert max(e) <= TOL[dtype], e
    return y, Wf, zf


SUM_CASES = [
    ("tiny_t64_d16_nu1_f32", {}, False),
    ("tiny_t64_d16_nu1_f32", {"T": 77, "w0_std": 0.05}, True),
    ("h8_t1024_d64_nu1_f32", {}, False),
    ("h8_t1024_d64_nu1_f32", {"T": 333, "nu": 2, "d_v": 100, "w0_std": 0.05}, True),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {}, True),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 999, "nu": 3, "w0_std": None}, False),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 2, "H": 3, "T": 45, "d_k": 32, "nu": 5, "d_v": 8}, True),
    # 16 heads x 4 column groups: 4 blocks of 24 chunks, the first three summed in 6 parts of 4,
    # the last block 22 chunks
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 2, "T": 3000}, True),
]


@pytest.mark.parametrize("name,ov,carried", SUM_CASES,
                         ids=[f"{n}-{i}" for i, (n, _, _) in enumerate(SUM_CASES)])
def test_sum_forward_parity(name, ov, carried):
    w = workload(name, **ov)
    log(f"sum forward {w} carried z0={carried}")
    _check(make_inputs(w), w.nu, w.torch_dtype, _z0(w) if carried else None, w.name)


@pytest.mark.parametrize("case", ["tiny_keys", "repeated_key", "zero_keys"])
@pytest.mark.parametrize("name,ov", [("tiny_t64_d16_nu1_f32", {"T": 150, "w0_std": 0.05}),
                                     ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 2, "T": 300})])
def test_sum_forward_edge_cases(name, ov, case):
    w = workload(name, **ov)
    _check(make_edge_inputs(w, case), w.nu, w.torch_dtype, _z0(w), f"{name} {case}")


def test_sum_forward_zero_denominator():
    """Zero queries (and a first step from zero state whose query shares no feature with the
    key) read 0."""
    w = workload("tiny_t64_d16_nu1_f32", T=40)
    inp = make_inputs(w)
    inp["q"][:, :, 5] = 0.0
    inp["q"][:, :, 20:23] = 0.0
    y, _, _ = _check(inp, w.nu, w.torch_dtype, None, "zero queries")
    assert not y[:, :, 5].any() and not y[:, :, 20:23].any()


def test_sum_forward_segments_in_place_and_deterministic():
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried", B=2, T=700)
    inp = {k: (None if v is None else v.to(DEV)) for k, v in make_inputs(w).items()}
    z0 = _z0(w).to(DEV)
    y, Wf, zf = fwa.sum_forward(inp["q"], inp["k"], inp["v"], inp["W0"], z0, nu=w.nu)
    y2, Wf2, zf2 = fwa.sum_forward(inp["q"], inp["k"], inp["v"], inp["W0"], z0, nu=w.nu)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(Wf, Wf2) and torch.equal(zf, zf2)
    W, z = inp["W0"].clone(), z0.clone()
    ys = []
    for lo, hi in [(0, 300), (300, 301), (301, 700)]:
        sl = {n: inp[n][:, :, lo:hi].contiguous() for n in ("q", "k", "v")}
        yy, _, _ = fwa.sum_forward(sl["q"], sl["k"], sl["v"], W, z, nu=w.nu, W_final=W,
                                   z_final=z)
        ys.append(yy)
    torch.cuda.synchronize()
    assert normwise(to_f64(torch.cat(ys, 2)), to_f64(y), 2) <= 2e-2
    assert normwise(to_f64(W), to_f64(Wf), 2) <= 1e-5
    assert normwise(to_f64(z), to_f64(zf), 2) <= 1e-5


def test_sum_forward_T0_and_empty():
    w = workload("h8_t1024_d64_nu1_f32", T=0, w0_std=0.1)
    inp = {k: (None if v is None else v.to(DEV)) for k, v in make_inputs(w).items()}
    z0 = _z0(w).to(DEV)
    _, Wf, zf = fwa.sum_forward(inp["q"], inp["k"], inp["v"], inp["W0"], z0, nu=w.nu)
    torch.cuda.synchronize()
    assert torch.equal(Wf, inp["W0"]) and torch.equal(zf, z0)
    w = workload("h8_t1024_d64_nu1_f32", B=0)
    inp = {k: (None if v is None else v.to(DEV)) for k, v in make_inputs(w).items()}
    y, _, _ = fwa.sum_forward(inp["q"], inp["k"], inp["v"], nu=w.nu)
    assert y.numel() == 0
