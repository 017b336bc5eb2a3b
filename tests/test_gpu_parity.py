"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Bars: fp32 inputs 1e-4, bf16 inputs 2e-2 (fp32 state), normwise per (b, h) slice; the DPFP
zero/nonzero pattern must match the oracle's sign predicate bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, log, normwise, oracle_forward
from weight_linear_attention_amd import fwa
from weight_linear_attention_amd.synthetic import (make_decode_inputs, make_inputs, to_f64,
                                                   workload)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


FORWARD_PATHS = ["chunked", "stream", "fused"]


@pytest.fixture(params=FORWARD_PATHS)
def path(request, monkeypatch):
    """Runs a forward test once per implementation (FWA_FORWARD_PATH)."""
    monkeypatch.setenv("FWA_FORWARD_PATH", request.param)
    return request.param


def _skip_unless(path, w):
    """Skips when the implementation forced by FWA_FORWARD_PATH does not take this shape."""
    try:
        got, _ = fwa.delta_forward_info(w.B, w.H, w.T, w.d_k, w.d_v, w.nu, w.chunk, w.torch_dtype)
    except fwa.FwaError as e:
        assert e.status == fwa.FWA_ERR_UNSUPPORTED
        pytest.skip(f"the {path} path does not take this shape: {e}")
    assert got in (path, "none")


def _forward(inp_d, nu, chunk, W0=True):
    y, Wf = fwa.delta_forward(inp_d["q"], inp_d["k"], inp_d["v"], inp_d["beta_logit"],
                              inp_d["W0"] if W0 else None, chunk=chunk, nu=nu)
    torch.cuda.synchronize()
    return y, Wf


# ------------------------------------------------------------------------------ DPFP

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d_k,nu", [(16, 1), (16, 3), (32, 2), (64, 1), (64, 2), (64, 3),
                                    (128, 1), (64, 7), (16, 31)])
def test_dpfp_parity_and_mask(dtype, d_k, nu):
    log(f"dpfp dtype={dtype} d_k={d_k} nu={nu}")
    g = torch.Generator().manual_seed(d_k * 100 + nu)
    n_vec = 1000 + 37                        # several workgroup rounds plus a ragged tail
    x = torch.randn(n_vec, d_k, generator=g).to(dtype)
    phi = fwa.dpfp(x.to(DEV), nu)
    torch.cuda.synchronize()
    got = to_f64(phi)
    ref = oracle.dpfp(to_f64(x), nu)
    assert got.shape == (n_vec, 2 * d_k * nu)
    assert np.array_equal(got != 0.0, oracle.dpfp_mask(to_f64(x), nu))
    assert np.array_equal(got != 0.0, ref != 0.0)
    assert not np.signbit(got).any()             # zeros are +0.0
    err = normwise(got, ref, 1)
    log(f"  normwise err {err:.3e}")
    assert err <= (1e-6 if dtype == torch.float32 else 4e-3)


def test_dpfp_empty_and_full_size_sample():
    x = torch.empty(0, 64, device=DEV)
    assert fwa.dpfp(x, 3).shape == (0, 384)
    # the q tensor of the 8 x 16 x 16384 workload (2M vectors), checked on a random sample
    w = workload("b8_h16_t16384_d64_nu3_bf16")
    g = torch.Generator().manual_seed(7)
    x = torch.randn(w.B * w.H * w.T, w.d_k, generator=g).to(torch.bfloat16)
    phi = fwa.dpfp(x.to(DEV), w.nu)
    torch.cuda.synchronize()
    idx = torch.randint(0, x.shape[0], (2000,), generator=g)
    got = to_f64(phi[idx.to(DEV)])
    ref = oracle.dpfp(to_f64(x[idx]), w.nu)
    assert np.array_equal(got != 0.0, ref != 0.0)
    assert normwise(got, ref, 1) <= 4e-3


# ------------------------------------------------------------------------------ forward

FWD_CASES = [
    # name, overrides
    ("tiny_t64_d16_nu1_f32", {}),
    ("tiny_t64_d16_nu1_f32", {"chunk": 16}),
    ("tiny_t64_d16_nu1_f32", {"chunk": 32, "T": 77}),
    ("h8_t1024_d64_nu1_f32", {}),
    ("h8_t1024_d64_nu1_f32", {"chunk": 32, "T": 1000}),
    ("h8_t1024_d64_nu1_f32", {"T": 300, "w0_std": 0.05, "nu": 2, "chunk": 32}),
    ("h8_t1024_d64_nu1_f32", {"T": 200, "d_k": 32, "nu": 3, "d_v": 32}),
    # more chunks (576) than prep workgroups fit at once, ragged tail: the persistent prep
    ("h8_t1024_d64_nu1_f32", {"B": 3, "T": 1500, "w0_std": 0.05}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"T": 1000, "chunk": 32}),
    # 6 chunks (a multiple of the direct chain's register sets), ragged tail
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 379}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 333, "chunk": 16, "d_v": 16}),
    # chunk 128 (shift-sliced streaming path): full size, a ragged tail, d_v 32 with nu 1,
    # nu 4 (D 512) on 3 heads, and a single partial chunk
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"chunk": 128}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 1000, "chunk": 128, "nu": 3}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 2, "T": 300, "chunk": 128, "nu": 1, "d_v": 32}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 3, "T": 257, "chunk": 128, "nu": 4}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 2, "H": 1, "T": 45, "chunk": 128}),
    # d_v 16 at chunk 64 (16-column sliced serial kernel)
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 2, "T": 200, "d_v": 16}),
]


@pytest.mark.parametrize("name,ov", FWD_CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(FWD_CASES)])
def test_forward_parity(name, ov, path):
    w = workload(name, **ov)
    _skip_unless(path, w)
    log(f"forward[{path}] {w}")
    inp = make_inputs(w)
    y, Wf = _forward(_dev(inp), w.nu, w.chunk)
    yr, Wr = oracle_forward(inp, w.nu)
    ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
    log(f"  y err {ey:.3e}  W_final err {ew:.3e}")
    tol = TOL[w.torch_dtype]
    assert ey <= tol and ew <= tol


_FULL_PICKS = [(0, 0), (3, 7), (7, 15), (5, 2), (1, 11), (6, 9)]


@pytest.fixture(scope="module")
def full_size_case():
    """Inputs of the 8 x 16 x 16384 workload and the oracle on 6 sampled (b, h) slices."""
    w = workload("b8_h16_t16384_d64_nu3_bf16")
    inp = make_inputs(w)
    return w, inp, oracle_forward(inp, w.nu, bh_index=_FULL_PICKS)


@pytest.mark.parametrize("chunk", [64, 128])
def test_forward_full_size_long_sequence_sampled(path, full_size_case, chunk):
    """The 8 x 16 x 16384 (D 384, bf16) workload at full size, chunk 64 and 128, in the launch
    configuration the benchmark uses; the oracle checks 6 sampled (b, h) slices end to end."""
    w, inp, (yr, Wr) = full_size_case
    w = workload(w.name, chunk=chunk)
    _skip_unless(path, w)
    log(f"forward[{path}] full {w}")
    y, Wf = _forward(_dev(inp), w.nu, chunk)
    assert torch.isfinite(y.float()).all() and torch.isfinite(Wf).all()
    picks = _FULL_PICKS
    sel = tuple(torch.tensor(ix) for ix in zip(*picks))
    ey = normwise(to_f64(y.cpu()[sel])[None], yr, 2)
    ew = normwise(to_f64(Wf.cpu()[sel])[None], Wr, 2)
    log(f"  sampled y err {ey:.3e}  W_final err {ew:.3e}")
    assert ey <= 2e-2 and ew <= 2e-2


@pytest.mark.parametrize("kernel", ["pc", "sliced"])
def test_stream_kernels_full_size(full_size_case, monkeypatch, kernel):
    """The 8 x 16 x 16384 workload at chunk 64 on the producer / consumer and the sliced serial
    kernels, checked like the default one on 6 sampled (b, h) slices."""
    w, inp, (yr, Wr) = full_size_case
    monkeypatch.setenv("FWA_FORWARD_PATH", "stream")
    monkeypatch.setenv("FWA_STREAM_KERNEL", kernel)
    log(f"forward[stream {kernel}] full {w}")
    y, Wf = _forward(_dev(inp), w.nu, 64)
    sel = tuple(torch.tensor(ix) for ix in zip(*_FULL_PICKS))
    ey = normwise(to_f64(y.cpu()[sel])[None], yr, 2)
    ew = normwise(to_f64(Wf.cpu()[sel])[None], Wr, 2)
    log(f"  sampled y err {ey:.3e}  W_final err {ew:.3e}")
    assert ey <= 2e-2 and ew <= 2e-2


def test_forward_T0_and_empty(path):
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried" if path == "stream" else "h8_t1024_d64_nu1_f32",
                 T=0, w0_std=0.1)
    _skip_unless(path, workload(w.name, T=1))
    inp = _dev(make_inputs(w))
    y, Wf = _forward(inp, w.nu, 64)
    assert torch.equal(Wf, inp["W0"])
    y, Wf = _forward(inp, w.nu, 64, W0=False)
    assert torch.count_nonzero(Wf) == 0
    w = workload(w.name, B=0)
    inp = _dev(make_inputs(w))
    y, Wf = _forward(inp, w.nu, 64)
    assert y.numel() == 0


def test_forward_in_place_carry_and_segments(path):
    """forward(T1) then forward(T2) with W0 = W_final (in place) equals forward(T1 + T2)."""
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried", T=700, B=2)
    _skip_unless(path, w)
    inp = _dev(make_inputs(w))
    y, Wf = _forward(inp, w.nu, 64)
    W = inp["W0"].clone()
    ys = []
    for lo, hi in [(0, 300), (300, 301), (301, 700)]:
        sl = {k: inp[k][:, :, lo:hi].contiguous() for k in ("q", "k", "v", "beta_logit")}
        yy, _ = fwa.delta_forward(sl["q"], sl["k"], sl["v"], sl["beta_logit"], W, chunk=64,
                                  nu=w.nu, W_final=W)
        ys.append(yy)
    torch.cuda.synchronize()
    e1 = normwise(to_f64(torch.cat(ys, 2)), to_f64(y), 2)
    e2 = normwise(to_f64(W), to_f64(Wf), 2)
    log(f"  segmented vs whole: y {e1:.3e} W {e2:.3e}")
    assert e1 <= 2e-2 and e2 <= 2e-2


def test_forward_chunk_independence_and_determinism(monkeypatch):
    """Every (implementation, chunk) pair agrees with the others; each is deterministic."""
    w = workload("h8_t1024_d64_nu1_f32", T=500, w0_std=0.02)
    inp = _dev(make_inputs(w))
    outs = {}
    paths = ("chunked", "fused")           # fp32 inputs: the streaming path takes bf16 only
    for p in paths:
        monkeypatch.setenv("FWA_FORWARD_PATH", p)
        for c in ((32, 64) if p == "chunked" else (16, 32, 64)):
            outs[(p, c)] = _forward(inp, w.nu, c)
    ref = outs[("fused", 64)]
    for key, (y, Wf) in outs.items():
        assert normwise(to_f64(y), to_f64(ref[0]), 2) <= 1e-4, key
        assert normwise(to_f64(Wf), to_f64(ref[1]), 2) <= 1e-4, key
    for p in paths:
        monkeypatch.setenv("FWA_FORWARD_PATH", p)
        y2, W2 = _forward(inp, w.nu, 64)
        assert torch.equal(y2, outs[(p, 64)][0]) and torch.equal(W2, outs[(p, 64)][1])


@pytest.mark.parametrize("name,ov", [("h8_t1024_d64_nu1_f32", {"T": 555, "w0_std": 0.05}),
                                     ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 700})])
def test_chunked_prep_forms(monkeypatch, name, ov):
    """The chunked path's prep as two workgroups per chunk (K side and Q side) and as one,
    against the oracle and against each other; each form is deterministic."""
    monkeypatch.setenv("FWA_FORWARD_PATH", "chunked")
    w = workload(name, **ov)
    inp = make_inputs(w)
    d = _dev(inp)
    yr, Wr = oracle_forward(inp, w.nu)
    tol = TOL[w.torch_dtype]
    outs = {}
    for split in ("1", "0"):
        monkeypatch.setenv("FWA_PREP_SPLIT", split)
        y, Wf = _forward(d, w.nu, 64)
        ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
        log(f"  chunked prep split={split}: y err {ey:.3e}  W_final err {ew:.3e}")
        assert ey <= tol and ew <= tol
        y2, W2 = _forward(d, w.nu, 64)
        assert torch.equal(y, y2) and torch.equal(Wf, W2)
        outs[split] = (y, Wf)
    assert normwise(to_f64(outs["1"][0]), to_f64(outs["0"][0]), 2) <= tol
    assert normwise(to_f64(outs["1"][1]), to_f64(outs["0"][1]), 2) <= tol


@pytest.mark.parametrize("kernel,prep", [("default", "full"), ("default", "sliced"), ("sliced", "sliced"),
                                         ("pc", "sliced")])
def test_stream_prep_variants_and_chunks(monkeypatch, kernel, prep):
    """The streaming path with each serial kernel and prep kernel at chunk 64, and at chunk
    128, against the oracle and against each other; each is deterministic."""
    monkeypatch.setenv("FWA_FORWARD_PATH", "stream")
    monkeypatch.setenv("FWA_STREAM_KERNEL", kernel)
    monkeypatch.setenv("FWA_STREAM_PREP", prep)
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried", B=1, H=4, T=777, nu=3)
    inp = make_inputs(w)
    d = _dev(inp)
    yr, Wr = oracle_forward(inp, w.nu)
    outs = {}
    for c in (64, 128):
        y, Wf = _forward(d, w.nu, c)
        ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
        log(f"  stream kernel={kernel} prep={prep} chunk={c}: y err {ey:.3e}  W_final err {ew:.3e}")
        assert ey <= 2e-2 and ew <= 2e-2
        y2, W2 = _forward(d, w.nu, c)
        assert torch.equal(y, y2) and torch.equal(Wf, W2)
        outs[c] = (y, Wf)
    assert normwise(to_f64(outs[64][0]), to_f64(outs[128][0]), 2) <= 2e-2
    assert normwise(to_f64(outs[64][1]), to_f64(outs[128][1]), 2) <= 2e-2


def test_forward_unsupported_shapes_raise():
    q = torch.zeros(1, 1, 4, 64, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(fwa.FwaError) as e:          # D = 2*64*5 = 640 > 512
        fwa.delta_forward(q, q, q, torch.zeros(1, 1, 4, device=DEV, dtype=torch.bfloat16),
                          nu=5)
    assert e.value.status == fwa.FWA_ERR_UNSUPPORTED
    with pytest.raises(fwa.FwaError) as e:
        fwa.delta_forward(q, q, q, torch.zeros(1, 1, 4, device=DEV, dtype=torch.bfloat16),
                          chunk=48)
    assert e.value.status == fwa.FWA_ERR_INVALID_ARG


# ------------------------------------------------------------------------------ decode

# Few (b, h) slices make the step split each slice's rows over several workgroups: B*H = 24
# gives one row round per workgroup; B*H = 64 with d_v = 40 (5 rounds of 8 rows) gives two
# rounds per workgroup, a one-round part and an empty one.
@pytest.mark.parametrize("dtype,d_k,nu,d_v,B,H", [(torch.float32, 64, 1, 64, 8, 3),
                                                  (torch.bfloat16, 64, 3, 64, 8, 3),
                                                  (torch.float32, 16, 1, 16, 8, 3),
                                                  (torch.float32, 128, 2, 48, 8, 3),
                                                  (torch.bfloat16, 32, 4, 24, 8, 3),
                                                  (torch.float32, 64, 1, 40, 16, 4),
                                                  (torch.float32, 64, 1, 64, 1, 1)])
def test_step_parity_many_steps(dtype, d_k, nu, d_v, B, H):
    w = workload("decode_b256_h8_d64_nu1_f32", B=B, H=H, d_k=d_k, d_v=d_v, nu=nu,
                 dtype="bf16" if dtype == torch.bfloat16 else "f32", w0_std=0.05)
    steps = 40
    log(f"step {w} steps={steps}")
    inp = make_decode_inputs(w, steps=steps)
    dev = _dev(inp)
    W = dev["W0"].clone()
    ys = []
    for s in range(steps):
        # fresh copies: the entry point takes 16-byte aligned pointers, and a step's slice of a
        # small batch (beta at B*H = 1) is not
        ys.append(fwa.delta_step(dev["q"][s].clone(), dev["k"][s].clone(), dev["v"][s].clone(),
                                 dev["beta_logit"][s].clone(), W, nu=nu))
    torch.cuda.synchronize()
    # the oracle runs the same tokens as one T = steps sequence
    perm = lambda t: to_f64(t).transpose(1, 2, 0, *range(3, t.dim()))
    yr, Wr = oracle.delta_forward(perm(inp["q"]), perm(inp["k"]), perm(inp["v"]),
                                  to_f64(inp["beta_logit"]).transpose(1, 2, 0),
                                  to_f64(inp["W0"]), nu=nu)
    ey = normwise(to_f64(torch.stack(ys, 2)), yr, 2)
    ew = normwise(to_f64(W), Wr, 2)
    log(f"  y err {ey:.3e}  W err {ew:.3e}")
    assert ey <= TOL[dtype] and ew <= TOL[dtype]


def test_step_matches_forward_full_decode_shape():
    """The 256 x 8 (D 128) decode state at full size: 16 steps through fwa_delta_step equal
    fwa_delta_forward over the same 16 tokens, and a sample of slices matches the oracle."""
    w = workload("decode_b256_h8_d64_nu1_f32")
    inp = make_decode_inputs(w, steps=16)
    dev = _dev(inp)
    W = dev["W0"].clone()
    ys = [fwa.delta_step(dev["q"][s], dev["k"][s], dev["v"][s], dev["beta_logit"][s], W)
          for s in range(16)]
    perm = lambda t: t.permute(1, 2, 0, *range(3, t.dim())).contiguous()
    yf, Wf = fwa.delta_forward(perm(dev["q"]), perm(dev["k"]), perm(dev["v"]),
                               dev["beta_logit"].permute(1, 2, 0).contiguous(), dev["W0"],
                               chunk=16)
    torch.cuda.synchronize()
    ys = torch.stack(ys, 2)
    assert normwise(to_f64(ys), to_f64(yf), 2) <= 1e-4
    assert normwise(to_f64(W), to_f64(Wf), 2) <= 1e-4
    picks = [0, 77, 1000, 2047]
    flat = lambda t: to_f64(perm(t)).reshape(1, 2048, *perm(t).shape[2:])[:, picks]
    yr, Wr = oracle.delta_forward(flat(inp["q"]), flat(inp["k"]), flat(inp["v"]),
                                  to_f64(inp["beta_logit"].permute(1, 2, 0)).reshape(1, 2048, 16)[:, picks],
                                  to_f64(inp["W0"]).reshape(1, 2048, 64, 128)[:, picks])
    assert normwise(to_f64(ys).reshape(1, 2048, 16, 64)[:, picks], yr, 2) <= 1e-4
    assert normwise(to_f64(W).reshape(1, 2048, 64, 128)[:, picks], Wr, 2) <= 1e-4
