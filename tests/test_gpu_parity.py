"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Bars: fp32 inputs 1e-4, bf16 inputs 2e-2 (fp32 state), normwise per (b, h) slice; the DPFP
zero/nonzero pattern must match the oracle's sign predicate bit for bit.  Every forward test
runs once per implementation (chunked, stream, fused) that takes its shape, named through
fwa_delta_forward_path.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import TOL, log, normwise, oracle_forward, oracle_forward_batched
from weight_linear_attention_amd import fwa
from weight_linear_attention_amd.synthetic import (EDGE_CASES, make_decode_inputs,
                                                   make_edge_inputs, make_inputs, to_f64,
                                                   workload)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


FORWARD_PATHS = ["chunked", "stream", "fused"]


@pytest.fixture(params=FORWARD_PATHS)
def path(request):
    """Runs a forward test once per implementation."""
    return request.param


def _skip_unless(path, w):
    """Skips when the named implementation does not take this shape."""
    try:
        got, _ = fwa.delta_forward_info(w.B, w.H, w.T, w.d_k, w.d_v, w.nu, w.chunk,
                                        w.torch_dtype, path=path)
    except fwa.FwaError as e:
        assert e.status == fwa.FWA_ERR_UNSUPPORTED
        pytest.skip(f"the {path} path does not take this shape: {e}")
    assert got in (path, "none")


def _forward(inp_d, nu, chunk, W0=True, path="auto"):
    y, Wf = fwa.delta_forward(inp_d["q"], inp_d["k"], inp_d["v"], inp_d["beta_logit"],
                              inp_d["W0"] if W0 else None, chunk=chunk, nu=nu, path=path)
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


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dpfp_degenerate_vectors(dtype):
    """Zero vectors, keys near eps (k scaled by 1e-3 at d_k 16) and alternating signs, against
    the oracle; the mask stays bit-exact."""
    g = torch.Generator().manual_seed(99)
    x = torch.randn(300, 16, generator=g)
    x[:50] = 0.0
    x[50:150] *= 1e-3
    x[150:200] = torch.tensor([(-1.0) ** j for j in range(16)]) * x[150:200].abs()
    x = x.to(dtype)
    for nu in (1, 3):
        phi = fwa.dpfp(x.to(DEV), nu)
        torch.cuda.synchronize()
        got, ref = to_f64(phi), oracle.dpfp(to_f64(x), nu)
        assert np.array_equal(got != 0.0, oracle.dpfp_mask(to_f64(x), nu))
        assert not got[:50].any()
        assert normwise(got[50:], ref[50:], 1) <= (1e-6 if dtype == torch.float32 else 4e-3)


def test_dpfp_empty_and_full_size():
    """The q tensor of the 8 x 16 x 16384 workload (2.1M vectors) in full: mask bit-exact and
    every vector within the bf16 bar."""
    x = torch.empty(0, 64, device=DEV)
    assert fwa.dpfp(x, 3).shape == (0, 384)
    w = workload("b8_h16_t16384_d64_nu3_bf16")
    q = make_inputs(w)["q"].reshape(-1, w.d_k)
    phi = fwa.dpfp(q.to(DEV), w.nu)
    torch.cuda.synchronize()
    n = q.shape[0]
    worst = 0.0
    for lo in range(0, n, 1 << 18):
        xs = to_f64(q[lo:lo + (1 << 18)])
        got = to_f64(phi[lo:lo + (1 << 18)])
        assert np.array_equal(got != 0.0, oracle.dpfp_mask(xs, w.nu))
        worst = max(worst, normwise(got, oracle.dpfp(xs, w.nu), 1))
    log(f"  full-size DPFP worst normwise err {worst:.3e}")
    assert worst <= 4e-3


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
    # the chunked prep in each of its three forms: two workgroups per chunk (72 chunks, twice
    # that fits at once), one per chunk (256 chunks), persistent (576 chunks, a ragged tail)
    ("h8_t1024_d64_nu1_f32", {"T": 555, "w0_std": 0.05}),
    ("h8_t1024_d64_nu1_f32", {"B": 2, "w0_std": 0.05}),
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
    # the streaming path's full-tile compact prep (d_k 32 and 16) at chunk 64
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 4, "T": 777, "d_k": 32, "nu": 4}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 4, "T": 500, "d_k": 16, "nu": 4}),
]


@pytest.mark.parametrize("name,ov", FWD_CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(FWD_CASES)])
def test_forward_parity(name, ov, path):
    w = workload(name, **ov)
    _skip_unless(path, w)
    log(f"forward[{path}] {w}")
    inp = make_inputs(w)
    y, Wf = _forward(_dev(inp), w.nu, w.chunk, path=path)
    yr, Wr = oracle_forward(inp, w.nu)
    ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
    log(f"  y err {ey:.3e}  W_final err {ew:.3e}")
    tol = TOL[w.torch_dtype]
    assert ey <= tol and ew <= tol


# The method's edge cases on the first three workloads' shapes (the long ones shortened so the
# oracle stays within seconds), on every implementation that takes them; tiny_keys also at d_k
# 16 in bf16 and with a carried memory.
EDGE_SHAPES = [
    ("tiny_t64_d16_nu1_f32", {"T": 150}),
    ("h8_t1024_d64_nu1_f32", {"T": 300}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 700}),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 4, "T": 300, "d_k": 16, "nu": 4}),
]


@pytest.mark.parametrize("case", EDGE_CASES)
@pytest.mark.parametrize("name,ov", EDGE_SHAPES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(EDGE_SHAPES)])
def test_forward_edge_cases(name, ov, case, path):
    w = workload(name, **ov)
    _skip_unless(path, w)
    log(f"forward[{path}] edge {case} {w}")
    inp = make_edge_inputs(w, case)
    y, Wf = _forward(_dev(inp), w.nu, w.chunk, path=path)
    yr, Wr = oracle_forward(inp, w.nu)
    ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
    log(f"  y err {ey:.3e}  W_final err {ew:.3e}")
    tol = TOL[w.torch_dtype]
    assert ey <= tol and ew <= tol
    assert torch.isfinite(y.float()).all() and torch.isfinite(Wf).all()


@pytest.fixture(scope="module")
def full_size_case():
    """Inputs of the 8 x 16 x 16384 workload (D 384, bf16) and the oracle on all 128 (b, h)
    slices, computed once, one batch row of 16 slices at a time."""
    w = workload("b8_h16_t16384_d64_nu3_bf16")
    inp = make_inputs(w)
    log("oracle on the 8 x 16 x 16384 workload (128 slices)")
    return w, inp, oracle_forward_batched(inp, w.nu)


@pytest.mark.parametrize("chunk", [64, 128])
def test_forward_full_size_long_sequence(path, full_size_case, chunk):
    """The 8 x 16 x 16384 workload at full size, chunk 64 and 128, in the launch configuration
    the benchmark uses, against the oracle on every (b, h) slice."""
    w, inp, (yr, Wr) = full_size_case
    w = workload(w.name, chunk=chunk)
    _skip_unless(path, w)
    log(f"forward[{path}] full {w}")
    y, Wf = _forward(_dev(inp), w.nu, chunk, path=path)
    ycpu, Wcpu = y.cpu(), Wf.cpu()
    del y, Wf
    ey = max(normwise(to_f64(ycpu[b]), yr[b], 1) for b in range(w.B))
    ew = normwise(to_f64(Wcpu), Wr, 2)
    log(f"  all 128 slices: y err {ey:.3e}  W_final err {ew:.3e}")
    assert ey <= 2e-2 and ew <= 2e-2


def test_forward_T0_and_empty(path):
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried" if path == "stream" else "h8_t1024_d64_nu1_f32",
                 T=0, w0_std=0.1)
    _skip_unless(path, workload(w.name, T=1))
    inp = _dev(make_inputs(w))
    y, Wf = _forward(inp, w.nu, 64, path=path)
    assert torch.equal(Wf, inp["W0"])
    y, Wf = _forward(inp, w.nu, 64, W0=False, path=path)
    assert torch.count_nonzero(Wf) == 0
    w = workload(w.name, B=0)
    inp = _dev(make_inputs(w))
    y, Wf = _forward(inp, w.nu, 64, path=path)
    assert y.numel() == 0


def test_forward_in_place_carry_and_segments(path):
    """forward(T1) then forward(T2) with W0 = W_final (in place) equals forward(T1 + T2)."""
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried", T=700, B=2)
    _skip_unless(path, w)
    inp = _dev(make_inputs(w))
    y, Wf = _forward(inp, w.nu, 64, path=path)
    W = inp["W0"].clone()
    ys = []
    for lo, hi in [(0, 300), (300, 301), (301, 700)]:
        sl = {k: inp[k][:, :, lo:hi].contiguous() for k in ("q", "k", "v", "beta_logit")}
        yy, _ = fwa.delta_forward(sl["q"], sl["k"], sl["v"], sl["beta_logit"], W, chunk=64,
                                  nu=w.nu, W_final=W, path=path)
        ys.append(yy)
    torch.cuda.synchronize()
    e1 = normwise(to_f64(torch.cat(ys, 2)), to_f64(y), 2)
    e2 = normwise(to_f64(W), to_f64(Wf), 2)
    log(f"  segmented vs whole: y {e1:.3e} W {e2:.3e}")
    assert e1 <= 2e-2 and e2 <= 2e-2


def test_forward_chunk_independence_and_determinism():
    """Every (implementation, chunk) pair agrees with the others; each is deterministic."""
    w = workload("h8_t1024_d64_nu1_f32", T=500, w0_std=0.02)
    inp = _dev(make_inputs(w))
    outs = {}
    paths = ("chunked", "fused")           # fp32 inputs: the streaming path takes bf16 only
    for p in paths:
        for c in ((32, 64) if p == "chunked" else (16, 32, 64)):
            outs[(p, c)] = _forward(inp, w.nu, c, path=p)
    ref = outs[("fused", 64)]
    for key, (y, Wf) in outs.items():
        assert normwise(to_f64(y), to_f64(ref[0]), 2) <= 1e-4, key
        assert normwise(to_f64(Wf), to_f64(ref[1]), 2) <= 1e-4, key
    for p in paths:
        y2, W2 = _forward(inp, w.nu, 64, path=p)
        assert torch.equal(y2, outs[(p, 64)][0]) and torch.equal(W2, outs[(p, 64)][1])


def test_stream_chunks_agree_and_are_deterministic():
    """The streaming path at chunk 64 and 128 against the oracle and each other; each is
    deterministic."""
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried", B=1, H=4, T=777, nu=3)
    inp = make_inputs(w)
    d = _dev(inp)
    yr, Wr = oracle_forward(inp, w.nu)
    outs = {}
    for c in (64, 128):
        y, Wf = _forward(d, w.nu, c, path="stream")
        ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
        log(f"  stream chunk={c}: y err {ey:.3e}  W_final err {ew:.3e}")
        assert ey <= 2e-2 and ew <= 2e-2
        y2, W2 = _forward(d, w.nu, c, path="stream")
        assert torch.equal(y, y2) and torch.equal(Wf, W2)
        outs[c] = (y, Wf)
    assert normwise(to_f64(outs[64][0]), to_f64(outs[128][0]), 2) <= 2e-2
    assert normwise(to_f64(outs[64][1]), to_f64(outs[128][1]), 2) <= 2e-2


GRAPH_CASES = [
    ("h8_t1024_d64_nu1_f32", {}, "auto"),                                   # chunked, fp32
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 1000}, "auto"),     # chunked, bf16, W0
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 1000, "nu": 3}, "stream"),
    ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 1000, "chunk": 128}, "stream"),
    ("h8_t1024_d64_nu1_f32", {"T": 300}, "fused"),
]


@pytest.mark.parametrize("name,ov,fpath", GRAPH_CASES, ids=[f"{c[0]}-{c[2]}-{i}" for i, c in enumerate(GRAPH_CASES)])
def test_forward_in_hip_graph(name, ov, fpath):
    """One forward captured in a HIP graph (its workspace allocated inside the capture),
    replayed three times with eager forwards on other inputs in between; every replay equals
    the eager result bit for bit and matches the oracle."""
    w = workload(name, **ov)
    inp = make_inputs(w)
    d = _dev(inp)
    other = _dev(make_inputs(w, seed=w.seed + 50))
    y_eager, W_eager = _forward(d, w.nu, w.chunk, path=fpath)      # also sets kernel attributes
    y_st = torch.empty_like(y_eager)
    W_st = torch.empty_like(W_eager)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwa.delta_forward(d["q"], d["k"], d["v"], d["beta_logit"], d["W0"], chunk=w.chunk,
                          nu=w.nu, out=y_st, W_final=W_st, path=fpath)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fwa.delta_forward(d["q"], d["k"], d["v"], d["beta_logit"], d["W0"], chunk=w.chunk,
                          nu=w.nu, out=y_st, W_final=W_st, path=fpath)
    yr, Wr = oracle_forward(inp, w.nu)
    for r in range(3):
        y_st.fill_(float("nan"))
        W_st.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_st, y_eager) and torch.equal(W_st, W_eager), f"replay {r}"
        ey, ew = normwise(to_f64(y_st), yr, 2), normwise(to_f64(W_st), Wr, 2)
        assert ey <= TOL[w.torch_dtype] and ew <= TOL[w.torch_dtype]
        _forward(other, w.nu, w.chunk, path=fpath)                  # eager work between replays
    log(f"  graph replays match eager and the oracle ({fpath})")


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


def test_forward_workspace_too_small_raises():
    w = workload("h8_t1024_d64_nu1_f32", T=100)
    d = _dev(make_inputs(w))
    _, need = fwa.delta_forward_info(w.B, w.H, w.T, w.d_k, w.d_v, w.nu, w.chunk, w.torch_dtype)
    assert need > 0
    ws = torch.empty(need - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(fwa.FwaError) as e:
        fwa.delta_forward(d["q"], d["k"], d["v"], d["beta_logit"], None, nu=w.nu, workspace=ws)
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


def test_step_full_decode_workload_1024_steps():
    """The decode workload in full: 1024 successive fwa_delta_step calls on the persistent
    [256, 8, 64, 128] fp32 state, each step with fresh tokens (as the benchmark runs it),
    against the oracle's T = 1024 forward on all 2048 (b, h) slices: y of every step and the
    final state."""
    w = workload("decode_b256_h8_d64_nu1_f32")
    S = w.steps
    inp = make_decode_inputs(w, steps=S)
    dev = _dev(inp)
    W = dev["W0"].clone()
    ys = torch.empty(S, w.B, w.H, w.d_v, device=DEV)
    for s in range(S):
        fwa.delta_step(dev["q"][s], dev["k"][s], dev["v"][s], dev["beta_logit"][s], W, out=ys[s])
    torch.cuda.synchronize()
    del dev
    log("oracle: 1024 steps over 2048 slices")
    perm = lambda t: np.ascontiguousarray(to_f64(t).transpose(1, 2, 0, *range(3, t.dim())))
    yr, Wr = oracle.delta_forward(perm(inp["q"]), perm(inp["k"]), perm(inp["v"]),
                                  perm(inp["beta_logit"]), to_f64(inp["W0"]), nu=w.nu)
    ey = normwise(perm(ys.cpu()), yr, 2)
    ew = normwise(to_f64(W), Wr, 2)
    log(f"  all 2048 slices, 1024 steps: y err {ey:.3e}  W err {ew:.3e}")
    assert ey <= 1e-4 and ew <= 1e-4


def test_step_matches_forward_full_decode_shape():
    """The 256 x 8 (D 128) decode state at full size: 16 steps through fwa_delta_step equal
    fwa_delta_forward over the same 16 tokens."""
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


@pytest.mark.parametrize("case", EDGE_CASES)
def test_step_edge_cases(case):
    """The decode step on the method's edge cases (tokens of one sequence fed one by one)."""
    w = workload("tiny_t64_d16_nu1_f32", B=2, H=3, T=120, w0_std=0.05)
    inp = make_edge_inputs(w, case)
    d = _dev(inp)
    W = d["W0"].clone()
    ys = []
    for t in range(w.T):
        sl = {n: d[n][:, :, t].contiguous() for n in ("q", "k", "v", "beta_logit")}
        ys.append(fwa.delta_step(sl["q"], sl["k"], sl["v"], sl["beta_logit"], W, nu=w.nu))
    torch.cuda.synchronize()
    yr, Wr = oracle_forward(inp, w.nu)
    ey, ew = normwise(to_f64(torch.stack(ys, 2)), yr, 2), normwise(to_f64(W), Wr, 2)
    log(f"  step edge {case}: y err {ey:.3e}  W err {ew:.3e}")
    assert ey <= 1e-4 and ew <= 1e-4


def test_step_in_hip_graph():
    """Eight successive decode steps captured in one HIP graph and replayed twice (sixteen
    steps in all) equal sixteen eager steps bit for bit."""
    w = workload("decode_b256_h8_d64_nu1_f32", B=32)
    inp = _dev(make_decode_inputs(w, steps=8))
    W_eager = inp["W0"].clone()
    ys_eager = []
    for rep in range(2):
        for s in range(8):
            ys_eager.append(fwa.delta_step(inp["q"][s], inp["k"][s], inp["v"][s],
                                           inp["beta_logit"][s], W_eager))
    W = inp["W0"].clone()
    ys = torch.empty(8, w.B, w.H, w.d_v, device=DEV)
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for s in range(8):
            fwa.delta_step(inp["q"][s], inp["k"][s], inp["v"][s], inp["beta_logit"][s], W,
                           out=ys[s])
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        for s in range(8):
            assert torch.equal(ys[s], ys_eager[8 * rep + s]), (rep, s)
    assert torch.equal(W, W_eager)
