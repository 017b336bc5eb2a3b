"""The linear maps around the layer (fwa_layer_project, fwa_layer_output) and the multi-layer
token-wise decode (fwa_decode_layers), through the C ABI, against the fp64 oracle composed the
same way: projections, then the layer oracle, then the output map.  Random-init weights
(N(0, 1/d_model)) at the pages' layer shape (d_model 512, 8 heads of 64).  Bars: fp32 1e-4,
bf16 2e-2, normwise per slice."""
import pytest
import torch

import oracle
from parity_util import TOL, log, normwise
from weight_linear_attention_amd import fwa
from weight_linear_attention_amd.synthetic import to_f64

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _weights(seed, d_model, H, d_k, d_v, dtype, L=1):
    g = torch.Generator().manual_seed(seed)
    out = []
    for _ in range(L):
        N = 2 * H * d_k + H * d_v + H
        Wp = torch.randn(N, d_model, generator=g) / d_model ** 0.5
        Wo = torch.randn(d_model, H * d_v, generator=g) / (H * d_v) ** 0.5
        bo = torch.randn(d_model, generator=g) * 0.1
        out.append(tuple(t.to(dtype) for t in (Wp, Wo, bo)))
    return out


@pytest.mark.parametrize("B,T,d_model,H,d_k,d_v,dtype", [
    (1, 1024, 512, 8, 64, 64, torch.float32),
    (4, 256, 512, 8, 64, 64, torch.bfloat16),
    (2, 77, 136, 3, 16, 24, torch.float32),
    (3, 45, 72, 5, 32, 8, torch.bfloat16),
    # ragged rows, columns and k runs with 32-row tiles (the projection here; both maps below)
    (3, 333, 264, 5, 40, 48, torch.float32),
    (2, 700, 520, 4, 32, 40, torch.bfloat16),
])
def test_layer_project_and_output(B, T, d_model, H, d_k, d_v, dtype):
    log(f"layer maps B{B} T{T} d_model{d_model} H{H} d_k{d_k} d_v{d_v} {dtype}")
    g = torch.Generator().manual_seed(B * 1000 + T)
    x = torch.randn(B, T, d_model, generator=g).to(dtype)
    (Wp, Wo, bo), = _weights(T, d_model, H, d_k, d_v, dtype)
    got = fwa.layer_project(x.to(DEV), Wp.to(DEV), H, d_k, d_v)
    ref = oracle.layer_project(to_f64(x), to_f64(Wp), H, d_k, d_v)
    errs = [normwise(to_f64(a), r, 2) for a, r in zip(got, ref)]
    y = torch.randn(B, H, T, d_v, generator=g).to(dtype)
    res = torch.randn(B, T, d_model, generator=g).to(dtype)
    o1 = fwa.layer_output(y.to(DEV), Wo.to(DEV), bo.to(DEV), res.to(DEV))
    rd = res.to(DEV).clone()
    o2 = fwa.layer_output(y.to(DEV), Wo.to(DEV), bo.to(DEV), rd, out=rd)      # in place
    o3 = fwa.layer_output(y.to(DEV), Wo.to(DEV))
    torch.cuda.synchronize()
    r1 = oracle.layer_output(to_f64(y), to_f64(Wo), to_f64(bo), to_f64(res))
    r3 = oracle.layer_output(to_f64(y), to_f64(Wo))
    errs += [normwise(to_f64(o1), r1, 1), normwise(to_f64(o3), r3, 1)]
    assert torch.equal(o1, o2)
    log("  errors " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= TOL[dtype]


@pytest.mark.parametrize("dtype,T", [(torch.float32, 1024), (torch.bfloat16, 512)])
def test_layer_forward_composed(dtype, T):
    """x -> projections -> fwa_delta_forward -> output map with the residual, at the pages'
    layer shape, against the oracle composed the same way."""
    B, d_model, H, d, nu = 2, 512, 8, 64, 1
    g = torch.Generator().manual_seed(77)
    x = torch.randn(B, T, d_model, generator=g).to(dtype)
    (Wp, Wo, bo), = _weights(78, d_model, H, d, d, dtype)
    xd = x.to(DEV)
    q, k, v, bl = fwa.layer_project(xd, Wp.to(DEV), H, d, d)
    y, _ = fwa.delta_forward(q, k, v, bl, None, nu=nu)
    out = fwa.layer_output(y, Wo.to(DEV), bo.to(DEV), xd)
    torch.cuda.synchronize()
    rq, rk, rv, rb = oracle.layer_project(to_f64(x), to_f64(Wp), H, d, d)
    # the oracle layer runs on the projections rounded as the GPU stores them (bf16 runs)
    cast = (lambda a: to_f64(torch.from_numpy(a).to(dtype))) if dtype == torch.bfloat16 else (lambda a: a)
    ry, _ = oracle.delta_forward(cast(rq), cast(rk), cast(rv), cast(rb), None, nu=nu)
    rout = oracle.layer_output(cast(ry), to_f64(Wo), to_f64(bo), to_f64(x))
    e = normwise(to_f64(out), rout, 1)
    log(f"  composed layer {dtype} T{T}: out err {e:.2e}")
    assert e <= TOL[dtype]


def _oracle_decode(x, layers, Ws, H, d_k, d_v, nu, tokens):
    """The oracle's decode: per token (its embedding as the layer input), per layer:
    projections, one delta step, output map with the residual."""
    x = to_f64(x)
    Ws = [to_f64(W) for W in Ws]
    outs = []
    for tok in tokens:
        x = to_f64(tok)
        for l, (Wp, Wo, bo) in enumerate(layers):
            q, k, v, bl = oracle.layer_project(x[:, None], to_f64(Wp), H, d_k, d_v)
            y, Ws[l] = oracle.delta_step(q[:, :, 0], k[:, :, 0], v[:, :, 0], bl[:, :, 0], Ws[l], nu=nu)
            x = oracle.layer_output(y[:, :, None], to_f64(Wo), to_f64(bo), x[:, None])[:, 0]
        outs.append(x.copy())
    return outs, Ws


def test_decode_layers_matches_separate_calls_and_oracle():
    """Eight tokens through three layers with fwa_decode_layers equal the same steps issued as
    separate fwa_layer_project / fwa_delta_step / fwa_layer_output calls bit for bit, and the
    oracle's composition within the fp32 bar."""
    B, d_model, H, d, nu, L = 32, 512, 8, 64, 1, 3
    layers = _weights(90, d_model, H, d, d, torch.float32, L)
    g = torch.Generator().manual_seed(91)
    tokens = [torch.randn(B, d_model, generator=g) for _ in range(8)]
    W0 = [torch.randn(B, H, d, 2 * d * nu, generator=g) * 0.02 for _ in range(L)]
    dl = [tuple(t.to(DEV) for t in p) for p in layers]
    x = torch.zeros(B, d_model, device=DEV)
    Ws = [W.to(DEV) for W in W0]
    x2 = torch.zeros(B, d_model, device=DEV)
    Ws2 = [W.to(DEV) for W in W0]
    outs = []
    for tok in tokens:
        x.copy_(tok)
        fwa.decode_layers(x, dl, Ws, H, d, d, nu)
        outs.append(x.clone())
        x2.copy_(tok)
        for l, (Wp, Wo, bo) in enumerate(dl):
            q, k, v, bl = fwa.layer_project(x2[:, None], Wp, H, d, d)
            y = fwa.delta_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(),
                               v[:, :, 0].contiguous(), bl[:, :, 0].contiguous(), Ws2[l], nu=nu)
            fwa.layer_output(y[:, :, None], Wo, bo, x2[:, None], out=x2[:, None])
        assert torch.equal(x, x2)
    torch.cuda.synchronize()
    for a, b in zip(Ws, Ws2):
        assert torch.equal(a, b)
    ref, rW = _oracle_decode(torch.zeros(B, d_model), layers, W0, H, d, d, nu, tokens)
    ex = max(normwise(to_f64(o)[None], r[None], 1) for o, r in zip(outs, ref))
    ew = max(normwise(to_f64(W), r, 2) for W, r in zip(Ws, rW))
    log(f"  decode 3 layers x 8 tokens: x err {ex:.2e}  W err {ew:.2e}")
    assert ex <= 1e-4 and ew <= 1e-4


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_layers_in_hip_graph(dtype):
    """One token through four layers captured once in a HIP graph and replayed for six tokens
    (the token's embedding copied into x before each replay) equals eager calls bit for bit."""
    B, d_model, H, d, nu, L = 64, 512, 8, 64, 1, 4
    layers = [tuple(t.to(DEV) for t in p) for p in _weights(95, d_model, H, d, d, dtype, L)]
    g = torch.Generator().manual_seed(96)
    tokens = [torch.randn(B, d_model, generator=g).to(dtype).to(DEV) for _ in range(6)]
    W_e = [torch.zeros(B, H, d, 2 * d * nu, device=DEV) for _ in range(L)]
    W_g = [torch.zeros(B, H, d, 2 * d * nu, device=DEV) for _ in range(L)]
    x_e = torch.zeros(B, d_model, dtype=dtype, device=DEV)
    x_g = torch.zeros(B, d_model, dtype=dtype, device=DEV)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=DEV)
    # warm-up on a scratch copy (nothing to set up, but keeps capture free of first-call work)
    fwa.decode_layers(x_g.clone(), layers, [W.clone() for W in W_g], H, d, d, nu, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwa.decode_layers(x_g, layers, W_g, H, d, d, nu, workspace=ws)
    for tok in tokens:
        x_e.copy_(tok)
        fwa.decode_layers(x_e, layers, W_e, H, d, d, nu)
        x_g.copy_(tok)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(x_g, x_e)
    for a, b in zip(W_g, W_e):
        assert torch.equal(a, b)
