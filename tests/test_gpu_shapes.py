"""Parity of the forward over every chain-kernel configuration the chunked path's planner can
pick (each D it accepts, both dtypes, chunks of 32 and 64), over every memory split and roll
length of the streaming path, and over seeded random shapes (chunks 32, 64, 128) on all
implementations.  Same bars as test_gpu_parity: fp32 1e-4, bf16 2e-2 normwise per
(b, h) slice against the fp64 oracle."""
import random

import pytest
import torch

from parity_util import TOL, log, normwise, oracle_forward
from weight_linear_attention_amd import fwa
from weight_linear_attention_amd.synthetic import make_inputs, to_f64, workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _run(w, path):
    got, _ = fwa.delta_forward_info(w.B, w.H, w.T, w.d_k, w.d_v, w.nu, w.chunk, w.torch_dtype,
                                    path=path)
    assert got == path
    inp = make_inputs(w)
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    y, Wf = fwa.delta_forward(d["q"], d["k"], d["v"], d["beta_logit"], d["W0"], chunk=w.chunk,
                              nu=w.nu, path=path)
    torch.cuda.synchronize()
    yr, Wr = oracle_forward(inp, w.nu)
    ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
    log(f"  [{path}] {w.name} B{w.B} H{w.H} T{w.T} dk{w.d_k} dv{w.d_v} nu{w.nu} C{w.chunk} "
        f"{w.dtype}: y {ey:.2e}  W {ew:.2e}")
    tol = TOL[w.torch_dtype]
    assert ey <= tol and ew <= tol


# (d_k, nu) giving each D the chunked path accepts; the chain kernel's (waves, d-tiles per
# wave) differ between them (fp32: D 32 -> 2x1, 64 -> 4x1, 96 -> 6x1, 128 -> 4x2, 192 -> 6x2,
# 256 -> 8x2; bf16: 32 -> 1x2, 64 -> 2x2, 96 -> 3x2, 128 -> 4x2, 192 -> 6x2, 256 -> 4x4,
# 384 -> 6x4, 512 -> 8x4).
D_SHAPES = {32: (16, 1), 64: (32, 1), 96: (16, 3), 128: (64, 1), 192: (32, 3), 256: (64, 2),
            384: (64, 3), 512: (64, 4)}
CASES = []
for dt, Ds in (("f32", (32, 64, 96, 128, 192, 256)), ("bf16", (32, 64, 96, 128, 192, 256, 384, 512))):
    for D in Ds:
        for C in (32, 64):
            CASES.append((dt, D, C))


@pytest.mark.parametrize("dt,D,C", CASES, ids=[f"{a}-D{b}-C{c}" for a, b, c in CASES])
def test_chunked_every_chain_config(dt, D, C):
    d_k, nu = D_SHAPES[D]
    w = workload("h8_t1024_d64_nu1_f32", B=1, H=2, T=3 * C + 11, d_k=d_k, nu=nu,
                 d_v=32 if D >= 384 else 64, dtype=dt, chunk=C, w0_std=0.05,
                 seed=7000 + D + C)
    try:
        fwa.delta_forward_info(w.B, w.H, w.T, d_k, w.d_v, nu, C, w.torch_dtype, path="chunked")
    except fwa.FwaError as e:
        assert e.status == fwa.FWA_ERR_UNSUPPORTED
        pytest.skip(f"the chunked path does not take this shape: {e}")
    _run(w, "chunked")


# Streaming path at chunk 64 (bf16).  The planner takes the full-tile serial kernel for d_v in
# {32, 64} and D in {128, 256, 384} (each D a different number of memory d-tiles per wave, 1-3;
# each d_k a different roll window; nu up to 8 the longest roll the extended q rows hold), with
# the shift-sliced prep for d_k = 64 and the full-tile compact prep for d_k 16 and 32.  It falls
# back to the shift-sliced serial kernel (16-column workgroups, d_k = 64, nu <= 4) for d_v 16 and
# D 512.  T covers a lone partial chunk, an exact chunk and ragged tails.  Shapes neither kernel
# takes are refused.
STREAM_CASES = [
    # (d_k, nu, d_v, B, H, T)
    (64, 1, 64, 1, 2, 203), (64, 2, 64, 2, 2, 64), (64, 3, 32, 1, 3, 17), (64, 4, 64, 1, 2, 140),
    (64, 3, 16, 2, 1, 150), (64, 1, 16, 1, 1, 64),
    (32, 2, 64, 1, 2, 129), (32, 4, 32, 2, 1, 200), (32, 6, 64, 1, 1, 75), (16, 4, 64, 1, 2, 100),
    (16, 8, 32, 1, 2, 190), (16, 12, 64, 1, 1, 70),
    (64, 3, 64, 1, 2, 300),           # an odd chunk count above one (the chunk loop's tail)
]


@pytest.mark.parametrize("case", STREAM_CASES,
                         ids=[f"dk{c[0]}-nu{c[1]}-dv{c[2]}-T{c[5]}" for c in STREAM_CASES])
def test_stream_every_split(case):
    d_k, nu, d_v, B, H, T = case
    w = workload("b4_h8_t4096_d64_nu2_bf16_carried", B=B, H=H, T=T, d_k=d_k, nu=nu, d_v=d_v,
                 chunk=64, w0_std=0.05, seed=9000 + d_k * 10 + nu)
    sliced_ok = d_k == 64 and nu <= 4
    full_ok = nu <= 8 and 2 * d_k * nu <= 384 and d_v % 32 == 0
    if not (full_ok or sliced_ok):
        with pytest.raises(fwa.FwaError) as e:
            fwa.delta_forward_info(B, H, T, d_k, d_v, nu, 64, w.torch_dtype, path="stream")
        assert e.value.status == fwa.FWA_ERR_UNSUPPORTED
        return
    _run(w, "stream")


def _random_cases(n, seed):
    rng = random.Random(seed)
    out = []
    while len(out) < n:
        d_k = rng.choice((16, 32, 64))
        d_v = rng.choice((16, 32, 64))
        nu = rng.choice((1, 2, 3, 4))
        if 2 * d_k * nu > 512:
            continue
        dt = rng.choice(("f32", "bf16"))
        C = rng.choice((32, 64, 128))
        B, H = rng.choice(((1, 1), (1, 3), (2, 4), (3, 8)))
        T = rng.randint(1, 300)
        w0 = rng.choice((None, 0.02))
        out.append((len(out), B, H, T, d_k, d_v, nu, dt, C, w0))
    return out


RANDOM = _random_cases(24, 20261202)


@pytest.mark.parametrize("case", RANDOM, ids=[f"r{c[0]}" for c in RANDOM])
def test_random_shapes_every_path(case):
    i, B, H, T, d_k, d_v, nu, dt, C, w0 = case
    w = workload("h8_t1024_d64_nu1_f32", B=B, H=H, T=T, d_k=d_k, d_v=d_v, nu=nu, dtype=dt,
                 chunk=C, w0_std=w0, seed=8000 + i)
    ran = 0
    for path in ("chunked", "stream", "fused"):
        try:
            fwa.delta_forward_info(B, H, T, d_k, d_v, nu, C, w.torch_dtype, path=path)
        except fwa.FwaError as e:
            assert e.status == fwa.FWA_ERR_UNSUPPORTED
            log(f"  [{path}] unsupported: {e}")
            continue
        _run(w, path)
        ran += 1
    if ran == 0:
        pytest.skip("neither implementation takes this shape")
