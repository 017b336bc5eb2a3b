"""fwa_delta_forward_noalloc (the forward that takes its scratch from a static device array)
against fwa_delta_forward on the same inputs, through the C ABI: two calls in a row, the second
with a smaller input, on the planned implementation and on the fused one that runs where the
plan needs more scratch than the static array holds."""
import ctypes

import pytest
import torch

from parity_util import TOL, log, normwise, oracle_forward
from weight_linear_attention_amd import fwa
from weight_linear_attention_amd.synthetic import make_inputs, to_f64, workload

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SCRATCH_BYTES = 64 << 20


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(d, w):
    y = torch.full((w.B, w.H, w.T, w.d_v), float("nan"), dtype=w.torch_dtype, device=DEV)
    Wf = torch.full((w.B, w.H, w.d_v, w.D), float("nan"), dtype=torch.float32, device=DEV)
    st = fwa.lib().fwa_delta_forward_noalloc(
        _p(d["q"]), _p(d["k"]), _p(d["v"]), _p(d["beta_logit"]), _p(d["W0"]), _p(y), _p(Wf),
        w.B, w.H, w.T, w.d_k, w.d_v, w.nu, w.chunk, fwa._dtype_code(w.torch_dtype),
        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    fwa._check(st)
    return y, Wf


# each pair: a first call, then a smaller one (fewer heads and steps) on the same scratch
PAIRS = [
    (("h8_t1024_d64_nu1_f32", {"w0_std": 0.05}), ("h8_t1024_d64_nu1_f32", {"H": 3, "T": 333})),
    (("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 2000}),
     ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "H": 2, "T": 700})),
    # the plan needs 253 MB of workspace, more than the scratch: the fused implementation runs
    (("b4_h8_t4096_d64_nu2_bf16_carried", {}), ("b4_h8_t4096_d64_nu2_bf16_carried", {"B": 1, "T": 999})),
]


@pytest.mark.parametrize("pair", PAIRS, ids=["fp32-chunked", "bf16-chunked", "bf16-fused"])
def test_noalloc_matches_forward_on_two_calls(pair):
    for name, ov in pair:
        w = workload(name, **ov)
        path, need = fwa.delta_forward_info(w.B, w.H, w.T, w.d_k, w.d_v, w.nu, w.chunk,
                                            w.torch_dtype)
        expect = path if need <= SCRATCH_BYTES else "fused"
        log(f"noalloc {w} plan={path} ({need} B of workspace) -> {expect}")
        inp = make_inputs(w)
        d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
        y_ref, W_ref = fwa.delta_forward(d["q"], d["k"], d["v"], d["beta_logit"], d["W0"],
                                         chunk=w.chunk, nu=w.nu, path=expect)
        y, Wf = _noalloc(d, w)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref) and torch.equal(Wf, W_ref)
        yr, Wr = oracle_forward(inp, w.nu)
        ey, ew = normwise(to_f64(y), yr, 2), normwise(to_f64(Wf), Wr, 2)
        log(f"  y err {ey:.3e}  W_final err {ew:.3e}")
        assert ey <= TOL[w.torch_dtype] and ew <= TOL[w.torch_dtype]


def test_noalloc_refuses_what_fits_nowhere():
    """The 8 x 16 x 16384 workload at chunk 128 plans 1.6 GB of scratch and no fused kernel
    takes it: the call is refused before anything is launched."""
    w = workload("b8_h16_t16384_d64_nu3_bf16", chunk=128)
    # pointers that are never dereferenced: the sizes are refused before any launch
    st = fwa.lib().fwa_delta_forward_noalloc(
        ctypes.c_void_p(1 << 40), ctypes.c_void_p(2 << 40), ctypes.c_void_p(3 << 40),
        ctypes.c_void_p(4 << 40), None, ctypes.c_void_p(5 << 40), None, w.B, w.H, w.T, w.d_k,
        w.d_v, w.nu, w.chunk, fwa.FWA_BF16, None)
    assert st == fwa.FWA_ERR_UNSUPPORTED
    assert "static scratch" in fwa.lib().fwa_last_error().decode()
