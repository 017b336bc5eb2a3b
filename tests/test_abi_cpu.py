"""The C ABI on the CPU: the library loads, exports every function include/fwa.h declares,
and rejects invalid arguments on the host before any HIP call (no GPU needed).

The rejection tests pass pointers that are never dereferenced; should a check ever let one of
them through, its launch must not reach a real device, so this module runs only where no GPU is
visible."""
import ctypes
import os
import re
import subprocess

import pytest

from weight_linear_attention_amd import fwa

pytestmark = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="passes never-dereferenced pointers: CPU-only (a GPU is visible here)")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fwa.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fwa_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fwa_dpfp", "fwa_delta_forward", "fwa_delta_forward_path", "fwa_delta_forward_info",
              "fwa_delta_step", "fwa_status_string", "fwa_last_error", "fwa_version"):
        assert n in names
    assert set(names) == set(fwa.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = fwa.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fwa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (fwa_\w+)", out))
    assert set(declared_functions()) <= exported


def test_version_and_status_strings():
    L = fwa.lib()
    assert L.fwa_version() == 10200
    assert L.fwa_status_string(0) == b"FWA_OK"
    assert L.fwa_status_string(1) == b"FWA_ERR_INVALID_ARG"
    assert L.fwa_status_string(2) == b"FWA_ERR_UNSUPPORTED"
    assert L.fwa_status_string(3) == b"FWA_ERR_HIP"


P = ctypes.c_void_p
FAKE = P(0x10000)        # aligned, never dereferenced: every call below fails validation first
MISALIGNED = P(0x10008)


@pytest.mark.parametrize("args,status,msg", [
    ((None, None, 10, 16, 1, 0, None), 1, "NULL"),
    ((FAKE, FAKE, -1, 16, 1, 0, None), 1, "n_vec"),
    ((FAKE, FAKE, 10, 0, 1, 0, None), 1, "d_k"),
    ((FAKE, FAKE, 10, 16, 32, 0, None), 1, "nu"),
    ((FAKE, FAKE, 10, 16, 0, 0, None), 1, "nu"),
    ((FAKE, FAKE, 10, 16, 1, 7, None), 1, "dtype"),
    ((MISALIGNED, FAKE, 10, 16, 1, 0, None), 1, "aligned"),
    ((FAKE, FAKE, 10, 24, 1, 0, None), 2, "d_k"),
    ((FAKE, FAKE, 10, 16, 1, 0, None), 1, "overlap"),
])
def test_dpfp_rejects(args, status, msg):
    L = fwa.lib()
    assert L.fwa_dpfp(*args) == status
    assert msg in L.fwa_last_error().decode()


def test_dpfp_zero_vectors_is_noop():
    assert fwa.lib().fwa_dpfp(None, None, 0, 16, 1, 0, None) == 0


def _fwd(path=None, **kw):
    a = dict(q=FAKE, k=P(0x20000), v=P(0x30000), bl=P(0x40000), W0=None, y=P(0x50000),
             Wf=None, B=1, H=1, T=8, d_k=16, d_v=16, nu=1, chunk=64, dtype=0,
             ws=P(0x1000000), ws_bytes=1 << 20)
    a.update(kw)
    args = (a["q"], a["k"], a["v"], a["bl"], a["W0"], a["y"], a["Wf"], a["B"], a["H"], a["T"],
            a["d_k"], a["d_v"], a["nu"], a["chunk"], a["dtype"], a["ws"], a["ws_bytes"], None)
    if path is None:
        return fwa.lib().fwa_delta_forward(*args)
    return fwa.lib().fwa_delta_forward_path(path, *args)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(q=None), 1, "NULL"),
    (dict(B=-1), 1, "negative"),
    (dict(T=-3), 1, "negative"),
    (dict(d_v=0), 1, "d_v"),
    (dict(nu=40), 1, "nu"),
    (dict(chunk=48), 1, "chunk"),
    (dict(dtype=3), 1, "dtype"),
    (dict(y=MISALIGNED), 1, "aligned"),
    (dict(y=FAKE), 1, "overlap"),
    (dict(Wf=P(0x20000)), 1, "overlap"),
    (dict(d_k=128), 2, "d_k"),
    (dict(d_v=48), 2, "d_v"),
    (dict(d_k=64, nu=5), 2, "512"),
    (dict(d_k=64, nu=3, chunk=128, dtype=1), 2, "on-chip"),
    (dict(ws=None), 1, "workspace of"),                         # the chunked path needs one
    (dict(ws_bytes=1000), 1, "workspace of"),                   # too small
    (dict(ws_bytes=-1), 1, "workspace_bytes"),
    (dict(ws=P(0x1000008)), 1, "aligned"),
    (dict(ws=P(0x20000)), 1, "workspace overlaps an input"),
    (dict(ws=P(0x4ff00)), 1, "workspace overlaps an output"),
])
def test_forward_rejects(kw, status, msg):
    assert _fwd(**kw) == status
    assert msg in fwa.lib().fwa_last_error().decode()


@pytest.mark.parametrize("path,kw,status,msg", [
    (7, {}, 1, "unknown forward path"),
    (-1, {}, 1, "unknown forward path"),
    (fwa.FWA_PATH_NONE, {}, 1, "unknown forward path"),
    (fwa.FWA_PATH_CHUNKED, dict(chunk=16), 2, "chunked path does not support"),
    (fwa.FWA_PATH_STREAM, {}, 2, "takes bf16"),
])
def test_forward_path_rejects(path, kw, status, msg):
    assert _fwd(path=path, **kw) == status
    assert msg in fwa.lib().fwa_last_error().decode()


def test_forward_empty_batch_is_noop():
    assert _fwd(B=0, q=None, k=None, v=None, bl=None, y=None) == 0
    assert _fwd(H=0) == 0


def _step(**kw):
    a = dict(q=FAKE, k=P(0x20000), v=P(0x30000), bl=P(0x40000), W=P(0x100000), y=P(0x50000),
             B=2, H=2, d_k=16, d_v=16, nu=1, dtype=0)
    a.update(kw)
    return fwa.lib().fwa_delta_step(a["q"], a["k"], a["v"], a["bl"], a["W"], a["y"], a["B"],
                                    a["H"], a["d_k"], a["d_v"], a["nu"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(W=None), 1, "NULL"),
    (dict(H=-1), 1, "negative"),
    (dict(nu=0), 1, "nu"),
    (dict(dtype=2), 1, "dtype"),
    (dict(W=MISALIGNED), 1, "aligned"),
    (dict(y=P(0x100000)), 1, "overlap"),
    (dict(d_k=24), 2, "d_k"),
    (dict(d_k=64, nu=5), 2, "row layout"),
])
def test_step_rejects(kw, status, msg):
    assert _step(**kw) == status
    assert msg in fwa.lib().fwa_last_error().decode()


def test_step_empty_batch_is_noop():
    assert _step(B=0, q=None, W=None) == 0


# ------------------------------------------------------------------ forward implementation choice

def _workspace_formula(B, H, T, d_k, d_v, nu, chunk, es):
    """The chunked path's workspace as fwa.h states it: the chunk-start memories and U only
    where the outputs take a launch of their own."""
    D = 2 * d_k * nu
    nc = -(-T // chunk)
    if es == 4:
        chain_outputs = D in (64, 128) and (T + chunk) * d_v * 4 < 2 ** 31
    else:
        chain_outputs = chunk == 64 and D in (128, 256) and (T + chunk) * d_v * 2 < 2 ** 31
    per_chunk = 3 * chunk * D + chunk * chunk + (0 if chain_outputs else D * d_v + chunk * d_v)
    return B * H * nc * per_chunk * es + B * H * nc * chunk * (d_v + 2) * 4


def _stream_workspace_formula(B, H, T, d_k, chunk):
    """The streaming path's workspace as fwa.h states it: at d_k = 64 only the operand blocks
    on and below the diagonal are stored."""
    nc = -(-T // chunk)
    s = 1024 * (chunk // 32) * (chunk // 32 + 1) if d_k == 64 else chunk * chunk * 2
    return B * H * nc * (3 * s + 2 * chunk * 4)


@pytest.mark.parametrize("shape,dtype,path", [
    ((1, 8, 1024, 64, 64, 1, 64), "f32", "chunked"),      # 8 heads x 1024, D 128
    ((4, 8, 4096, 64, 64, 2, 64), "bf16", "chunked"),     # 32 heads x 4096, D 256
    ((4, 8, 4096, 64, 64, 3, 64), "bf16", "stream"),      # D 384: 64 serial workgroups suffice
    ((8, 16, 4096, 64, 64, 2, 64), "bf16", "stream"),     # 256 serial workgroups
    ((2, 8, 16384, 64, 64, 2, 64), "bf16", "chunked"),    # 32 serial workgroups: too few
    ((8, 16, 16384, 64, 64, 3, 64), "bf16", "stream"),    # 128 heads x 16384: 7.6 GB chunked workspace
    ((8, 16, 16384, 64, 16, 3, 64), "bf16", "stream"),    # d_v 16: 16-column sliced serial kernel
    ((8, 16, 16384, 32, 16, 4, 64), "bf16", "fused"),     # d_k 32, d_v 16: no streaming plan
    ((8, 16, 16384, 64, 64, 3, 128), "bf16", "stream"),   # chunk 128: shift-sliced streaming
    ((8, 16, 16384, 64, 16, 3, 128), "bf16", "none"),     # d_v 16, chunk 128: nothing fits
    ((1, 1, 64, 16, 16, 1, 16), "f32", "fused"),          # chunk 16: fused only
    ((1, 1, 77, 16, 16, 1, 32), "f32", "chunked"),
    ((2, 2, 300, 64, 64, 6, 64), "f32", "fused"),         # fp32 D 768 > 512: unsupported
    ((0, 8, 1024, 64, 64, 1, 64), "f32", "empty"),
])
def test_forward_info_auto_choice(shape, dtype, path):
    import torch
    B, H, T, d_k, d_v, nu, chunk = shape
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    if path == "none" or 2 * d_k * nu > 512:
        with pytest.raises(fwa.FwaError) as e:
            fwa.delta_forward_info(B, H, T, d_k, d_v, nu, chunk, td)
        assert e.value.status == fwa.FWA_ERR_UNSUPPORTED
        return
    got, ws = fwa.delta_forward_info(B, H, T, d_k, d_v, nu, chunk, td)
    if path == "empty":
        assert (got, ws) == ("none", 0)
        return
    assert got == path
    if path == "chunked":
        assert ws == _workspace_formula(B, H, T, d_k, d_v, nu, chunk, 2 if dtype == "bf16" else 4)
    elif path == "stream":
        assert ws == _stream_workspace_formula(B, H, T, d_k, chunk)
    else:
        assert ws == 0


@pytest.mark.parametrize("shape,dtype,chain_outputs", [
    ((1, 2, 100, 32, 32, 1, 64), "f32", True),      # D 64: the staged chain forms y
    ((1, 2, 100, 64, 32, 1, 32), "f32", True),      # D 128 at chunk 32
    ((1, 2, 100, 16, 16, 1, 32), "f32", False),     # D 32: the output launch runs
    ((1, 2, 100, 64, 32, 2, 32), "f32", False),     # D 256
    ((1, 2, 100, 64, 32, 1, 64), "bf16", True),     # bf16 chunk 64, D 128: direct chain
    ((1, 2, 100, 64, 32, 1, 32), "bf16", False),    # bf16 chunk 32: staged chain + outputs
    ((1, 2, 100, 64, 32, 3, 64), "bf16", False),    # bf16 D 384
])
def test_forward_info_chunked_workspace(shape, dtype, chain_outputs):
    """The chunked workspace leaves out the chunk-start memories and U exactly where the chain
    forms the outputs itself."""
    import torch
    B, H, T, d_k, d_v, nu, chunk = shape
    es = 2 if dtype == "bf16" else 4
    path, ws = fwa.delta_forward_info(B, H, T, d_k, d_v, nu, chunk,
                                      torch.bfloat16 if dtype == "bf16" else torch.float32,
                                      path="chunked")
    D, nc = 2 * d_k * nu, -(-T // chunk)
    extra = B * H * nc * (D * d_v + chunk * d_v) * es
    assert path == "chunked"
    assert ws == _workspace_formula(B, H, T, d_k, d_v, nu, chunk, es)
    base = B * H * nc * ((3 * chunk * D + chunk * chunk) * es + chunk * (d_v + 2) * 4)
    assert ws == base + (0 if chain_outputs else extra)


def test_forward_info_path_request():
    import torch
    big = (8, 16, 16384, 64, 64, 3, 64, torch.bfloat16)
    path, ws = fwa.delta_forward_info(*big, path="chunked")
    assert path == "chunked" and ws == _workspace_formula(*big[:7], 2)
    assert fwa.delta_forward_info(1, 8, 1024, 64, 64, 1, 64, path="fused") == ("fused", 0)
    with pytest.raises(fwa.FwaError) as e:                # chunk 16 has no chunked plan
        fwa.delta_forward_info(1, 1, 64, 16, 16, 1, 16, path="chunked")
    assert e.value.status == fwa.FWA_ERR_UNSUPPORTED
    assert fwa.delta_forward_info(4, 8, 4096, 64, 64, 2, 64, torch.bfloat16, path="stream") == (
        "stream", _stream_workspace_formula(4, 8, 4096, 64, 64))
    # d_k = 32 takes the compact prep, which stores every operand block
    assert fwa.delta_forward_info(4, 8, 4096, 32, 64, 2, 64, torch.bfloat16, path="stream") == (
        "stream", _stream_workspace_formula(4, 8, 4096, 32, 64))
    for args in ((1, 8, 1024, 64, 64, 1, 64),                       # fp32
                 (1, 8, 1024, 64, 64, 1, 32, torch.bfloat16),       # chunk 32
                 (1, 8, 1024, 32, 16, 2, 64, torch.bfloat16),       # d_k 32 with d_v 16
                 (1, 8, 1024, 32, 64, 3, 64, torch.bfloat16)):      # D 192
        with pytest.raises(fwa.FwaError) as e:
            fwa.delta_forward_info(*args, path="stream")
        assert e.value.status == fwa.FWA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        fwa.delta_forward_info(1, 8, 1024, 64, 64, 1, 64, path="fast")
    L = fwa.lib()
    got, ws = ctypes.c_int(7), ctypes.c_int64(7)
    assert L.fwa_delta_forward_info(1, 8, 1024, 64, 64, 1, 64, 0, 9, ctypes.byref(got),
                                    ctypes.byref(ws)) == fwa.FWA_ERR_INVALID_ARG
    assert (got.value, ws.value) == (7, 7)
    assert L.fwa_delta_forward_info(0, 8, 1024, 64, 64, 1, 64, 0, 9, ctypes.byref(got),
                                    ctypes.byref(ws)) == fwa.FWA_ERR_INVALID_ARG


@pytest.mark.parametrize("args", [
    (1, 1, 64, 16, 16, 1, 48, 0),     # chunk
    (1, 1, 64, 16, 16, 0, 64, 0),     # nu
    (1, -1, 64, 16, 16, 1, 64, 0),    # H
    (1, 1, 64, 16, 16, 1, 64, 9),     # dtype
])
def test_forward_info_invalid(args):
    L = fwa.lib()
    path, ws = ctypes.c_int(7), ctypes.c_int64(7)
    assert L.fwa_delta_forward_info(*args, 0, ctypes.byref(path), ctypes.byref(ws)) == fwa.FWA_ERR_INVALID_ARG
    assert (path.value, ws.value) == (7, 7)      # outputs untouched on error


# ------------------------------------------------------------------ binding shape checks

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(*shape, dtype=dtype or torch.float32)


@pytest.mark.parametrize("bad", ["k", "v", "beta_logit", "W0", "out", "W_final", "q3"])
def test_binding_forward_rejects_wrong_shapes(bad):
    """Every wrong shape raises ValueError in the binding before any device work (CPU tensors:
    a correct shape would fail later, on the device check)."""
    B, H, T, dk, dv, nu = 2, 3, 5, 16, 8, 2
    a = dict(q=_t(B, H, T, dk), k=_t(B, H, T, dk), v=_t(B, H, T, dv), beta_logit=_t(B, H, T),
             W0=_t(B, H, dv, 2 * dk * nu), out=_t(B, H, T, dv), W_final=_t(B, H, dv, 2 * dk * nu))
    wrong = {"k": _t(B, H, T, dk + 1), "v": _t(B, H, T + 1, dv), "beta_logit": _t(B, H, T, 1),
             "W0": _t(B, H, dv, 2 * dk), "out": _t(B, H, T - 1, dv),
             "W_final": _t(B, H, dv + 1, 2 * dk * nu), "q3": _t(H, T, dk)}
    if bad == "q3":
        a["q"] = wrong[bad]
    else:
        a[bad] = wrong[bad]
    with pytest.raises(ValueError, match="shape|must be"):
        fwa.delta_forward(a["q"], a["k"], a["v"], a["beta_logit"], a["W0"], nu=nu,
                          out=a["out"], W_final=a["W_final"])
    # the same tensors with correct shapes get past the shape checks to the device check
    if bad != "q3":
        a[bad] = {"k": _t(B, H, T, dk), "v": _t(B, H, T, dv), "beta_logit": _t(B, H, T),
                  "W0": _t(B, H, dv, 2 * dk * nu), "out": _t(B, H, T, dv),
                  "W_final": _t(B, H, dv, 2 * dk * nu)}[bad]
        with pytest.raises(ValueError, match="must be on"):
            fwa.delta_forward(a["q"], a["k"], a["v"], a["beta_logit"], a["W0"], nu=nu,
                              out=a["out"], W_final=a["W_final"])


@pytest.mark.parametrize("bad", ["k", "v", "beta_logit", "W", "out", "q2"])
def test_binding_step_rejects_wrong_shapes(bad):
    B, H, dk, dv, nu = 4, 2, 16, 8, 1
    a = dict(q=_t(B, H, dk), k=_t(B, H, dk), v=_t(B, H, dv), beta_logit=_t(B, H),
             W=_t(B, H, dv, 2 * dk * nu), out=_t(B, H, dv))
    wrong = {"k": _t(B, H, dk // 2), "v": _t(B, H + 1, dv), "beta_logit": _t(B * H),
             "W": _t(B, H, dv, 2 * dk * nu + 4), "out": _t(B, H, dv, 1), "q2": _t(B, dk)}
    if bad == "q2":
        a["q"] = wrong[bad]
    else:
        a[bad] = wrong[bad]
    with pytest.raises(ValueError, match="shape|must be"):
        fwa.delta_step(a["q"], a["k"], a["v"], a["beta_logit"], a["W"], nu=nu, out=a["out"])


def test_binding_dpfp_rejects_wrong_out_shape():
    x = _t(10, 16)
    with pytest.raises(ValueError, match="shape"):
        fwa.dpfp(x, 2, out=_t(10, 32))
    with pytest.raises(ValueError, match="must be on"):
        fwa.dpfp(x, 2, out=_t(10, 64))


def test_binding_rejects_unknown_path():
    B, H, T, dk = 1, 1, 4, 16
    with pytest.raises(ValueError, match="path"):
        fwa.delta_forward(_t(B, H, T, dk), _t(B, H, T, dk), _t(B, H, T, dk), _t(B, H, T),
                          path="fastest")


# ------------------------------------------------------------------ backward

def _bwd(**kw):
    a = dict(q=FAKE, k=P(0x20000), v=P(0x30000), bl=P(0x40000), W0=None, dy=P(0x60000),
             dWf=None, dq=P(0x70000), dk=P(0x80000), dv=P(0x90000), dbl=P(0xa0000), dW0=None,
             B=1, H=1, T=8, d_k=16, d_v=16, nu=1, dtype=0, ws=P(0x1000000), ws_bytes=1 << 24)
    a.update(kw)
    return fwa.lib().fwa_delta_backward(
        a["q"], a["k"], a["v"], a["bl"], a["W0"], a["dy"], a["dWf"], a["dq"], a["dk"], a["dv"],
        a["dbl"], a["dW0"], a["B"], a["H"], a["T"], a["d_k"], a["d_v"], a["nu"], a["dtype"],
        a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(dy=None), 1, "NULL"),
    (dict(dq=None), 1, "NULL"),
    (dict(T=-1), 1, "negative"),
    (dict(nu=0), 1, "nu"),
    (dict(dtype=5), 1, "dtype"),
    (dict(dk=MISALIGNED), 1, "aligned"),
    (dict(ws=None), 1, "workspace of"),
    (dict(ws_bytes=64), 1, "workspace of"),
    (dict(dq=P(0x20000)), 1, "output overlaps an input"),
    (dict(dv=P(0x80000)), 1, "two outputs overlap"),
    (dict(d_k=24), 2, "d_k"),
    (dict(d_v=65), 2, "d_v"),
    (dict(d_k=64, nu=4), 2, "384"),
])
def test_backward_rejects(kw, status, msg):
    assert _bwd(**kw) == status
    assert msg in fwa.lib().fwa_last_error().decode()


def test_backward_info_and_empty_batch():
    import torch
    assert _bwd(B=0, q=None, dy=None, dq=None) == 0
    ws = fwa.delta_backward_info(4, 8, 4096, 64, 64, 2, torch.bfloat16)
    nc = 4096 // 32
    D = 256
    per_chunk = 4 * 32 * D + 3 * 32 * 32 + 32 + 3 * 32 * 64 + 2 * 64 * D
    assert ws == 4 * 8 * nc * per_chunk * 4        # B * H chunks of nc, fp32
    assert fwa.delta_backward_info(0, 8, 100, 64, 64, 1) == 0
    with pytest.raises(fwa.FwaError) as e:
        fwa.delta_backward_info(1, 1, 10, 64, 128, 1)
    assert e.value.status == fwa.FWA_ERR_UNSUPPORTED


# ------------------------------------------------------------------ sum-update forward

def _sum(**kw):
    a = dict(q=FAKE, k=P(0x20000), v=P(0x30000), W0=None, z0=None, y=P(0x50000), Wf=None,
             zf=None, B=1, H=1, T=8, d_k=16, d_v=16, nu=1, dtype=0, ws=P(0x1000000),
             ws_bytes=1 << 24)
    a.update(kw)
    return fwa.lib().fwa_sum_forward(a["q"], a["k"], a["v"], a["W0"], a["z0"], a["y"], a["Wf"],
                                     a["zf"], a["B"], a["H"], a["T"], a["d_k"], a["d_v"], a["nu"],
                                     a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(v=None), 1, "NULL"),
    (dict(H=-2), 1, "negative"),
    (dict(nu=32), 1, "nu"),
    (dict(y=MISALIGNED), 1, "aligned"),
    (dict(ws=None), 1, "workspace of"),
    (dict(y=P(0x30000)), 1, "output overlaps an input"),
    (dict(W0=P(0x60000), Wf=P(0x60010)), 1, "output overlaps an input"),
    (dict(zf=P(0x50000)), 1, "two outputs overlap"),
    (dict(d_k=8), 2, "d_k"),
    (dict(d_v=129), 2, "d_v"),
    (dict(d_k=64, nu=4), 2, "384"),
])
def test_sum_forward_rejects(kw, status, msg):
    assert _sum(**kw) == status
    assert msg in fwa.lib().fwa_last_error().decode()


def test_sum_forward_info_and_empty_batch():
    import torch
    assert _sum(B=0, q=None, y=None) == 0
    D, d_v, nc = 256, 64, 4096 // 32
    per_chunk = 2 * 32 * D + 32 * d_v + 32 + D
    # 32 heads x 4 column groups = 128 scan workgroups: two blocks per sequence, the first
    # summed in 2048 / 128 = 16 parts, so the workspace adds the W0 copy and sixteen parts'
    # K^T V sums and key sums
    blocked = 32 * d_v * D + 16 * 32 * d_v * D + 16 * 32 * D
    assert fwa.sum_forward_info(4, 8, 4096, 64, d_v, 2, torch.bfloat16) == (4 * 8 * nc * per_chunk + blocked) * 4
    # 64 heads x 4 column groups fill the GPU: one block, no extra regions
    assert fwa.sum_forward_info(8, 8, 4096, 64, d_v, 2, torch.bfloat16) == 8 * 8 * nc * per_chunk * 4


# ------------------------------------------------------------------ linear maps and multi-layer decode

@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=None), 1, "NULL"),
    (dict(d_model=100), 2, "multiples of 8"),
    (dict(T=-1), 1, "negative"),
    (dict(q=P(0x10000)), 1, "output overlaps an input"),
    (dict(bl=P(0x2000010)), 1, "two outputs overlap"),
    (dict(x=MISALIGNED), 1, "aligned"),
])
def test_layer_project_rejects(kw, status, msg):
    a = dict(x=FAKE, W=P(0x1000000), q=P(0x2000000), k=P(0x3000000), v=P(0x4000000),
             bl=P(0x5000000), B=1, T=4, d_model=64, H=2, d_k=16, d_v=16, dtype=0)
    a.update(kw)
    st = fwa.lib().fwa_layer_project(a["x"], a["W"], a["q"], a["k"], a["v"], a["bl"], a["B"],
                                     a["T"], a["d_model"], a["H"], a["d_k"], a["d_v"], a["dtype"],
                                     None)
    assert st == status
    assert msg in fwa.lib().fwa_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(out=None), 1, "NULL"),
    (dict(d_v=12), 2, "multiples of 8"),
    (dict(out=FAKE), 1, "out overlaps an input"),
    (dict(res=P(0x3000010)), 1, "partially overlaps residual"),
])
def test_layer_output_rejects(kw, status, msg):
    a = dict(y=FAKE, Wo=P(0x1000000), bo=None, res=None, out=P(0x3000000), B=1, T=4, H=2,
             d_v=16, d_model=64, dtype=0)
    a.update(kw)
    st = fwa.lib().fwa_layer_output(a["y"], a["Wo"], a["bo"], a["res"], a["out"], a["B"], a["T"],
                                    a["H"], a["d_v"], a["d_model"], a["dtype"], None)
    assert st == status
    assert msg in fwa.lib().fwa_last_error().decode()


def test_decode_layers_rejects_before_launch():
    L = fwa.lib()
    arr = lambda *p: (ctypes.c_void_p * len(p))(*p)
    Wp, Wo, W = arr(0x1000000, 0x2000000), arr(0x3000000, 0x4000000), arr(0x5000000, 0x5000000)
    args = (FAKE, 2, Wp, Wo, None, W, 4, 64, 2, 16, 16, 1, 0)
    ws = ctypes.c_int64(0)
    assert L.fwa_decode_layers_info(4, 64, 2, 16, 16, 1, 0, ctypes.byref(ws)) == 0
    assert ws.value == 2 * 4 * 2 * 16 * 4 + 2 * 4 * 2 * 16 * 4 + 32
    # the two layers share one memory
    assert L.fwa_decode_layers(*args, P(0x8000000), ws.value, None) == 1
    assert "memories of layers" in L.fwa_last_error().decode()
    assert L.fwa_decode_layers(*args, None, 0, None) == 1
    assert "workspace" in L.fwa_last_error().decode()
    assert L.fwa_decode_layers(FAKE, 0, None, None, None, None, 4, 64, 2, 16, 16, 1, 0, None, 0,
                               None) == 0
