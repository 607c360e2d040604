"""Host-side checks of the C ABI (no GPU): the library loads, exports every entry point
declared in include/beam_moe.h, and rejects bad arguments before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_moe_layer_04_amd as bm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "beam_moe.h")

FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced by these calls


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(beam_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared_functions()
    assert set(names) == set(bm.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", bm.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(bm.lib(), n) is not None


def test_abi_version_and_status_strings():
    assert bm.abi_version() == 1
    assert bm.status_string(bm.BEAM_OK) == "ok"
    assert "workspace" in bm.status_string(bm.BEAM_ERR_WORKSPACE)
    assert bm.status_string(99) == "unknown status"


def _beam(T=64, **kw):
    d = dict(T=T, H=5120, E=256, I=2560, n_group=8, topk_group=4, top_k=8, routed_scaling=2.5, dtype="bf16")
    d.update(kw)
    return bm.make_shape(**d)


@pytest.mark.parametrize("bad", [
    dict(E=255), dict(n_group=0), dict(n_group=65, E=130), dict(topk_group=9), dict(topk_group=0), dict(top_k=33),
    dict(top_k=0), dict(E=16, n_group=8, topk_group=1, top_k=3), dict(E=2048, n_group=8), dict(T=-1), dict(H=0),
    dict(I=0), dict(dtype=7), dict(T=1 << 28), dict(routed_scaling=float("inf")),
])
def test_workspace_size_rejects_invalid_shapes(bad):
    with pytest.raises(bm.BeamError) as ei:
        bm.workspace_size(_beam(**bad), bm.OP_FORWARD)
    assert ei.value.status == bm.BEAM_ERR_INVALID_ARG


def test_unsupported_shapes():
    for bad in (dict(H=5000), dict(I=2500), dict(H=384), dict(I=192)):
        with pytest.raises(bm.BeamError) as ei:
            bm.workspace_size(_beam(**bad), bm.OP_FORWARD)
        assert ei.value.status == bm.BEAM_ERR_UNSUPPORTED
    with pytest.raises(bm.BeamError) as ei:
        bm.workspace_size(_beam(dtype="f32"), bm.OP_FORWARD_SUBLAYER)
    assert ei.value.status == bm.BEAM_ERR_UNSUPPORTED
    # the fp32 path takes any H, I; routing alone only needs H % 128 in bf16
    assert bm.workspace_size(_beam(H=100, I=30, dtype="f32"), bm.OP_FORWARD) > 0
    assert bm.workspace_size(_beam(H=384, I=30), bm.OP_ROUTE) > 0
    with pytest.raises(bm.BeamError):
        bm.workspace_size(_beam(H=96), bm.OP_ROUTE)
    assert bm.workspace_size(_beam(H=80, I=30), bm.OP_PERMUTE) > 0


def test_workspace_sizes():
    s = _beam(T=8192)
    fw = bm.workspace_size(s, bm.OP_FORWARD)
    P = 8192 * 8
    assert fw >= P * (2560 + 5120) * 2 + 8192 * 256 * 4
    assert fw < P * (2560 + 5120) * 2 * 1.05 + 64 * 2 ** 20
    assert bm.workspace_size(s, bm.OP_FORWARD_SUBLAYER) >= fw + 8192 * 5120 * 2
    assert bm.workspace_size(s, bm.OP_ROUTE) >= 8192 * 256 * 4
    assert bm.workspace_size(s, bm.OP_PERMUTE) >= 256 * 4
    assert bm.workspace_size(_beam(T=0), bm.OP_FORWARD) >= 0
    with pytest.raises(bm.BeamError):
        bm.workspace_size(s, 9)


def _raw_forward(shape, ws_bytes, out=FAKE, sub=None, events=None):
    f = bm.lib().beam_moe_forward
    return f(ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(sub) if sub else None, out, None,
             None, None, FAKE if ws_bytes else None, ws_bytes, events, None)


def test_forward_validation_happens_before_launch():
    s = _beam(T=64)
    need = bm.workspace_size(s, bm.OP_FORWARD)
    assert _raw_forward(s, need - 1) == bm.BEAM_ERR_WORKSPACE
    assert _raw_forward(s, 0) == bm.BEAM_ERR_WORKSPACE
    assert _raw_forward(s, need, out=None) == bm.BEAM_ERR_INVALID_ARG
    assert _raw_forward(s, need, out=FAKE + 2) == bm.BEAM_ERR_INVALID_ARG  # misaligned
    bad_sub = bm.Sublayer(FAKE, FAKE, 0.0, 40.0)  # eps must be > 0
    assert _raw_forward(s, need, sub=bad_sub) == bm.BEAM_ERR_INVALID_ARG
    bad_sub = bm.Sublayer(FAKE, None, 1e-6, 40.0)
    assert _raw_forward(s, need, sub=bad_sub) == bm.BEAM_ERR_INVALID_ARG
    bad_sub = bm.Sublayer(FAKE, FAKE, 1e-6, 0.5)  # k >= 1
    assert _raw_forward(s, need, sub=bad_sub) == bm.BEAM_ERR_INVALID_ARG
    events = (ctypes.c_void_p * (bm.NUM_STAGES + 1))(*([FAKE] * bm.NUM_STAGES + [None]))
    assert _raw_forward(s, need, events=events) == bm.BEAM_ERR_INVALID_ARG
    # sublayer workspace is larger than the plain one
    good_sub = bm.Sublayer(FAKE, FAKE, 1e-6, 40.0)
    assert _raw_forward(s, need, sub=good_sub) == bm.BEAM_ERR_WORKSPACE
    # T = 0 is a valid no-op: nothing is launched, so fake pointers are fine
    s0 = _beam(T=0)
    assert _raw_forward(s0, bm.workspace_size(s0, bm.OP_FORWARD)) == bm.BEAM_OK


def _raw_forward_fp8(shape, ws_bytes, scales=(FAKE, FAKE, FAKE), w=FAKE, entry="beam_moe_forward_fp8"):
    f = getattr(bm.lib(), entry)
    return f(ctypes.byref(shape), FAKE, FAKE, FAKE, w, FAKE, FAKE, scales[0], scales[1], scales[2], None, FAKE, None,
             None, None, FAKE if ws_bytes else None, ws_bytes, None, None)


@pytest.mark.parametrize("entry", ["beam_moe_forward_fp8", "beam_moe_forward_mxfp4"])
def test_forward_quantized_validation_happens_before_launch(entry):
    s = _beam(T=64)
    need = bm.workspace_size(s, bm.OP_FORWARD)   # the same workspace as the bf16 forward
    assert _raw_forward_fp8(s, need - 1, entry=entry) == bm.BEAM_ERR_WORKSPACE
    for i in range(3):   # every scale tensor is required
        sc = [FAKE, FAKE, FAKE]
        sc[i] = None
        assert _raw_forward_fp8(s, need, scales=tuple(sc), entry=entry) == bm.BEAM_ERR_INVALID_ARG
    assert _raw_forward_fp8(s, need, scales=(FAKE, FAKE + 4, FAKE), entry=entry) == bm.BEAM_ERR_INVALID_ARG
    assert _raw_forward_fp8(s, need, w=None, entry=entry) == bm.BEAM_ERR_INVALID_ARG
    assert _raw_forward_fp8(s, need, w=FAKE + 8, entry=entry) == bm.BEAM_ERR_INVALID_ARG   # 16-byte loads
    sf = _beam(T=64, H=256, I=128, dtype="f32")
    assert _raw_forward_fp8(sf, bm.workspace_size(sf, bm.OP_FORWARD), entry=entry) == bm.BEAM_ERR_UNSUPPORTED
    s0 = _beam(T=0)
    assert _raw_forward_fp8(s0, 0, entry=entry) == bm.BEAM_OK


def test_route_permute_rmsnorm_validation():
    L = bm.lib()
    s = _beam(T=64)
    # route: missing outputs; missing or short workspace (with or without logits_out)
    assert L.beam_moe_route(ctypes.byref(s), FAKE, FAKE, FAKE, None, FAKE, None, None, 0, None) == \
        bm.BEAM_ERR_INVALID_ARG
    assert L.beam_moe_route(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == \
        bm.BEAM_ERR_WORKSPACE
    need = bm.workspace_size(s, bm.OP_ROUTE)
    assert L.beam_moe_route(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        bm.BEAM_ERR_WORKSPACE
    s0 = _beam(T=0)
    assert L.beam_moe_route(ctypes.byref(s0), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == bm.BEAM_OK
    # permute: workspace required
    assert L.beam_moe_permute(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, None, 0, None) == bm.BEAM_ERR_WORKSPACE
    assert L.beam_moe_permute(ctypes.byref(s), FAKE, None, FAKE, FAKE, FAKE, 1 << 20, None) == \
        bm.BEAM_ERR_INVALID_ARG
    # rmsnorm: bf16 only, no aliasing, eps >= 0
    assert L.beam_moe_rmsnorm(ctypes.byref(_beam(dtype="f32")), FAKE, FAKE, ctypes.c_float(1e-6), FAKE + 64,
                              None) == bm.BEAM_ERR_UNSUPPORTED
    assert L.beam_moe_rmsnorm(ctypes.byref(s), FAKE, FAKE, ctypes.c_float(1e-6), FAKE, None) == \
        bm.BEAM_ERR_INVALID_ARG
    assert L.beam_moe_rmsnorm(ctypes.byref(s), FAKE, FAKE, ctypes.c_float(-1.0), FAKE + 64, None) == \
        bm.BEAM_ERR_INVALID_ARG
    assert L.beam_moe_rmsnorm(ctypes.byref(s), FAKE, FAKE, ctypes.c_float(1e-6), FAKE + 72, None) == \
        bm.BEAM_ERR_INVALID_ARG  # misaligned output
    assert L.beam_moe_rmsnorm(ctypes.byref(_beam(H=100)), FAKE, FAKE, ctypes.c_float(1e-6), FAKE + 64, None) == \
        bm.BEAM_ERR_UNSUPPORTED  # rows are read in 16-byte chunks
    assert L.beam_moe_rmsnorm(ctypes.byref(s0), FAKE, FAKE, ctypes.c_float(1e-6), FAKE + 64, None) == bm.BEAM_OK


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(4)
    with pytest.raises(ValueError):
        bm._ptr(x)
