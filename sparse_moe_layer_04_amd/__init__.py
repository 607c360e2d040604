"""Python binding of the Beam MoE C ABI (``include/beam_moe.h``).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libbeam_moe.so``.  Tensors are torch tensors on the GPU (torch supplies device memory
and the current stream).  There is no CPU fallback: importing fails loudly when the
library is not built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbeam_moe.so")

# torch first: its HIP runtime (soname libamdhip64.so.7) is then the one the library binds to,
# so streams and device pointers from torch are valid in the library.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError("libbeam_moe.so is not built; run `python -m sparse_moe_layer_04_amd.build` "
                      "(or __graft_entry__.build())")

_lib = ctypes.CDLL(LIB_PATH)

# ---- C types -----------------------------------------------------------------------

BEAM_OK, BEAM_ERR_INVALID_ARG, BEAM_ERR_UNSUPPORTED, BEAM_ERR_WORKSPACE, BEAM_ERR_HIP = range(5)
BEAM_F32, BEAM_BF16 = 0, 1
OP_ROUTE, OP_PERMUTE, OP_FORWARD, OP_FORWARD_SUBLAYER = range(4)
NUM_STAGES = 7
STAGE_NAMES = ("prenorm", "router_logits", "router_select", "permute", "gate_up", "down", "combine")

# exported C symbols (declared in include/beam_moe.h)
EXPORTS = ("beam_moe_workspace_size", "beam_moe_rmsnorm", "beam_moe_route", "beam_moe_permute", "beam_moe_forward",
           "beam_moe_forward_fp8", "beam_moe_forward_mxfp4", "beam_moe_forward_noalloc", "beam_status_string",
           "beam_moe_abi_version")


class Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("E", ctypes.c_int32), ("I", ctypes.c_int32),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float), ("dtype", ctypes.c_int32)]


class Sublayer(ctypes.Structure):
    _fields_ = [("pre_gain", ctypes.c_void_p), ("post_gain", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("residual_k", ctypes.c_float)]


_vp, _sz = ctypes.c_void_p, ctypes.c_size_t
_lib.beam_moe_workspace_size.argtypes = [ctypes.POINTER(Shape), ctypes.c_int32, ctypes.POINTER(_sz)]
_lib.beam_moe_rmsnorm.argtypes = [ctypes.POINTER(Shape), _vp, _vp, ctypes.c_float, _vp, _vp]
_lib.beam_moe_route.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.beam_moe_permute.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.beam_moe_forward.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(Sublayer), _vp,
                                  _vp, _vp, _vp, _vp, _sz, ctypes.POINTER(_vp), _vp]
_lib.beam_moe_forward_fp8.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.POINTER(Sublayer), _vp, _vp, _vp, _vp, _vp, _sz, ctypes.POINTER(_vp), _vp]
_lib.beam_moe_forward_mxfp4.argtypes = _lib.beam_moe_forward_fp8.argtypes
_lib.beam_moe_forward_noalloc.argtypes = [ctypes.POINTER(Shape), _vp, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.POINTER(Sublayer), _vp, _vp, _vp, _vp, ctypes.POINTER(_vp), _vp]
NOALLOC_SCRATCH_BYTES = 128 << 20   # BEAM_NOALLOC_SCRATCH_BYTES
for _f in ("beam_moe_workspace_size", "beam_moe_rmsnorm", "beam_moe_route", "beam_moe_permute", "beam_moe_forward",
           "beam_moe_forward_fp8", "beam_moe_forward_mxfp4", "beam_moe_forward_noalloc"):
    getattr(_lib, _f).restype = ctypes.c_int
_lib.beam_status_string.argtypes = [ctypes.c_int]
_lib.beam_status_string.restype = ctypes.c_char_p
_lib.beam_moe_abi_version.argtypes = []
_lib.beam_moe_abi_version.restype = ctypes.c_int32


class BeamError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def status_string(status: int) -> str:
    return _lib.beam_status_string(status).decode()


def abi_version() -> int:
    return _lib.beam_moe_abi_version()


def lib():
    """The loaded ctypes library (raw entry points)."""
    return _lib


def _check(status: int, where: str):
    if status != BEAM_OK:
        raise BeamError(status, where)


def make_shape(T, H, E, I, n_group, topk_group, top_k, routed_scaling=2.5, dtype="bf16") -> Shape:
    d = {"bf16": BEAM_BF16, "f32": BEAM_F32}[dtype] if isinstance(dtype, str) else int(dtype)
    return Shape(int(T), int(H), int(E), int(I), int(n_group), int(topk_group), int(top_k), float(routed_scaling), d)


def workspace_size(shape: Shape, op: int) -> int:
    n = _sz(0)
    _check(_lib.beam_moe_workspace_size(ctypes.byref(shape), op, ctypes.byref(n)), "beam_moe_workspace_size")
    return n.value


# ---- torch marshalling ------------------------------------------------------------------

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def rmsnorm(shape: Shape, x, gain, eps: float, u, stream=None):
    _check(_lib.beam_moe_rmsnorm(ctypes.byref(shape), _ptr(x), _ptr(gain), eps, _ptr(u), _stream(stream)),
           "beam_moe_rmsnorm")


def route(shape: Shape, x, w_router, bias, topk_idx, topk_w, logits_out=None, ws=None, stream=None):
    _check(_lib.beam_moe_route(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(topk_idx),
                               _ptr(topk_w), _ptr(logits_out), _ptr(ws), _nbytes(ws), _stream(stream)),
           "beam_moe_route")


def permute(shape: Shape, topk_idx, offsets, sorted_pairs, pair_pos, ws, stream=None):
    _check(_lib.beam_moe_permute(ctypes.byref(shape), _ptr(topk_idx), _ptr(offsets), _ptr(sorted_pairs),
                                 _ptr(pair_pos), _ptr(ws), _nbytes(ws), _stream(stream)), "beam_moe_permute")


def forward(shape: Shape, x, w_router, bias, w_gate, w_up, w_down, out, ws, sublayer: Optional[Sublayer] = None,
            topk_idx=None, topk_w=None, moe_y=None, stage_events: Optional[Sequence[int]] = None, stream=None,
            w_scales=None, w_format: str = "e4m3"):
    """beam_moe_forward; with ``w_scales`` = (s_gate, s_up, s_down) the expert weights are codes
    with E8M0 block scales: E4M3 bytes (``w_format`` "e4m3", beam_moe_forward_fp8) or E2M1
    codes two per byte ("e2m1", beam_moe_forward_mxfp4)."""
    ev = None
    if stage_events is not None:
        if len(stage_events) != NUM_STAGES + 1:
            raise ValueError("need %d stage events" % (NUM_STAGES + 1))
        ev = (_vp * (NUM_STAGES + 1))(*stage_events)
    sub = ctypes.byref(sublayer) if sublayer is not None else None
    if w_scales is None:
        _check(_lib.beam_moe_forward(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
                                     _ptr(w_up), _ptr(w_down), sub, _ptr(out), _ptr(topk_idx), _ptr(topk_w),
                                     _ptr(moe_y), _ptr(ws), _nbytes(ws), ev, _stream(stream)), "beam_moe_forward")
    else:
        sg, su, sd = w_scales
        name = {"e4m3": "beam_moe_forward_fp8", "e2m1": "beam_moe_forward_mxfp4"}.get(w_format)
        if name is None:
            raise ValueError("w_format must be 'e4m3' or 'e2m1'")
        _check(getattr(_lib, name)(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
                                   _ptr(w_up), _ptr(w_down), _ptr(sg), _ptr(su), _ptr(sd), sub, _ptr(out),
                                   _ptr(topk_idx), _ptr(topk_w), _ptr(moe_y), _ptr(ws), _nbytes(ws), ev,
                                   _stream(stream)), name)


def forward_noalloc(shape: Shape, x, w_router, bias, w_gate, w_up, w_down, out, sublayer: Optional[Sublayer] = None,
                    topk_idx=None, topk_w=None, moe_y=None, stage_events: Optional[Sequence[int]] = None,
                    stream=None):
    """beam_moe_forward_noalloc: beam_moe_forward with the library's static device scratch
    instead of a workspace (no allocation; calls overlapping on one GPU race)."""
    ev = None
    if stage_events is not None:
        if len(stage_events) != NUM_STAGES + 1:
            raise ValueError("need %d stage events" % (NUM_STAGES + 1))
        ev = (_vp * (NUM_STAGES + 1))(*stage_events)
    sub = ctypes.byref(sublayer) if sublayer is not None else None
    _check(_lib.beam_moe_forward_noalloc(ctypes.byref(shape), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
                                         _ptr(w_up), _ptr(w_down), sub, _ptr(out), _ptr(topk_idx), _ptr(topk_w),
                                         _ptr(moe_y), ev, _stream(stream)), "beam_moe_forward_noalloc")


def sublayer(pre_gain, post_gain, eps: float, residual_k: float) -> Sublayer:
    return Sublayer(_ptr(pre_gain), _ptr(post_gain), float(eps), float(residual_k))


# ---- HIP events for stage timing (plumbing through the HIP runtime) ----------------------

class StageTimer:
    """NUM_STAGES + 1 hipEvent_t handles to hand to ``forward(stage_events=...)``.

    ``elapsed_ms()`` returns the per-stage durations of the last recorded call (after the
    stream has been synchronised)."""

    def __init__(self):
        self._hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime already loaded by torch
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        self._hip.hipEventDestroy.argtypes = [_vp]
        self.events = []
        for _ in range(NUM_STAGES + 1):
            h = _vp()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.events.append(h.value)

    def elapsed_ms(self):
        out = []
        for i in range(NUM_STAGES):
            ms = ctypes.c_float(0.0)
            rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.events[i], self.events[i + 1])
            if rc != 0:
                raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
            out.append(ms.value)
        return out

    def close(self):
        for h in self.events:
            self._hip.hipEventDestroy(h)
        self.events = []
