"""CPU oracle of one Beam mixture-of-experts layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library and never calls it.

The arithmetic lives in ``beam_oracle.c`` (plain loops, fp64; the routing choice is taken
on fp32 values as the Beam model doc's FP32-numerics paragraph fixes).  This wrapper only
marshals numpy arrays.  Each function cites the passage it follows in the C file.

Pins: every function here is checked against closed forms, invariants, brute force and
hand-worked cases in ``tests/test_oracle_pins.py`` (see that file's docstring).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "beam_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# a planted-mistake copy of the oracle can be loaded instead (tests/test_oracle_mutations.py)
_LIB_OVERRIDE = os.environ.get("BEAM_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (portable x86-64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-o", tmp, _SRC,
                               "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=False)
            lib = ctypes.CDLL(_LIB)
        vp, i64, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        lib.oracle_rmsnorm_pinned.argtypes = [vp, vp, f32, i64, i64, vp]
        lib.oracle_rmsnorm_pinned.restype = None
        lib.oracle_route.argtypes = [vp, i32, i64, i64, vp, vp, i32, i32, i32, i32, f64, vp, vp, vp, vp, vp]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_experts.argtypes = [vp, i32, i64, i64, vp, vp, vp, i32, vp, vp, vp, i32, vp, vp, vp, i64, vp]
        lib.oracle_experts.restype = None
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = f64
        lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e2m1_value.restype = f64
        lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e8m0_value.restype = f64
        lib.oracle_post_residual.argtypes = [vp, vp, i32, vp, f32, i64, i64, f64, vp]
        lib.oracle_post_residual.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Threads for the oracle's later OpenMP loops (the arithmetic does not depend on it)."""
    _load().oracle_set_threads(int(n))


def _is_bf16(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError("expected bf16 bit patterns (uint16) or float32, got %s" % a.dtype)


def _c(a: np.ndarray) -> np.ndarray:
    if not a.flags.c_contiguous:
        raise ValueError("array must be C-contiguous")
    return a


def rmsnorm_pinned(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """Pre-RMSNorm with pinned fp32 rounding: x [T,H] bf16 -> u [T,H] bf16 (uint16)."""
    x = _c(x)
    if x.dtype != np.uint16:
        raise TypeError("pinned RMSNorm takes bf16 input")
    T, H = x.shape
    g = np.ascontiguousarray(gain, dtype=np.float32)
    u = np.empty_like(x)
    _load().oracle_rmsnorm_pinned(x.ctypes.data, g.ctypes.data, eps, T, H, u.ctypes.data)
    return u


class Routing:
    """idx [T,K] int32 (decision order), w [T,K] fp64, logits [T,E] fp64 or None,
    margin [T,2] fp64 (group, expert) or None, agree [T] int32 or None."""

    def __init__(self, idx, w, logits, margin, agree):
        self.idx, self.w, self.logits, self.margin, self.agree = idx, w, logits, margin, agree

    def min_margin(self) -> float:
        return float(np.min(self.margin)) if self.margin is not None and self.margin.size else float("inf")


def route(act: np.ndarray, w_router: np.ndarray, bias: np.ndarray, n_group: int, topk_group: int, top_k: int,
          rho: float = 2.5, want_logits: bool = False, want_margin: bool = True) -> Routing:
    """Sigmoid group-limited top-k routing (see ``beam_oracle.c`` header, steps 1-5)."""
    act = _c(act)
    T, H = act.shape
    E = w_router.shape[0]
    wr = np.ascontiguousarray(w_router, dtype=np.float32)
    b = np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    logits = np.empty((T, E), dtype=np.float64) if want_logits else None
    margin = np.empty((T, 2), dtype=np.float64) if want_margin else None
    agree = np.empty((T,), dtype=np.int32) if want_margin else None
    rc = _load().oracle_route(act.ctypes.data, _is_bf16(act), T, H, wr.ctypes.data, b.ctypes.data, E, n_group,
                              topk_group, top_k, rho, idx.ctypes.data, w.ctypes.data,
                              logits.ctypes.data if logits is not None else None,
                              margin.ctypes.data if margin is not None else None,
                              agree.ctypes.data if agree is not None else None)
    if rc != 0:
        raise ValueError("invalid routing shape")
    return Routing(idx, w, logits, margin, agree)


def e4m3_value(code: int) -> float:
    """The value of one OCP FP8 E4M3 code (the oracle's decoding)."""
    return float(_load().oracle_e4m3_value(int(code)))


def e8m0_value(s: int) -> float:
    """The factor of one E8M0 scale byte, 0..255 (the oracle's decoding)."""
    return float(_load().oracle_e8m0_value(int(s)))


def e2m1_value(code: int) -> float:
    """The value of one OCP FP4 E2M1 code, 0..15 (the oracle's decoding)."""
    return float(_load().oracle_e2m1_value(int(code)))


def experts(act: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray, w_down: np.ndarray, idx: np.ndarray,
            w: np.ndarray, tokens: Optional[np.ndarray] = None, w_scales=None) -> np.ndarray:
    """y[n] = sum_j w[t,j] * SwiGLU-expert_{idx[t,j]}(act[t]) for t = tokens[n]; fp64 [n,H].

    Weights are fp32, bf16 (uint16 bit patterns) or, with ``w_scales`` = (s_gate, s_up,
    s_down), one E8M0 scale byte per 32 elements of a row and either OCP FP8 E4M3 codes
    (uint8, the bf16 shapes) or OCP FP4 E2M1 codes two per byte (uint8, the last dimension
    halved; the even element in the low nibble)."""
    act = _c(act)
    T, H = act.shape
    E, I, H2 = w_gate.shape
    packed = w_scales is not None and 2 * H2 == H
    if packed:
        assert w_up.shape == (E, I, H // 2) and w_down.shape[:2] == (E, H)
        I2 = w_down.shape[2]
        assert 2 * I2 == I
    else:
        assert H2 == H and w_up.shape == (E, I, H) and w_down.shape == (E, H, I)
    if w_scales is not None:
        assert w_gate.dtype == w_up.dtype == w_down.dtype == np.uint8
        sg, su, sd = (np.ascontiguousarray(a, dtype=np.uint8) for a in w_scales)
        assert sg.shape == (E, I, H // 32) and su.shape == (E, I, H // 32) and sd.shape == (E, H, I // 32)
        fmt, sp = (3 if packed else 2), (sg.ctypes.data, su.ctypes.data, sd.ctypes.data)
    else:
        fmt = _is_bf16(w_gate)
        assert _is_bf16(w_up) == fmt and _is_bf16(w_down) == fmt
        sp = (None, None, None)
    K = idx.shape[1]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    y = np.empty((tok.size, H), dtype=np.float64)
    _load().oracle_experts(act.ctypes.data, _is_bf16(act), H, I, _c(w_gate).ctypes.data, _c(w_up).ctypes.data,
                           _c(w_down).ctypes.data, fmt, sp[0], sp[1], sp[2], K, idx.ctypes.data, w.ctypes.data,
                           tok.ctypes.data, tok.size, y.ctypes.data)
    return y


def post_residual(y: np.ndarray, x: np.ndarray, gain: np.ndarray, eps: float, k: float) -> np.ndarray:
    """out = sqrt((k-1)/k) x + RMSNorm(y; gain, eps) / sqrt(k), fp64 [n,H]."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    x = _c(x)
    n, H = y.shape
    assert x.shape == (n, H)
    g = np.ascontiguousarray(gain, dtype=np.float32)
    out = np.empty((n, H), dtype=np.float64)
    _load().oracle_post_residual(y.ctypes.data, x.ctypes.data, _is_bf16(x), g.ctypes.data, eps, n, H, float(k),
                                 out.ctypes.data)
    return out


def permutation(idx: np.ndarray, E: int):
    """Stable counting sort of the (token, choice) pairs by expert, in plain loops.

    Pair p = t*K + j goes to expert idx[t, j].  Returns (offsets [E+1], sorted_pairs [P],
    pair_pos [P]): offsets[e] = number of pairs with expert < e; sorted_pairs lists the
    pairs expert by expert, ascending p within an expert; pair_pos[p] = position of p.
    Expert e's rows of the grouped products are sorted_pairs[offsets[e]:offsets[e+1]].
    """
    flat = [int(v) for v in np.asarray(idx).reshape(-1)]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    cursor = offsets[:-1]
    sorted_pairs = [0] * len(flat)
    pair_pos = [0] * len(flat)
    for p, e in enumerate(flat):
        sorted_pairs[cursor[e]] = p
        pair_pos[p] = cursor[e]
        cursor[e] += 1
    return (np.array(offsets, dtype=np.int32), np.array(sorted_pairs, dtype=np.int32),
            np.array(pair_pos, dtype=np.int32))


class LayerResult:
    """Oracle results of one layer call: u (layer input after the optional pre-norm),
    routing (all tokens), tokens (the token rows evaluated), y (MoE output, fp64 [n,H]),
    out (final output, fp64 [n,H]; equals y without the sublayer)."""

    def __init__(self, u, routing, tokens, y, out):
        self.u, self.routing, self.tokens, self.y, self.out = u, routing, tokens, y, out


def layer(inp, tokens: Optional[np.ndarray] = None, want_logits: bool = False) -> LayerResult:
    """The whole layer for ``synth.MoEInputs``; routing on all tokens, experts on ``tokens``."""
    cfg = inp.cfg
    u = rmsnorm_pinned(inp.x, inp.pre_gain, cfg.eps) if cfg.sublayer else inp.x
    r = route(u, inp.w_router, inp.bias, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.rho, want_logits=want_logits)
    tok = np.arange(cfg.T, dtype=np.int64) if tokens is None else np.asarray(tokens, dtype=np.int64)
    y = experts(u, inp.w_gate, inp.w_up, inp.w_down, r.idx, r.w, tok, w_scales=inp.w_scales)
    out = post_residual(y, np.ascontiguousarray(inp.x[tok]), inp.post_gain, cfg.eps, cfg.residual_k) \
        if cfg.sublayer else y
    return LayerResult(u, r, tok, y, out)
