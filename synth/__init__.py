"""Seeded synthetic inputs for the Beam MoE layer (test and benchmark infrastructure).

This module only draws numbers: it holds none of the layer's arithmetic.  Both the
GPU library's tests/benchmark and the CPU oracle consume the arrays it returns.
The generator (SplitMix64 in counter mode + Box-Muller) lives in ``synth.c``.

bf16 tensors are returned as ``numpy.uint16`` bit patterns; fp32 as ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` (plain gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        u64, f64, vp = ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
        for name in ("synth_normal_f32", "synth_normal_bf16", "synth_uniform_f32"):
            fn = getattr(lib, name)
            fn.argtypes = [u64, u64, u64, u64, f64, f64, vp]
            fn.restype = None
        lib.synth_words.argtypes = [u64, u64, u64, u64, vp]
        lib.synth_words.restype = None
        lib.synth_quant_e4m3.argtypes = [vp, u64, u64, vp, vp]
        lib.synth_quant_e4m3.restype = None
        lib.synth_quant_e2m1.argtypes = [vp, u64, u64, vp, vp]
        lib.synth_quant_e2m1.restype = None
        _lib = lib
    return _lib


def normal_f32(seed: int, tid: int, shape, mean: float = 0.0, std: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_normal_f32(seed, tid, first, out.size, mean, std, out.ctypes.data)
    return out


def normal_bf16(seed: int, tid: int, shape, mean: float = 0.0, std: float = 1.0, first: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)
    _load().synth_normal_bf16(seed, tid, first, out.size, mean, std, out.ctypes.data)
    return out


def uniform_f32(seed: int, tid: int, shape, lo: float, hi: float, first: int = 0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _load().synth_uniform_f32(seed, tid, first, out.size, lo, hi, out.ctypes.data)
    return out


def words(seed: int, tid: int, n: int, first: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint64)
    _load().synth_words(seed, tid, first, n, out.ctypes.data)
    return out


def permutation(seed: int, tid: int, n: int) -> np.ndarray:
    """Seeded permutation of range(n) (Fisher-Yates driven by the counter stream)."""
    w = words(seed, tid, n)
    p = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = int(w[i] % np.uint64(i + 1))
        p[i], p[j] = p[j], p[i]
    return p


def subset(seed: int, tid: int, n: int, m: int) -> np.ndarray:
    """Seeded, sorted subset of m distinct indices from range(n)."""
    if m >= n:
        return np.arange(n, dtype=np.int64)
    return np.sort(permutation(seed, tid, n)[:m])


def quantize_e4m3(w: np.ndarray):
    """bf16 weights [..., K] (uint16 bit patterns, K % 32 == 0) in 8-bit storage: OCP FP8
    E4M3 codes [..., K] and E8M0 block scales [..., K/32] (uint8), as described in synth.c."""
    if w.dtype != np.uint16 or w.shape[-1] % 32:
        raise ValueError("expected bf16 bit patterns with a last dimension divisible by 32")
    w = np.ascontiguousarray(w)
    cols = w.shape[-1]
    rows = w.size // cols
    codes = np.empty(w.shape, dtype=np.uint8)
    scales = np.empty(w.shape[:-1] + (cols // 32,), dtype=np.uint8)
    _load().synth_quant_e4m3(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def quantize_e2m1(w: np.ndarray):
    """bf16 weights [..., K] (uint16 bit patterns, K % 32 == 0) in 4-bit storage (MXFP4): OCP
    FP4 E2M1 codes two per byte [..., K/2] (the even element in the low nibble) and E8M0
    block scales [..., K/32] (uint8), as described in synth.c."""
    if w.dtype != np.uint16 or w.shape[-1] % 32:
        raise ValueError("expected bf16 bit patterns with a last dimension divisible by 32")
    w = np.ascontiguousarray(w)
    cols = w.shape[-1]
    rows = w.size // cols
    codes = np.empty(w.shape[:-1] + (cols // 2,), dtype=np.uint8)
    scales = np.empty(w.shape[:-1] + (cols // 32,), dtype=np.uint8)
    _load().synth_quant_e2m1(w.ctypes.data, rows, cols, codes.ctypes.data, scales.ctypes.data)
    return codes, scales


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of float32 to bf16 bit patterns (finite inputs)."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return (b >> np.uint64(16)).astype(np.uint16)


from .configs import CONFIGS, MoEInputs, make_inputs, expert_weights  # noqa: E402,F401
