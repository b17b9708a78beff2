"""Seeded synthetic inputs shared by the CPU oracle's tests and the GPU path.

This module only draws random numbers and stores them in the dtypes the
cache uses; it holds none of the attention method's arithmetic. The
generator (counter-based SplitMix64 -> Box-Muller -> round-to-nearest-even)
lives in ``synth.c``; ``workloads.py`` assembles the five workloads from it.
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
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i64, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        for name in ("synth_uniform_f64", "synth_normal_f64", "synth_normal_f32",
                     "synth_normal_bf16"):
            fn = getattr(L, name)
            fn.argtypes = [u64, u64, u64, i64, vp]
            fn.restype = None
        for name in ("synth_round_bf16", "synth_round_f32"):
            fn = getattr(L, name)
            fn.argtypes = [vp, i64, vp]
            fn.restype = None
        L.synth_normal_one.argtypes = [u64, u64, u64]
        L.synth_normal_one.restype = ctypes.c_double
        L.synth_mix64.argtypes = [u64]
        L.synth_mix64.restype = u64
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def uniform(seed: int, stream: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform_f64(seed, stream, start, n, _ptr(out))
    return out


def normal(seed: int, stream: int, start: int, n: int, dtype: str = "f64") -> np.ndarray:
    """Normal values with indices start .. start+n-1 of (seed, stream).

    dtype 'f64' -> float64, 'f32' -> float32 (RNE), 'bf16' -> uint16 bit
    patterns of bfloat16 (RNE from the double)."""
    if dtype == "f64":
        out = np.empty(n, np.float64)
        lib().synth_normal_f64(seed, stream, start, n, _ptr(out))
    elif dtype == "f32":
        out = np.empty(n, np.float32)
        lib().synth_normal_f32(seed, stream, start, n, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(n, np.uint16)
        lib().synth_normal_bf16(seed, stream, start, n, _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype ('f32' or 'bf16' bits)."""
    x = np.ascontiguousarray(x, np.float64)
    if dtype == "f32":
        out = np.empty(x.shape, np.float32)
        lib().synth_round_f32(_ptr(x), x.size, _ptr(out))
    elif dtype == "bf16":
        out = np.empty(x.shape, np.uint16)
        lib().synth_round_bf16(_ptr(x), x.size, _ptr(out))
    else:
        raise ValueError(dtype)
    return out


def widen(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored f32 / bf16-bit data."""
    if dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, np.uint16).astype(np.uint32) << 16
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)
