"""Seeded synthetic inputs for the certified quantized-KV decode step.

Shared by the oracle tests, the GPU tests and the benchmark.  This module
only produces inputs (FP16 keys, values and queries); it holds none of the
method's arithmetic.  The heavy loops live in ``dg.c`` (Philox4x32-10
counter-based generator + Box-Muller), built into ``libdg.so`` by
:func:`build`.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libdg.so")
_lib = None


def build():
    """Compile dg.c into libdg.so (gcc, OpenMP)."""
    src = os.path.join(_HERE, "dg.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
    os.replace(tmp, _SO)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, u32, i64, i32, dbl = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                   ctypes.c_int, ctypes.c_double)
        vp = ctypes.c_void_p
        L.dg_normal.argtypes = [u64, u32, i64, i64, vp]
        L.dg_uniform.argtypes = [u64, u32, i64, i64, vp]
        L.dg_to_f16.argtypes = [vp, i64, vp]
        L.dg_keys.argtypes = [u64, i32, i32, i32, i32, vp, i32, vp, dbl, vp, vp, dbl, vp, vp]
        L.dg_values.argtypes = [u64, i32, i32, i32, i32, i32, dbl, vp]
        L.dg_philox_raw.argtypes = [vp, vp, vp]
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def normal(seed, tag, n, start=0):
    out = np.empty(n, np.float64)
    lib().dg_normal(seed, tag, start, n, _ptr(out))
    return out


def uniform(seed, tag, n, start=0):
    out = np.empty(n, np.float64)
    lib().dg_uniform(seed, tag, start, n, _ptr(out))
    return out


def to_f16(x):
    """Round float64 values to FP16 (nearest even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().dg_to_f16(_ptr(x), x.size, _ptr(out))
    return out


def philox(ctr, key):
    c = np.ascontiguousarray(ctr, np.uint32)
    k = np.ascontiguousarray(key, np.uint32)
    out = np.empty(4, np.uint32)
    lib().dg_philox_raw(_ptr(c), _ptr(k), _ptr(out))
    return out


def keys(seed, B, T, Hkv, d, chan_scale, amp, direction, rank=0, W=None, noise_std=1.0,
         tie_eps=0.0, tie_mode=None):
    out = np.empty((B, T, Hkv, d), np.uint16)
    tm = np.ascontiguousarray(tie_mode if tie_mode is not None else np.ones(Hkv), np.int32)
    cs = np.ascontiguousarray(chan_scale, np.float32)
    am = np.ascontiguousarray(amp, np.float32)
    dr = np.ascontiguousarray(direction, np.float32)
    Wa = np.ascontiguousarray(W if W is not None else np.zeros(1), np.float32)
    lib().dg_keys(seed, B, T, Hkv, d, _ptr(cs), rank, _ptr(Wa), noise_std, _ptr(am), _ptr(dr),
                  tie_eps, _ptr(tm), _ptr(out))
    return out


def values(seed, B, T, Hkv, d, nu=0, scale=1.0):
    out = np.empty((B, T, Hkv, d), np.uint16)
    lib().dg_values(seed, B, T, Hkv, d, nu, scale, _ptr(out))
    return out


from .workloads import CONFIGS, Layer, make_layer, seed_for  # noqa: E402,F401
