"""CPU oracle for certified quantized-KV decode attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
The arithmetic lives in ``ckv_oracle.c`` (plain C, FP64 values, canonical
FP32 / fixed-point decisions); this module only builds it and marshals
arrays in and out.
"""
import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libckv_oracle.so")
_lib = None

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared"]


def build():
    """Compile ckv_oracle.c with gcc (no fast-math, no contraction)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, os.path.join(_HERE, "ckv_oracle.c"), "-lm"])
    os.replace(tmp, _SO)


class Thresholds(ctypes.Structure):
    _fields_ = [("tau_cov", ctypes.c_float), ("k_tol", ctypes.c_float),
                ("v_tol", ctypes.c_float), ("rank_tol", ctypes.c_float),
                ("sm_scale", ctypes.c_float), ("f_layer", ctypes.c_float),
                ("n_widen", ctypes.c_int), ("v_cap_blocks", ctypes.c_int)]


REPORT_DTYPE = np.dtype([("e_key", "<f4"), ("e_val", "<f4"), ("tv_bound", "<f4"),
                         ("tau_final", "<f4"), ("kstar", "<i4"), ("n_v_promoted", "<i4"),
                         ("rank_ok", "<i4"), ("rung_max", "<i4"), ("rung_mask", "<i4"),
                         ("n_discordant", "<i4")])

_TRACE_FIELDS = ["k_code", "k_s", "k_z", "v_code", "v_s", "v_z", "eta", "vrange", "score",
                 "bmax", "bl", "delta", "rho", "mref", "mfx", "sel", "bounds", "seq_flags",
                 "score16", "m16fx", "err_key", "err_val", "o_cert", "o_dense", "cval"]


class _Trace(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in _TRACE_FIELDS]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        vp, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_double
        L.orc_h2f.argtypes, L.orc_h2f.restype = [ctypes.c_uint16], f32
        L.orc_f2h_up.argtypes, L.orc_f2h_up.restype = [f32], ctypes.c_uint16
        L.orc_ru32.argtypes, L.orc_ru32.restype = [f64], f32
        L.orc_exp_c.argtypes, L.orc_exp_c.restype = [f32], f32
        for fn in ("orc_expu", "orc_em1u", "orc_tanhu"):
            getattr(L, fn).argtypes, getattr(L, fn).restype = [f64], f64
        L.orc_fx.argtypes, L.orc_fx.restype = [f64], ctypes.c_uint64
        L.orc_quant_k_block.argtypes = [i32, vp, vp, vp, vp]
        L.orc_quant_v_block.argtypes = [i32, vp, vp, vp, vp, vp]
        L.orc_quant_v_block_bits.argtypes = [i32, i32, vp, vp, vp, vp, vp]
        L.orc_score_q8.argtypes = [i32, vp, vp, vp, vp, f32, vp]
        L.orc_score_f16.argtypes = [i32, vp, vp, i32, f32, vp]
        L.orc_delta_rho.argtypes = [i32, vp, vp, vp, f32, vp, vp]
        L.orc_block_est.argtypes = [vp, i32, vp, vp]
        L.orc_select.argtypes, L.orc_select.restype = [i32, vp, ctypes.c_uint64, vp], i32
        L.orc_discordant.argtypes, L.orc_discordant.restype = [i32, vp, vp], ctypes.c_int64
        L.orc_certified_decode.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp,
                                           ctypes.POINTER(Thresholds), vp, vp,
                                           ctypes.POINTER(_Trace)]
        L.orc_certified_decode.restype = i32
        L.orc_certified_decode_vb.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                           ctypes.POINTER(Thresholds), vp, vp,
                                           ctypes.POINTER(_Trace)]
        L.orc_certified_decode_vb.restype = i32
        L.orc_dense_head.argtypes = [i32, i32, i32, i32, vp, vp, vp, f64, vp]
        L.orc_set_threads.argtypes, L.orc_set_threads.restype = [i32], None
        L.orc_get_threads.argtypes, L.orc_get_threads.restype = [], i32
        _lib = L
    return _lib


def set_mutation(flags):
    ctypes.c_int.in_dll(lib(), "orc_mutation").value = int(flags)


def set_threads(n):
    """OpenMP threads of the decode step (results do not depend on it)."""
    lib().orc_set_threads(int(n))


def get_threads():
    return lib().orc_get_threads()


def _p(a):
    return ctypes.c_void_p(a.ctypes.data)


def default_thresholds(sm_scale, **kw):
    t = dict(tau_cov=0.995, k_tol=1e-2, v_tol=1e-2, rank_tol=0.05, sm_scale=sm_scale,
             f_layer=0.5, n_widen=3, v_cap_blocks=0)
    t.update(kw)
    return t


@dataclass
class Result:
    out: np.ndarray
    report: np.ndarray
    trace: dict


def certified_decode(k, v, q, thresholds, trace=True, v_bits=4):
    """Run the oracle's decode step.

    k, v: uint16 FP16 bit patterns [B][T][Hkv][d]; q: uint16 [B][Hq][d].
    thresholds: dict of Thresholds fields.  Returns outputs [B][Hq][d] (FP64),
    the per-head report and (if ``trace``) every intermediate named in
    ckv_oracle.h.  v_bits: 4 (INT4 values, the design) or 8 (the symmetric
    cache configuration, values at the keys' width).
    """
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    q = np.ascontiguousarray(q, np.uint16)
    B, T, Hkv, d = k.shape
    Hq = q.shape[1]
    assert v.shape == k.shape and q.shape == (B, Hq, d)
    N = T // 64
    Np = N + (T % 64 != 0)
    ng = d // 32
    out = np.zeros((B, Hq, d), np.float64)
    rep = np.zeros((B, Hq), REPORT_DTYPE)
    tr = {}
    ctr = _Trace()
    if trace:
        shapes = dict(
            k_code=((B, Hkv, N, 64, d), np.uint8), k_s=((B, Hkv, N, d), np.uint16),
            k_z=((B, Hkv, N, d), np.uint16), v_code=((B, Hkv, N, 64, d * v_bits // 8), np.uint8),
            v_s=((B, Hkv, N, 64, ng), np.uint16), v_z=((B, Hkv, N, 64, ng), np.uint16),
            eta=((B, Hkv, N), np.float32), vrange=((B, Hkv), np.float32),
            score=((B, Hq, Np * 64), np.float32), bmax=((B, Hq, Np), np.float32),
            bl=((B, Hq, Np), np.float32), delta=((B, Hq, Np), np.float32),
            rho=((B, Hq, Np), np.float32), mref=((B, Hq), np.float32),
            mfx=((B, Hq, Np), np.uint64), sel=((B, Hq, N), np.uint8),
            bounds=((B, Hq, 4), np.float64), seq_flags=((B,), np.int32),
            score16=((B, Hq, N * 64), np.float32), m16fx=((B, Hq, N), np.uint64),
            err_key=((B, Hq), np.float64), err_val=((B, Hq), np.float64),
            o_cert=((B, Hq, d), np.float64), o_dense=((B, Hq, d), np.float64),
            cval=((B, Hq, N), np.uint64))
        for f, (shp, dt) in shapes.items():
            tr[f] = np.zeros(shp, dt)
            setattr(ctr, f, tr[f].ctypes.data if tr[f].size else None)
    th = Thresholds(**thresholds)
    rc = lib().orc_certified_decode_vb(B, T, Hq, Hkv, d, v_bits, _p(k), _p(v), _p(q), ctypes.byref(th),
                                    _p(out), _p(rep), ctypes.byref(ctr))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return Result(out, rep, tr)


# -- elementary pieces, for the oracle's own pins ---------------------------

def exp_c(x):
    return lib().orc_exp_c(float(x))


def quant_k_block(kblk):
    kblk = np.ascontiguousarray(kblk, np.uint16)
    d = kblk.shape[1]
    code = np.zeros((64, d), np.uint8)
    s = np.zeros(d, np.uint16)
    z = np.zeros(d, np.uint16)
    lib().orc_quant_k_block(d, _p(kblk), _p(code), _p(s), _p(z))
    return code, s, z


def quant_v_block(vblk, bits=4):
    vblk = np.ascontiguousarray(vblk, np.uint16)
    d = vblk.shape[1]
    code = np.zeros((64, d * bits // 8), np.uint8)
    s = np.zeros((64, d // 32), np.uint16)
    z = np.zeros((64, d // 32), np.uint16)
    eta = np.zeros(1, np.float32)
    lib().orc_quant_v_block_bits(d, bits, _p(vblk), _p(code), _p(s), _p(z), _p(eta))
    return code, s, z, float(eta[0])


def score_q8(q, code, s, z, sm):
    q = np.ascontiguousarray(q, np.uint16)
    out = np.zeros(64, np.float32)
    lib().orc_score_q8(q.size, _p(q), _p(np.ascontiguousarray(code, np.uint8)),
                       _p(np.ascontiguousarray(s, np.uint16)), _p(np.ascontiguousarray(z, np.uint16)),
                       sm, _p(out))
    return out


def score_f16(q, k, sm):
    q = np.ascontiguousarray(q, np.uint16)
    k = np.ascontiguousarray(k, np.uint16)
    out = np.zeros(k.shape[0], np.float32)
    lib().orc_score_f16(q.size, _p(q), _p(k), k.shape[0], sm, _p(out))
    return out


def delta_rho(q, s, z, sm):
    q = np.ascontiguousarray(q, np.uint16)
    dl = np.zeros(1, np.float32)
    rh = np.zeros(1, np.float32)
    lib().orc_delta_rho(q.size, _p(q), _p(np.ascontiguousarray(s, np.uint16)),
                        _p(np.ascontiguousarray(z, np.uint16)), sm, _p(dl), _p(rh))
    return float(dl[0]), float(rh[0])


def block_est(sc, n=64):
    sc = np.ascontiguousarray(sc, np.float32)
    mx = np.zeros(1, np.float32)
    l = np.zeros(1, np.float32)
    lib().orc_block_est(_p(sc), n, _p(mx), _p(l))
    return float(mx[0]), float(l[0])


def select(m, need):
    m = np.ascontiguousarray(m, np.uint64)
    in_set = np.zeros(m.size, np.uint8)
    k = lib().orc_select(m.size, _p(m), int(need), _p(in_set))
    return k, in_set


def discordant(key_a, key_b):
    a = np.ascontiguousarray(key_a, np.uint64)
    b = np.ascontiguousarray(key_b, np.uint64)
    return lib().orc_discordant(a.size, _p(a), _p(b))


def dense_head(k, v, q, g, sm):
    """k, v: [T][Hkv][d] uint16 of one sequence; q: [d] uint16."""
    k = np.ascontiguousarray(k, np.uint16)
    v = np.ascontiguousarray(v, np.uint16)
    q = np.ascontiguousarray(q, np.uint16)
    T, Hkv, d = k.shape
    out = np.zeros(d, np.float64)
    lib().orc_dense_head(T, Hkv, d, g, _p(k), _p(v), _p(q), sm, _p(out))
    return out
