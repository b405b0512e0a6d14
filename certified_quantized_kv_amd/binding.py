"""ctypes binding of libckv.so (same names as the C ABI in include/ckv.h)."""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libckv.so")
_lib = None

CKV_STATUS = {0: "CKV_OK", 1: "CKV_EINVAL", 2: "CKV_ENOMEM", 3: "CKV_EHIP", 4: "CKV_ERANGE",
              5: "CKV_ESTATE"}

EXPORTED = ["ckv_create", "ckv_destroy", "ckv_reset_sequence", "ckv_append_kv", "ckv_append_token",
            "ckv_certified_decode_attention", "ckv_dense_decode_attention", "ckv_footprint",
            "ckv_seq_length", "ckv_last_error", "ckv_export_block", "ckv_export_step",
            "ckv_set_profiling", "ckv_get_profile", "ckv_enable_fp16_cache",
            "ckv_set_device_paging", "ckv_set_staged_paging", "ckv_inject_paging_fault",
            "ckv_dense_decode_attention_noalloc", "ckv_read_probe"]


class CkvError(RuntimeError):
    def __init__(self, status, msg):
        self.status = status
        self.name = CKV_STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {msg}")


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int), ("max_batch", ctypes.c_int),
                ("n_q_heads", ctypes.c_int), ("n_kv_heads", ctypes.c_int),
                ("head_dim", ctypes.c_int), ("max_context", ctypes.c_int),
                ("device", ctypes.c_int), ("v_bits", ctypes.c_int)]


class Thresholds(ctypes.Structure):
    _fields_ = [("tau_cov", ctypes.c_float), ("k_tol", ctypes.c_float),
                ("v_tol", ctypes.c_float), ("rank_tol", ctypes.c_float),
                ("sm_scale", ctypes.c_float), ("f_layer", ctypes.c_float),
                ("n_widen", ctypes.c_int), ("v_cap_blocks", ctypes.c_int)]


class Profile(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * 10), ("counts", ctypes.c_int * 10), ("steps", ctypes.c_int),
                ("bytes_paged", ctypes.c_uint64), ("copies", ctypes.c_uint64),
                ("q8_blocks", ctypes.c_uint64), ("tail_blocks", ctypes.c_uint64),
                ("k16_blocks", ctypes.c_uint64), ("v16_blocks", ctypes.c_uint64),
                ("int4p_blocks", ctypes.c_uint64), ("dense_blocks", ctypes.c_uint64),
                ("gather_lead_ms", ctypes.c_double), ("gather_steps", ctypes.c_int),
                ("staged_threads", ctypes.c_int)]


PHASES = ["score", "select", "tail", "page", "promoted4", "fallback", "step", "merge", "keys16", "promoted16"]


REPORT_DTYPE = np.dtype([("e_key", "<f4"), ("e_val", "<f4"), ("tv_bound", "<f4"),
                         ("tau_final", "<f4"), ("kstar", "<i4"), ("n_v_promoted", "<i4"),
                         ("rank_ok", "<i4"), ("rung_max", "<i4"), ("rung_mask", "<i4"),
                         ("n_discordant", "<i4")])


def default_thresholds(sm_scale, **kw):
    t = dict(tau_cov=0.995, k_tol=1e-2, v_tol=1e-2, rank_tol=0.05, sm_scale=sm_scale,
             f_layer=0.5, n_widen=3, v_cap_blocks=0)
    t.update(kw)
    return t


def lib():
    """Load libckv.so; raise if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python certified_quantized_kv_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        szp = ctypes.POINTER(ctypes.c_size_t)
        L.ckv_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
        L.ckv_destroy.argtypes = [vp]
        L.ckv_destroy.restype = None
        L.ckv_reset_sequence.argtypes = [vp, i32]
        L.ckv_append_kv.argtypes = [vp, i32, i32, vp, vp, i32, i32, vp]
        L.ckv_append_token.argtypes = [vp, i32, i32, vp, vp, i32, vp]
        L.ckv_certified_decode_attention.argtypes = [vp, i32, vp, i32, ctypes.POINTER(Thresholds),
                                                     vp, vp, vp]
        L.ckv_dense_decode_attention.argtypes = [vp, vp, vp, i32, vp, i32, f32, vp, vp]
        L.ckv_dense_decode_attention_noalloc.argtypes = [vp, vp, i32, vp, i32, i32, i32, i32, f32,
                                                         vp, vp]
        L.ckv_footprint.argtypes = [vp, szp, szp, szp]
        L.ckv_seq_length.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_int)]
        L.ckv_last_error.argtypes = []
        L.ckv_last_error.restype = ctypes.c_char_p
        L.ckv_export_block.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]
        L.ckv_export_step.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int), vp, vp, vp, vp, vp,
                                      vp, vp, vp]
        L.ckv_set_profiling.argtypes = [vp, i32]
        L.ckv_get_profile.argtypes = [vp, ctypes.POINTER(Profile)]
        L.ckv_enable_fp16_cache.argtypes = [vp, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)]
        L.ckv_set_device_paging.argtypes = [vp, i32]
        L.ckv_set_staged_paging.argtypes = [vp, i32]
        L.ckv_inject_paging_fault.argtypes = [vp, i32]
        L.ckv_read_probe.argtypes = [vp, ctypes.c_size_t, i32, vp, vp]
        for name in EXPORTED:
            if name not in ("ckv_destroy", "ckv_last_error"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(st):
    if st != 0:
        raise CkvError(st, lib().ckv_last_error().decode())


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Cache:
    """A tiered KV cache: tier 1 (INT8 K / INT4 V / metadata / annotations)
    on the GPU, tier 2 (FP16 originals) in pinned host memory.  v_bits = 8
    stores the values at 8 bits (the symmetric cache configuration)."""

    def __init__(self, n_layers, max_batch, n_q_heads, n_kv_heads, head_dim, max_context, device=0, v_bits=4):
        self.cfg = Config(n_layers, max_batch, n_q_heads, n_kv_heads, head_dim, max_context, device, v_bits)
        self.n_layers, self.max_batch = n_layers, max_batch
        self.Hq, self.Hkv, self.d = n_q_heads, n_kv_heads, head_dim
        self.v_bits = v_bits
        self.device = device
        h = ctypes.c_void_p()
        _check(lib().ckv_create(ctypes.byref(self.cfg), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().ckv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    # -- tier construction -------------------------------------------------
    def reset_sequence(self, seq):
        _check(lib().ckv_reset_sequence(self._h, seq))

    def append_kv(self, layer, seq, k, v, stream=None):
        """k, v: [n_tokens][n_kv_heads][head_dim] FP16: torch tensors (device
        or host) or numpy uint16 / float16 arrays (host)."""
        if isinstance(k, np.ndarray):
            k = np.ascontiguousarray(k).view(np.uint16)
            v = np.ascontiguousarray(v).view(np.uint16)
            assert k.shape == v.shape and k.shape[1:] == (self.Hkv, self.d)
            _check(lib().ckv_append_kv(self._h, layer, seq, _np_ptr(k), _np_ptr(v), k.shape[0], 0,
                                       _stream_ptr(stream) if _torch_cuda() else None))
            return
        import torch
        assert k.dtype == torch.float16 and v.dtype == torch.float16 and k.shape == v.shape
        assert tuple(k.shape[1:]) == (self.Hkv, self.d)
        k = k.contiguous()
        v = v.contiguous()
        _check(lib().ckv_append_kv(self._h, layer, seq, ctypes.c_void_p(k.data_ptr()),
                                   ctypes.c_void_p(v.data_ptr()), k.shape[0], int(k.is_cuda),
                                   _stream_ptr(stream)))

    def append_token(self, layer, k, v, stream=None):
        """One decode token for each of sequences 0 .. batch-1: k, v
        [batch][n_kv_heads][head_dim] FP16 (torch tensors, device or host,
        or numpy arrays)."""
        if isinstance(k, np.ndarray):
            k = np.ascontiguousarray(k).view(np.uint16)
            v = np.ascontiguousarray(v).view(np.uint16)
            assert k.shape == v.shape and k.shape[1:] == (self.Hkv, self.d)
            _check(lib().ckv_append_token(self._h, layer, k.shape[0], _np_ptr(k), _np_ptr(v), 0,
                                          _stream_ptr(stream) if _torch_cuda() else None))
            return
        import torch
        assert k.dtype == torch.float16 and v.dtype == torch.float16 and k.shape == v.shape
        assert tuple(k.shape[1:]) == (self.Hkv, self.d)
        k = k.contiguous()
        v = v.contiguous()
        _check(lib().ckv_append_token(self._h, layer, k.shape[0], ctypes.c_void_p(k.data_ptr()),
                                      ctypes.c_void_p(v.data_ptr()), int(k.is_cuda), _stream_ptr(stream)))

    def set_device_paging(self, enable=True):
        """Page FP16 blocks with a device kernel reading pinned host memory
        (True) or with host-issued copies (False, the default)."""
        _check(lib().ckv_set_device_paging(self._h, int(bool(enable))))

    def set_staged_paging(self, threads):
        """Copy the listed FP16 blocks packed into 4 MiB pinned chunks by
        `threads` host threads (0: one copy per run of blocks)."""
        _check(lib().ckv_set_staged_paging(self._h, int(threads)))

    def enable_fp16_cache(self, max_bytes):
        """Keep paged FP16 blocks in device memory across steps for as many
        layers (from layer 0) as max_bytes allows; returns that layer count."""
        n = ctypes.c_int()
        _check(lib().ckv_enable_fp16_cache(self._h, ctypes.c_size_t(int(max_bytes)), ctypes.byref(n)))
        return n.value

    def seq_length(self, layer, seq):
        n = ctypes.c_int()
        _check(lib().ckv_seq_length(self._h, layer, seq, ctypes.byref(n)))
        return n.value

    def footprint(self):
        a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        _check(lib().ckv_footprint(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return dict(device=a.value, host=b.value, tier1=c.value)

    # -- the decode step ---------------------------------------------------
    def certified_decode_attention(self, layer, q, thresholds, out=None, stream=None):
        """q: torch.float16 CUDA tensor [batch][n_q_heads][head_dim].
        Returns (out [batch][n_q_heads][head_dim] float32 CUDA, report)."""
        import torch
        assert q.is_cuda and q.dtype == torch.float16 and q.shape[1:] == (self.Hq, self.d)
        q = q.contiguous()
        B = q.shape[0]
        if out is None:
            out = torch.empty((B, self.Hq, self.d), dtype=torch.float32, device=q.device)
        rep = np.zeros((B, self.Hq), REPORT_DTYPE)
        th = thresholds if isinstance(thresholds, Thresholds) else Thresholds(**thresholds)
        st = lib().ckv_certified_decode_attention(
            self._h, layer, ctypes.c_void_p(q.data_ptr()), B, ctypes.byref(th),
            ctypes.c_void_p(out.data_ptr()), _np_ptr(rep), _stream_ptr(stream))
        if st != 0:
            err = CkvError(st, lib().ckv_last_error().decode())
            err.report = rep   # every head at rung_max = -1
            raise err
        return out, rep

    def inject_paging_fault(self, after_copies=0):
        """Make the paging copy after `after_copies` further copies report
        failure (tests of the error path); < 0 clears the injection."""
        _check(lib().ckv_inject_paging_fault(self._h, int(after_copies)))

    def dense_decode_attention(self, k_blocks, v_blocks, n_tokens, q, sm_scale, out=None,
                               stream=None):
        """Exact dense attention on device FP16 K/V in the block layout
        [batch][n_kv_heads][n_tokens/64][64*head_dim] (K chunk-interleaved
        [head_dim/8][64][8], V channel-major [head_dim][64])."""
        import torch
        B = q.shape[0]
        if out is None:
            out = torch.empty((B, self.Hq, self.d), dtype=torch.float32, device=q.device)
        _check(lib().ckv_dense_decode_attention(
            self._h, ctypes.c_void_p(k_blocks.data_ptr()), ctypes.c_void_p(v_blocks.data_ptr()),
            n_tokens, ctypes.c_void_p(q.contiguous().data_ptr()), B, float(sm_scale),
            ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
        return out

    # -- introspection -----------------------------------------------------
    def export_block(self, layer, seq, kv_head, block):
        d = self.d
        r = dict(k_code=np.zeros((64, d), np.uint8), k_s=np.zeros(d, np.uint16),
                 k_z=np.zeros(d, np.uint16), v_code=np.zeros((64, d * self.v_bits // 8), np.uint8),
                 v_s=np.zeros((64, d // 32), np.uint16), v_z=np.zeros((64, d // 32), np.uint16),
                 eta=np.zeros(1, np.float32))
        _check(lib().ckv_export_block(self._h, layer, seq, kv_head, block,
                                      *[_np_ptr(r[k]) for k in ("k_code", "k_s", "k_z", "v_code",
                                                                 "v_s", "v_z", "eta")]))
        return r

    def export_step(self, batch):
        npo = ctypes.c_int()
        _check(lib().ckv_export_step(self._h, batch, ctypes.byref(npo), None, None, None, None,
                                     None, None, None, None))
        Np = npo.value
        B, Hq, Hkv = batch, self.Hq, self.Hkv
        # N: full blocks of the longest sequence in the step
        N = Np
        r = dict(score=np.zeros((B, Hq, Np * 64), np.float32),
                 bstat=np.zeros((B, Hq, Np, 4), np.float32), mref=np.zeros((B, Hq), np.float32),
                 mfx=np.zeros((B, Hq, Np), np.uint64), bounds=np.zeros((B, Hq, 4), np.float64),
                 seq_flags=np.zeros(B, np.int32))
        # sel and m16fx are sized by full blocks; ask with N = Np then trim
        sel = np.zeros((B, Hkv, N), np.uint32)
        m16 = np.zeros((B, Hq, N), np.uint64)
        _check(lib().ckv_export_step(self._h, batch, ctypes.byref(npo), _np_ptr(r["score"]),
                                     _np_ptr(r["bstat"]), _np_ptr(r["mref"]), _np_ptr(r["mfx"]),
                                     _np_ptr(sel), _np_ptr(m16), _np_ptr(r["bounds"]),
                                     _np_ptr(r["seq_flags"])))
        r["sel"] = sel
        r["m16fx"] = m16
        return r

    def set_profiling(self, enable=True):
        _check(lib().ckv_set_profiling(self._h, int(enable)))

    def profile(self):
        """Profile since set_profiling(True): phase times {name: (ms, count)}
        and the counters of ckv_profile."""
        p = Profile()
        _check(lib().ckv_get_profile(self._h, ctypes.byref(p)))
        r = {f: getattr(p, f) for f, _ in Profile._fields_ if f not in ("ms", "counts")}
        r["phases"] = {nm: (float(p.ms[i]), int(p.counts[i])) for i, nm in enumerate(PHASES)}
        return r


def dense_decode_attention_noalloc(k_blocks, v_blocks, n_tokens, q, sm_scale, n_kv_heads, out,
                                   stream=None):
    """ckv_dense_decode_attention_noalloc: exact dense attention without a
    cache and without allocating (the caller passes `out`, a float32 CUDA
    tensor [batch][n_q_heads][head_dim]); k_blocks, v_blocks in the block
    layout of Cache.dense_decode_attention."""
    B, Hq, d = q.shape
    _check(lib().ckv_dense_decode_attention_noalloc(
        ctypes.c_void_p(k_blocks.data_ptr()), ctypes.c_void_p(v_blocks.data_ptr()), int(n_tokens),
        ctypes.c_void_p(q.data_ptr()), B, Hq, int(n_kv_heads), d, float(sm_scale),
        ctypes.c_void_p(out.data_ptr()), _stream_ptr(stream)))
    return out


def read_probe(buf, wave_kib, sink, stream=None):
    """ckv_read_probe: enqueue one streaming read of the CUDA tensor `buf`
    (its whole storage) in waves of wave_kib KiB; `sink` is a one-word int32
    CUDA tensor."""
    assert buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.numel() >= 1
    _check(lib().ckv_read_probe(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                                int(wave_kib), ctypes.c_void_p(sink.data_ptr()), _stream_ptr(stream)))


def _torch_cuda():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False
