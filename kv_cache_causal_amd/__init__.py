"""Python binding of libkvc.so: causal GQA attention over a per-layer KV cache on MI355X.

Argument marshalling only.  Every step of the path (RoPE tables, RoPE + append,
split-K decode, MFMA prefill) runs in the library's gfx950 kernels; this module turns
torch device tensors into pointers, numpy/list host arrays into int32 buffers, picks the
current torch stream, and raises KvcError on a non-OK status.  There is no fallback: if
the library is not built, importing works but every call raises.

The functions carry the C names of include/kvc.h and take the same arguments, minus the
sizes the tensors already carry.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libkvc.so")

OK, E_ARG, E_GEOMETRY, E_RANGE, E_DUP, E_NOMEM, E_HIP = range(7)
ROPE_NEOX, ROPE_INTERLEAVED, ROPE_NONE = 0, 1, 2
KV_F32, KV_F16, KV_Q8_0 = 0, 1, 2
REGION_ROW_ALIGN = 64   # region rows = capacity rounded up to this
STATUS_NAMES = {0: "KVC_OK", 1: "KVC_E_ARG", 2: "KVC_E_GEOMETRY", 3: "KVC_E_RANGE",
                4: "KVC_E_DUP", 5: "KVC_E_NOMEM", 6: "KVC_E_HIP"}

# Every symbol include/kvc.h declares.
EXPORTS = ("kv_alloc", "kv_alloc_typed", "kv_free", "kv_view", "kv_seq_len", "kv_append_rope",
           "kv_qkv_rope_append", "gqa_attn_prefill", "gqa_attn_decode", "gqa_attn_decode_noalloc",
           "gqa_attn_decode_runs", "kv_last_error")
STATIC_SCRATCH_BYTES = 16 << 20   # the fixed scratch of gqa_attn_decode_noalloc


class KvcError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


_lib = None


def lib(path: str = LIB_PATH):
    """Load libkvc.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(python -m kv_cache_causal_amd._build)")
    # One HIP runtime per process: torch ships its own libamdhip64.so.7 (same soname as
    # the system one libkvc.so was linked against).  Loading torch first makes libkvc.so
    # bind to the runtime that owns torch's device memory and streams.
    import torch  # noqa: F401
    L = ctypes.CDLL(path)
    i32, f32, p = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    sig = {
        "kv_alloc": [ctypes.POINTER(p), i32, i32, i32, i32, i32, p],
        "kv_alloc_typed": [ctypes.POINTER(p), i32, i32, i32, i32, i32, ctypes.c_int, p],
        "kv_free": [p],
        "kv_view": [p, i32, i32, ctypes.POINTER(p), ctypes.POINTER(p)],
        "kv_seq_len": [p, i32, i32, ctypes.POINTER(i32)],
        "kv_append_rope": [p, i32, i32, p, p, p, i32, i32, p, p, f32, f32, ctypes.c_int, p],
        "kv_qkv_rope_append": [p, i32, i32, p, p, p, i32, p, p, p, p, p, p, i32, i32, p, f32, f32,
                               ctypes.c_int, p],
        "gqa_attn_prefill": [p, i32, i32, i32, p, p, i32, i32, f32, p, p],
        "gqa_attn_decode": [p, i32, i32, p, p, p, i32, i32, f32, p, p],
        "gqa_attn_decode_noalloc": [p, i32, i32, p, p, p, i32, i32, f32, p, p],
        "gqa_attn_decode_runs": [p, i32, i32, p, p, p, p, p, i32, i32, f32, p, p],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.kv_last_error.argtypes = []
    L.kv_last_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = L
    return L


def kv_last_error() -> str:
    return lib().kv_last_error().decode()


def _check(st: int):
    if st != OK:
        raise KvcError(st, kv_last_error())


def _stream(stream):
    if stream is not None:
        return int(stream)
    import torch
    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)   # no Stream object built
    if raw is not None:
        return int(raw(torch.cuda.current_device()))
    return int(torch.cuda.current_stream().cuda_stream)


def _dev(t, name, numel=0):
    """Device pointer of a dense f32 torch CUDA tensor (or None / a raw int pointer).
    numel: elements the call reads or writes through it; a shorter tensor raises
    ValueError (the kernels would run past its end).  A raw pointer is taken as is."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not (t.is_cuda and t.dtype.is_floating_point and t.element_size() == 4):
        raise TypeError(f"{name} must be an f32 tensor on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the call uses {numel}")
    return t.data_ptr()


# Data pointers of the last few small int32 arrays passed (id -> (array, pointer)).
# Reading ndarray.ctypes.data costs ~1 us, a large share of a small call's host time, and
# callers pass the same position / sequence arrays call after call.  The entry holds a
# reference, so the id cannot be reused and the buffer cannot move (an in-place resize
# refuses while another reference exists) until the entry is dropped.
_PTRS = {}
_PTRS_MAX = 16
_PTRS_MAX_SIZE = 64


def _host_i32(a):
    """(a contiguous 1-D int32 array holding a's values, its data pointer)."""
    if type(a) is np.ndarray and a.dtype == np.int32 and a.ndim == 1 and a.flags.c_contiguous:
        hit = _PTRS.get(id(a))
        if hit is not None and hit[0] is a:
            return a, hit[1]
        ptr = a.ctypes.data
        if a.size <= _PTRS_MAX_SIZE:
            if len(_PTRS) >= _PTRS_MAX:
                _PTRS.clear()
            _PTRS[id(a)] = (a, ptr)
        return a, ptr
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))
    return a, a.ctypes.data


class Cache:
    """Owning wrapper of a kvc_cache handle (kv_free on close / garbage collection).
    dtype KV_F32 (kv_alloc), KV_F16 (binary16 regions) or KV_Q8_0 (Q8_0 blocks), the
    last two through kv_alloc_typed."""

    def __init__(self, n_seq, n_layer, n_head_kv, hd_kv, capacity, stream=None, dtype=KV_F32):
        self.n_seq, self.n_layer = n_seq, n_layer
        self.n_head_kv, self.hd_kv, self.capacity = n_head_kv, hd_kv, capacity
        self.nkt = n_head_kv * hd_kv
        self.dtype = dtype
        h = ctypes.c_void_p()
        if dtype == KV_F32:
            st = lib().kv_alloc(ctypes.byref(h), n_seq, n_layer, n_head_kv, hd_kv, capacity,
                                _stream(stream))
        else:
            st = lib().kv_alloc_typed(ctypes.byref(h), n_seq, n_layer, n_head_kv, hd_kv,
                                      capacity, dtype, _stream(stream))
        _check(st)
        self.handle = h.value

    def close(self):
        if getattr(self, "handle", None):
            h, self.handle = self.handle, None
            _check(lib().kv_free(h))

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def kv_alloc(n_seq, n_layer, n_head_kv, hd_kv, capacity, stream=None, dtype=KV_F32) -> Cache:
    return Cache(n_seq, n_layer, n_head_kv, hd_kv, capacity, stream, dtype)


def kv_free(c: Cache):
    c.close()


def kv_view(c: Cache, seq: int, layer: int):
    """(k_ptr, v_ptr): device addresses of the [capacity][n_head_kv*hd_kv] regions."""
    k, v = ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib().kv_view(c.handle, seq, layer, ctypes.byref(k), ctypes.byref(v)))
    return k.value, v.value


def kv_seq_len(c: Cache, seq: int, layer: int) -> int:
    n = ctypes.c_int32()
    _check(lib().kv_seq_len(c.handle, seq, layer, ctypes.byref(n)))
    return n.value


def kv_append_rope(c: Cache, layer, seq_ids, pos, q, n_head, hd, k, v, freq_base,
                   freq_scale=1.0, style=ROPE_NEOX, stream=None):
    """q: [nt][n_head][hd] f32 CUDA tensor or None (rotated in place); k, v:
    [nt][n_head_kv][hd_kv].  seq_ids, pos: host int arrays of length nt."""
    s_arr, s_ptr = _host_i32(seq_ids)
    p_arr, p_ptr = _host_i32(pos)
    if s_arr.size != p_arr.size:
        raise ValueError("seq_ids and pos differ in length")
    nt = int(p_arr.size)
    nq = nt * n_head * hd if style != ROPE_NONE else 0   # NONE leaves q untouched
    _check(lib().kv_append_rope(c.handle, layer, nt, s_ptr, p_ptr, _dev(q, "q", nq),
                                n_head, hd, _dev(k, "k", nt * c.nkt), _dev(v, "v", nt * c.nkt),
                                freq_base, freq_scale, style, _stream(stream)))


def kv_qkv_rope_append(c: Cache, layer, seq_ids, pos, x, wq, bq, wk, bk, wv, bv, n_head, hd,
                       q_out, freq_base, freq_scale=1.0, style=ROPE_NEOX, stream=None):
    """Fused decode step: projections (x [nt][d_model] against row-major weights, optional
    biases), RoPE, K/V store; the rotated q goes to q_out [nt][n_head][hd]."""
    s_arr, s_ptr = _host_i32(seq_ids)
    p_arr, p_ptr = _host_i32(pos)
    if s_arr.size != p_arr.size:
        raise ValueError("seq_ids and pos differ in length")
    d_model = int(x.shape[-1]) if hasattr(x, "shape") else 0
    nt, rq, rkv = int(p_arr.size), n_head * hd, c.nkt
    _check(lib().kv_qkv_rope_append(c.handle, layer, nt, s_ptr, p_ptr, _dev(x, "x", nt * d_model),
                                    d_model, _dev(wq, "wq", rq * d_model), _dev(bq, "bq", rq),
                                    _dev(wk, "wk", rkv * d_model), _dev(bk, "bk", rkv),
                                    _dev(wv, "wv", rkv * d_model), _dev(bv, "bv", rkv), n_head, hd,
                                    _dev(q_out, "q_out", nt * rq), freq_base, freq_scale, style,
                                    _stream(stream)))


def gqa_attn_prefill(c: Cache, seq, layer, pos, q, n_head, hd, scale, out, stream=None):
    p_arr, p_ptr = _host_i32(pos)
    nt = int(p_arr.size)
    _check(lib().gqa_attn_prefill(c.handle, seq, layer, nt, p_ptr, _dev(q, "q", nt * n_head * hd),
                                  n_head, hd, scale, _dev(out, "out", nt * n_head * c.hd_kv),
                                  _stream(stream)))


def gqa_attn_decode(c: Cache, layer, seq_ids, pos, q, n_head, hd, scale, out, stream=None):
    s_arr, s_ptr = _host_i32(seq_ids)
    p_arr, p_ptr = _host_i32(pos)
    if s_arr.size != p_arr.size:
        raise ValueError("seq_ids and pos differ in length")
    n = int(p_arr.size)
    _check(lib().gqa_attn_decode(c.handle, layer, n, s_ptr, p_ptr, _dev(q, "q", n * n_head * hd),
                                 n_head, hd, scale, _dev(out, "out", n * n_head * c.hd_kv),
                                 _stream(stream)))


def gqa_attn_decode_noalloc(c: Cache, layer, seq_ids, pos, q, n_head, hd, scale, out,
                            stream=None):
    """gqa_attn_decode with its split-K records in the library's fixed scratch: the call
    allocates nothing (see kvc.h for the size limit and the sharing rule)."""
    s_arr, s_ptr = _host_i32(seq_ids)
    p_arr, p_ptr = _host_i32(pos)
    if s_arr.size != p_arr.size:
        raise ValueError("seq_ids and pos differ in length")
    n = int(p_arr.size)
    _check(lib().gqa_attn_decode_noalloc(c.handle, layer, n, s_ptr, p_ptr,
                                         _dev(q, "q", n * n_head * hd), n_head, hd, scale,
                                         _dev(out, "out", n * n_head * c.hd_kv), _stream(stream)))


def gqa_attn_decode_runs(c: Cache, layer, seq_ids, runs, q, n_head, hd, scale, out,
                         stream=None):
    """runs: for each entry, a list of (start, len) row runs -- its explicit window."""
    s_arr, s_ptr = _host_i32(seq_ids)
    if s_arr.size != len(runs):
        raise ValueError("seq_ids and runs differ in length")
    off = [0]
    starts, lens = [], []
    for rl in runs:
        for st, ln in rl:
            starts.append(st)
            lens.append(ln)
        off.append(len(starts))
    o_arr, o_ptr = _host_i32(off)
    st_arr, st_ptr = _host_i32(starts if starts else [0])
    ln_arr, ln_ptr = _host_i32(lens if lens else [0])
    n = int(s_arr.size)
    _check(lib().gqa_attn_decode_runs(c.handle, layer, n, s_ptr, o_ptr, st_ptr, ln_ptr,
                                      _dev(q, "q", n * n_head * hd), n_head, hd, scale,
                                      _dev(out, "out", n * n_head * c.hd_kv), _stream(stream)))


_hip = None


def kv_read(c: Cache, seq: int, layer: int, stream=None):
    """Copies (device to device, on `stream`) of one (seq, layer)'s K and V regions as
    [capacity][n_head_kv * hd_kv] torch tensors (float32, or float16 for a binary16
    cache).  For a Q8_0 cache each of K and V is a pair (codes int8 [rows][nkt], scales
    int16 holding binary16 bits [n_head_kv][rows][hd_kv / 32]) over all rows = capacity
    rounded up to 64; the scales come in that logical order (the region interleaves them
    by row quads, see kv_alloc_typed).  For inspection and tests."""
    global _hip
    import torch
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch already loaded (by soname)
        _hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_void_p]
        _hip.hipMemcpyAsync.restype = ctypes.c_int
    kp, vp = kv_view(c, seq, layer)
    out = []
    if c.dtype == KV_Q8_0:
        rows = -(-c.capacity // REGION_ROW_ALIGN) * REGION_ROW_ALIGN
        nbytes = rows * c.nkt + rows * (c.nkt // 32) * 2
        for src in (kp, vp):
            t = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            e = _hip.hipMemcpyAsync(t.data_ptr(), src, nbytes, 3, _stream(stream))
            if e != 0:
                raise RuntimeError(f"hipMemcpyAsync failed: {e}")
            codes = t[: rows * c.nkt].view(torch.int8).reshape(rows, c.nkt)
            scales = (t[rows * c.nkt:].view(torch.int16)
                      .reshape(c.n_head_kv, rows // 4, c.hd_kv // 32, 4)
                      .permute(0, 1, 3, 2).reshape(c.n_head_kv, rows, c.hd_kv // 32))
            out.append((codes, scales))
        return out[0], out[1]
    for src in (kp, vp):
        dt = torch.float16 if c.dtype == KV_F16 else torch.float32
        t = torch.empty((c.capacity, c.nkt), dtype=dt, device="cuda")
        e = _hip.hipMemcpyAsync(t.data_ptr(), src, c.capacity * c.nkt * t.element_size(), 3,
                                _stream(stream))
        if e != 0:
            raise RuntimeError(f"hipMemcpyAsync failed: {e}")
        out.append(t)
    return out[0], out[1]
