"""Plain CPU oracle for causal GQA attention over a per-layer KV cache.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product path (the HIP library and its
Python binding) never imports this package, and this package never imports the
product: the two share no code.

`oracle.c` holds every step, written from the pages (see its header for sources);
this module only compiles it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, E_ARG, E_GEOMETRY, E_RANGE, E_DUP, E_NOMEM = 0, 1, 2, 3, 4, 5
ROPE_NEOX, ROPE_INTERLEAVED, ROPE_NONE = 0, 1, 2
KV_F32, KV_F16, KV_Q8_0 = 0, 1, 2
Q8_BLOCK, Q8_BLOCK_BYTES = 32, 34

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
          "-std=c11", "-Wall", "-Wextra"]


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_lib = None


def _bind(lib):
    i32, f32, p = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
    sig = {
        "orc_rope_inv_freq": (ctypes.c_int, [i32, f32, f32, p]),
        "orc_rope_cos_sin": (ctypes.c_int, [i32, f32, f32, i32, p, p]),
        "orc_rope": (ctypes.c_int, [p, i32, i32, i32, p, f32, f32, i32]),
        "orc_cache_new": (p, [i32, i32, i32, i32, i32]),
        "orc_cache_new_typed": (p, [i32, i32, i32, i32, i32, i32]),
        "orc_f32_to_f16": (ctypes.c_uint16, [f32]),
        "orc_f16_to_f32": (f32, [ctypes.c_uint16]),
        "orc_q8_quantize_row": (ctypes.c_int, [p, i32, p]),
        "orc_q8_dequantize_row": (ctypes.c_int, [p, i32, p]),
        "orc_cache_free": (None, [p]),
        "orc_cache_region": (p, [p, i32, i32, i32]),
        "orc_cache_seq_len": (i32, [p, i32, i32]),
        "orc_append_rope": (ctypes.c_int, [p, i32, i32, p, p, p, i32, i32, p, p, f32, f32, i32]),
        "orc_attn_prefill": (ctypes.c_int, [p, i32, i32, i32, p, p, i32, i32, f32, p, i32]),
        "orc_attn_decode": (ctypes.c_int, [p, i32, i32, p, p, p, i32, i32, f32, p, i32]),
        "orc_attn_decode_runs": (ctypes.c_int, [p, i32, i32, p, p, p, p, p, i32, i32, f32, p,
                                                i32]),
        "orc_max_threads": (i32, []),
        "orc_project": (ctypes.c_int, [p, p, p, i32, i32, i32, p]),
        "orc_qkv_rope_append": (ctypes.c_int, [p, i32, i32, p, p, p, i32, p, p, p, p, p, p, i32,
                                               i32, p, f32, f32, i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def lib(path: str | None = None):
    """Load (building first if needed) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def _i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


class Oracle:
    """numpy-facing wrapper over one oracle library (the default one or a given path)."""

    def __init__(self, path: str | None = None):
        self.L = lib(path)

    def max_threads(self) -> int:
        return int(self.L.orc_max_threads())

    def rope_inv_freq(self, hd, base, scale=1.0):
        out = np.zeros(max(hd // 2, 1), np.float32)
        st = self.L.orc_rope_inv_freq(hd, base, scale, _ptr(out))
        if st:
            raise ValueError(f"orc_rope_inv_freq status {st}")
        return out[: hd // 2]

    def rope_cos_sin(self, hd, base, scale, p):
        cs = np.zeros(hd // 2, np.float32)
        sn = np.zeros(hd // 2, np.float32)
        st = self.L.orc_rope_cos_sin(hd, base, scale, p, _ptr(cs), _ptr(sn))
        if st:
            raise ValueError(f"orc_rope_cos_sin status {st}")
        return cs, sn

    def f32_to_f16(self, x):
        """Element-wise binary16 bit patterns (uint16) of f32 values."""
        x = np.asarray(x, np.float32).ravel()
        return np.array([self.L.orc_f32_to_f16(float(v)) for v in x], np.uint16)

    def f16_to_f32(self, h):
        h = np.asarray(h, np.uint16).ravel()
        return np.array([self.L.orc_f16_to_f32(int(v)) for v in h], np.float32)

    def q8_quantize(self, x):
        """Q8_0 blocks of a 1-D array (length a multiple of 32), as raw bytes
        [n/32][34]: binary16 scale (little-endian) then 32 int8 codes."""
        x = _f32(x).ravel()
        out = np.zeros((x.size // Q8_BLOCK, Q8_BLOCK_BYTES), np.uint8)
        st = self.L.orc_q8_quantize_row(_ptr(x), x.size, _ptr(out))
        if st:
            raise ValueError(f"orc_q8_quantize_row status {st}")
        return out

    def q8_dequantize(self, blocks):
        blocks = np.ascontiguousarray(blocks, np.uint8).reshape(-1, Q8_BLOCK_BYTES)
        out = np.zeros(blocks.shape[0] * Q8_BLOCK, np.float32)
        st = self.L.orc_q8_dequantize_row(_ptr(blocks), out.size, _ptr(out))
        if st:
            raise ValueError(f"orc_q8_dequantize_row status {st}")
        return out

    def project(self, x, w, b=None):
        """x [nt][d] . w[rows][d]^T + b -> [nt][rows] (exact dot rounded to f32, then + b)."""
        x, w = _f32(x), _f32(w)
        b = None if b is None else _f32(b)
        nt, d = x.shape
        rows = w.shape[0]
        out = np.zeros((nt, rows), np.float32)
        st = self.L.orc_project(_ptr(x), _ptr(w), _ptr(b), nt, rows, d, _ptr(out))
        if st:
            raise ValueError(f"orc_project status {st}")
        return out

    def rope(self, x, pos, base, scale=1.0, style=ROPE_NEOX):
        """x: [nt][nh][hd]; returns a rotated copy."""
        x = _f32(x).copy()
        pos = _i32(pos)
        nt, nh, hd = x.shape
        st = self.L.orc_rope(_ptr(x), nt, nh, hd, _ptr(pos), base, scale, style)
        if st:
            raise ValueError(f"orc_rope status {st}")
        return x


def q8_split(blocks):
    """Split Q8_0 blocks [..., 34] into (scales uint16 [...], codes int8 [..., 32])."""
    b = np.ascontiguousarray(blocks, np.uint8)
    scales = b[..., :2].copy().view(np.uint16)[..., 0]
    codes = b[..., 2:].copy().view(np.int8)
    return scales, codes


def runs_csr(runs):
    """Per-query lists of (start, len) runs -> (run_off [n+1], run_start, run_len) int32."""
    off = np.zeros(len(runs) + 1, np.int32)
    starts, lens = [], []
    for b, rl in enumerate(runs):
        for st, ln in rl:
            starts.append(st)
            lens.append(ln)
        off[b + 1] = len(starts)
    return off, np.array(starts, np.int32), np.array(lens, np.int32)


class OracleCache:
    """The oracle's KV cache: zeroed regions [n_seq][n_layer][capacity][n_head_kv*hd_kv] of
    f32 values (dtype KV_F32) or binary16 bit patterns (KV_F16)."""

    def __init__(self, n_seq, n_layer, n_head_kv, hd_kv, capacity, oracle: Oracle | None = None,
                 dtype: int = KV_F32):
        self.o = oracle or Oracle()
        self.L = self.o.L
        self.n_seq, self.n_layer = n_seq, n_layer
        self.n_head_kv, self.hd_kv, self.capacity = n_head_kv, hd_kv, capacity
        self.nkt = n_head_kv * hd_kv
        self.dtype = dtype
        self.h = self.L.orc_cache_new_typed(n_seq, n_layer, n_head_kv, hd_kv, capacity, dtype)
        if not self.h:
            raise ValueError("orc_cache_new rejected the geometry")

    def close(self):
        if self.h:
            self.L.orc_cache_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def region(self, which, seq, layer) -> np.ndarray:
        """Live numpy view of one region; which=0 for K, 1 for V.  [capacity][nkt]
        float32 for an f32 cache, uint16 (binary16 bits) for an f16 cache; for a Q8_0
        cache [capacity][nkt/32][34] bytes (see q8_split)."""
        ptr = self.L.orc_cache_region(self.h, which, seq, layer)
        if not ptr:
            raise IndexError("bad seq/layer")
        n = self.capacity * self.nkt
        if self.dtype == KV_Q8_0:
            nb = n // Q8_BLOCK * Q8_BLOCK_BYTES
            buf = (ctypes.c_uint8 * nb).from_address(ptr)
            return np.frombuffer(buf, dtype=np.uint8).reshape(self.capacity, self.nkt // Q8_BLOCK,
                                                              Q8_BLOCK_BYTES)
        if self.dtype == KV_F16:
            buf = (ctypes.c_uint16 * n).from_address(ptr)
            return np.frombuffer(buf, dtype=np.uint16).reshape(self.capacity, self.nkt)
        buf = (ctypes.c_float * n).from_address(ptr)
        return np.frombuffer(buf, dtype=np.float32).reshape(self.capacity, self.nkt)

    def k(self, seq, layer):
        return self.region(0, seq, layer)

    def v(self, seq, layer):
        return self.region(1, seq, layer)

    def seq_len(self, seq, layer) -> int:
        return int(self.L.orc_cache_seq_len(self.h, seq, layer))

    def append_rope(self, layer, seq_ids, pos, q, n_head, hd, k, v, base, scale=1.0,
                    style=ROPE_NEOX):
        """Returns (status, rotated q copy or None)."""
        seq_ids, pos = _i32(seq_ids), _i32(pos)
        nt = int(pos.shape[0])
        qq = None if q is None else _f32(q).copy()
        k, v = _f32(k), _f32(v)
        st = self.L.orc_append_rope(self.h, layer, nt, _ptr(seq_ids), _ptr(pos), _ptr(qq),
                                    n_head, hd, _ptr(k), _ptr(v), base, scale, style)
        return st, qq

    def attn_prefill(self, seq, layer, pos, q, n_head, hd, scale, nthreads=0):
        pos = _i32(pos)
        nt = int(pos.shape[0])
        q = _f32(q)
        out = np.zeros((nt, n_head, self.hd_kv), np.float32)
        st = self.L.orc_attn_prefill(self.h, seq, layer, nt, _ptr(pos), _ptr(q), n_head, hd,
                                     scale, _ptr(out), nthreads)
        return st, out

    def attn_decode(self, layer, seq_ids, pos, q, n_head, hd, scale, nthreads=0):
        seq_ids, pos = _i32(seq_ids), _i32(pos)
        n = int(pos.shape[0])
        q = _f32(q)
        out = np.zeros((n, n_head, self.hd_kv), np.float32)
        st = self.L.orc_attn_decode(self.h, layer, n, _ptr(seq_ids), _ptr(pos), _ptr(q), n_head,
                                    hd, scale, _ptr(out), nthreads)
        return st, out

    def attn_decode_runs(self, layer, seq_ids, runs, q, n_head, hd, scale, nthreads=0):
        """runs: per query, a list of (start, len) cell runs (its explicit window)."""
        seq_ids = _i32(seq_ids)
        n = int(seq_ids.shape[0])
        off, starts, lens = runs_csr(runs)
        if starts.size == 0:   # keep valid pointers for the call
            starts, lens = np.zeros(1, np.int32), np.zeros(1, np.int32)
        q = _f32(q)
        out = np.zeros((n, n_head, self.hd_kv), np.float32)
        st = self.L.orc_attn_decode_runs(self.h, layer, n, _ptr(seq_ids), _ptr(off), _ptr(starts),
                                         _ptr(lens), _ptr(q), n_head, hd, scale, _ptr(out),
                                         nthreads)
        return st, out

    def qkv_rope_append(self, layer, seq_ids, pos, x, wq, bq, wk, bk, wv, bv, n_head, hd, base,
                        scale=1.0, style=ROPE_NEOX):
        """Fused decode step; returns (status, rotated q [nt][n_head][hd])."""
        seq_ids, pos = _i32(seq_ids), _i32(pos)
        nt = int(pos.shape[0])
        ws = [None if a is None else _f32(a) for a in (wq, bq, wk, bk, wv, bv)]
        x = None if x is None else _f32(x)
        d_model = ws[0].shape[-1] if x is None else x.shape[-1]
        q = np.zeros((nt, n_head, hd), np.float32)
        st = self.L.orc_qkv_rope_append(self.h, layer, nt, _ptr(seq_ids), _ptr(pos), _ptr(x),
                                        d_model, *[_ptr(a) for a in ws], n_head, hd, _ptr(q),
                                        base, scale, style)
        return st, q
