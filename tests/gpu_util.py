"""Helpers for the GPU parity tests: move seeded numpy inputs to the device, run the same
call on the HIP library and on the oracle, compare.

Bars: cache regions, rotated q and high-water marks bit for bit; attention outputs
elementwise |gpu - oracle| <= ATOL + RTOL * |oracle| (max-abs 1e-4 / max-rel 1e-5 read
as an allclose rule, since a separate max-relative bar cannot hold where outputs pass
through zero)."""
from __future__ import annotations

import sys

import numpy as np

ATOL, RTOL = 1e-4, 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def bits(a):
    a = np.asarray(a)
    if a.dtype in (np.float16, np.uint16):
        return np.ascontiguousarray(a).view(np.uint16)
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def assert_bitwise(gpu, orc, what):
    g, o = bits(gpu), bits(orc)
    if not np.array_equal(g, o):
        bad = np.argwhere(g != o)
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements differ; first at {idx}: "
                             f"gpu {np.asarray(gpu)[idx]!r} oracle {np.asarray(orc)[idx]!r}")


def assert_close(gpu, orc, what):
    gpu = np.asarray(gpu, np.float64)
    orc = np.asarray(orc, np.float64)
    assert gpu.shape == orc.shape, (what, gpu.shape, orc.shape)
    assert np.isfinite(gpu).all(), f"{what}: non-finite GPU output"
    err = np.abs(gpu - orc)
    bound = ATOL + RTOL * np.abs(orc)
    ok = err <= bound
    if not ok.all():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} of {err.size} outside "
                             f"{ATOL} + {RTOL}|o|; worst at {i}: gpu {gpu[i]} oracle {orc[i]}")
    rel = err / np.maximum(np.abs(orc), 1e-30)
    say(f"  {what}: max-abs {err.max():.3e}  max-rel(|o|>1e-3) "
        f"{(rel[np.abs(orc) > 1e-3].max() if (np.abs(orc) > 1e-3).any() else 0.0):.3e}")


def assert_equal(gpu, orc, what):
    """Exact equality of integer arrays (codes, bit patterns)."""
    gpu, orc = np.asarray(gpu), np.asarray(orc)
    assert gpu.shape == orc.shape, (what, gpu.shape, orc.shape)
    if not np.array_equal(gpu, orc):
        bad = np.argwhere(gpu != orc)
        idx = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} elements differ; first at {idx}: "
                             f"gpu {gpu[idx]!r} oracle {orc[idx]!r}")


def compare_q8_cache(lib_cache, orc_cache, seq, layer, what, rows=None):
    """Q8_0 regions: the library's code and scale planes against the oracle's 34-byte
    blocks, bit for bit; the padding rows past the capacity must still be zero."""
    import kv_cache_causal_amd as kvc
    from oracle import q8_split
    cap, nkt = orc_cache.capacity, orc_cache.nkt
    sel = slice(None) if rows is None else rows
    for name, (codes, scales), reg in zip("KV", kvc.kv_read(lib_cache, seq, layer),
                                          (orc_cache.k(seq, layer), orc_cache.v(seq, layer))):
        codes = host(codes)
        # head-major [n_head_kv][rows][hd_kv/32] -> [rows][nkt/32] like the oracle's blocks
        scales = host(scales).view(np.uint16).transpose(1, 0, 2).reshape(codes.shape[0], -1)
        osc, ocd = q8_split(reg)
        assert_equal(codes[:cap][sel], ocd.reshape(cap, nkt)[sel], f"{what} {name} codes [{seq}][{layer}]")
        assert_equal(scales[:cap][sel], osc[sel], f"{what} {name} scales [{seq}][{layer}]")
        assert not codes[cap:].any() and not scales[cap:].any(), f"{what} {name}: padding rows written"


def compare_cache(lib_cache, orc_cache, seq, layer, what, rows=None):
    import kv_cache_causal_amd as kvc
    if lib_cache.dtype == kvc.KV_Q8_0:
        compare_q8_cache(lib_cache, orc_cache, seq, layer, what, rows)
    else:
        compare_dense_cache(lib_cache, orc_cache, seq, layer, what, rows)
    assert kvc.kv_seq_len(lib_cache, seq, layer) == orc_cache.seq_len(seq, layer), \
        (what, seq, layer, kvc.kv_seq_len(lib_cache, seq, layer), orc_cache.seq_len(seq, layer))


def compare_dense_cache(lib_cache, orc_cache, seq, layer, what, rows=None):
    import kv_cache_causal_amd as kvc
    K, V = kvc.kv_read(lib_cache, seq, layer)
    K, V = host(K), host(V)   # float16 arrays for a binary16 cache: compared as bits
    ok, ov = orc_cache.k(seq, layer), orc_cache.v(seq, layer)
    if rows is not None:
        K, V, ok, ov = K[rows], V[rows], ok[rows], ov[rows]
    assert_bitwise(K, ok, f"{what} K[{seq}][{layer}]")
    assert_bitwise(V, ov, f"{what} V[{seq}][{layer}]")


class Pair:
    """A library cache and an oracle cache of the same geometry, driven in lock step."""

    def __init__(self, n_seq, n_layer, n_head_kv, hd_kv, capacity, dtype=0):
        import kv_cache_causal_amd as kvc
        from oracle import OracleCache
        self.kvc = kvc
        self.g = kvc.kv_alloc(n_seq, n_layer, n_head_kv, hd_kv, capacity, dtype=dtype)
        self.o = OracleCache(n_seq, n_layer, n_head_kv, hd_kv, capacity, dtype=dtype)
        self.n_head_kv, self.hd_kv = n_head_kv, hd_kv

    def close(self):
        self.g.close()
        self.o.close()

    def append(self, layer, seq_ids, pos, q, n_head, hd, k, v, base=1e6, fscale=1.0, style=0,
               check_q=True):
        """Append on both; returns (gpu rotated q as numpy or None, oracle rotated q)."""
        qd = None if q is None else dev(q)
        self.kvc.kv_append_rope(self.g, layer, seq_ids, pos, qd, n_head, hd, dev(k), dev(v), base,
                                fscale, style)
        st, qo = self.o.append_rope(layer, seq_ids, pos, q, n_head, hd, k, v, base, fscale, style)
        assert st == 0, st
        if q is not None and check_q:
            assert_bitwise(host(qd), qo, "rotated q")
        return qd, qo

    def prefill(self, seq, layer, pos, q_dev, q_host, n_head, hd, scale, sample=None):
        import torch
        nt = len(pos)
        out = torch.empty((nt, n_head, self.hd_kv), dtype=torch.float32, device="cuda")
        self.kvc.gqa_attn_prefill(self.g, seq, layer, pos, q_dev, n_head, hd, scale, out)
        got = host(out)
        idx = np.arange(nt) if sample is None else np.asarray(sample)
        st, want = self.o.attn_prefill(seq, layer, np.asarray(pos)[idx], q_host[idx], n_head, hd,
                                       scale)
        assert st == 0
        return got[idx], want

    def decode(self, layer, seq_ids, pos, q_dev, q_host, n_head, hd, scale):
        import torch
        n = len(pos)
        out = torch.empty((n, n_head, self.hd_kv), dtype=torch.float32, device="cuda")
        self.kvc.gqa_attn_decode(self.g, layer, seq_ids, pos, q_dev, n_head, hd, scale, out)
        got = host(out)
        st, want = self.o.attn_decode(layer, seq_ids, pos, q_host, n_head, hd, scale)
        assert st == 0
        return got, want

    def decode_runs(self, layer, seq_ids, runs, q_dev, q_host, n_head, hd, scale):
        """Explicit-window decode on both; returns (gpu out, oracle out)."""
        import torch
        n = len(seq_ids)
        out = torch.empty((n, n_head, self.hd_kv), dtype=torch.float32, device="cuda")
        self.kvc.gqa_attn_decode_runs(self.g, layer, seq_ids, runs, q_dev, n_head, hd, scale, out)
        got = host(out)
        st, want = self.o.attn_decode_runs(layer, seq_ids, runs, q_host, n_head, hd, scale)
        assert st == 0, st
        return got, want

    def qkv(self, layer, seq_ids, pos, x, ws, n_head, hd, base=1e6, fscale=1.0, style=0):
        """Fused projection + RoPE + store on both; ws = (wq, bq, wk, bk, wv, bv) numpy
        (biases may be None).  Returns (gpu rotated q, oracle rotated q)."""
        import torch
        nt = len(pos)
        q_out = torch.empty((nt, n_head, hd), dtype=torch.float32, device="cuda")
        dws = [None if a is None else dev(a) for a in ws]
        self.kvc.kv_qkv_rope_append(self.g, layer, seq_ids, pos, dev(x), *dws, n_head, hd, q_out,
                                    base, fscale, style)
        st, qo = self.o.qkv_rope_append(layer, seq_ids, pos, x, *ws, n_head, hd, base, fscale,
                                        style)
        assert st == 0, st
        return host(q_out), qo
