"""The C ABI on the CPU: the library loads and exports every symbol include/kvc.h declares,
the header's enums match the binding, and every host-side argument check returns the
status the oracle's own checks return (no GPU, no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_causal_amd as kvc
from oracle import OracleCache
from tests.workloads import custom

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")
HOSTCHECK = os.path.join(ROOT, "kv_cache_causal_amd", "lib", "libkvc_hostcheck.so")

pytestmark = pytest.mark.skipif(not os.path.exists(kvc.LIB_PATH),
                                reason="libkvc.so not built (run __graft_entry__.build())")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert header_functions() == sorted(kvc.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(kvc.LIB_PATH)
    for name in header_functions():
        assert hasattr(L, name), name


def test_header_enum_values_match_binding():
    text = open(HEADER).read()
    for name, val in [("KVC_OK", kvc.OK), ("KVC_E_ARG", kvc.E_ARG),
                      ("KVC_E_GEOMETRY", kvc.E_GEOMETRY), ("KVC_E_RANGE", kvc.E_RANGE),
                      ("KVC_E_DUP", kvc.E_DUP), ("KVC_E_NOMEM", kvc.E_NOMEM),
                      ("KVC_E_HIP", kvc.E_HIP), ("KVC_ROPE_NEOX", kvc.ROPE_NEOX),
                      ("KVC_ROPE_INTERLEAVED", kvc.ROPE_INTERLEAVED),
                      ("KVC_ROPE_NONE", kvc.ROPE_NONE)]:
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == val, name


def test_header_fixed_scratch_size_matches_binding():
    m = re.search(r"#define KVC_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == kvc.STATIC_SCRATCH_BYTES


def test_null_handle_is_rejected_without_device_work():
    L = kvc.lib()
    pos = (ctypes.c_int32 * 1)(0)
    st = L.kv_append_rope(None, 0, 1, pos, pos, None, 1, 16, 16, 16, 1e6, 1.0, 0, None)
    assert st == kvc.E_ARG and "NULL" in kvc.kv_last_error()
    assert L.gqa_attn_decode(None, 0, 1, pos, pos, 16, 1, 16, 0.25, 16, None) == kvc.E_ARG
    assert L.gqa_attn_prefill(None, 0, 0, 1, pos, 16, 1, 16, 0.25, 16, None) == kvc.E_ARG
    assert L.gqa_attn_decode_noalloc(None, 0, 1, pos, pos, 16, 1, 16, 0.25, 16, None) == kvc.E_ARG
    assert L.kv_free(None) == kvc.OK
    out = ctypes.c_void_p()
    assert L.kv_alloc(ctypes.byref(out), 1, 1, 1, 24, 8, None) == kvc.E_ARG
    assert out.value is None and "unsupported" in kvc.kv_last_error()
    # Region formats are checked before any device call too.
    assert L.kv_alloc_typed(ctypes.byref(out), 1, 1, 2, 16, 8, kvc.KV_Q8_0, None) == kvc.E_GEOMETRY
    assert out.value is None and "Q8_0" in kvc.kv_last_error()
    assert L.kv_alloc_typed(ctypes.byref(out), 1, 1, 2, 32, 8, 3, None) == kvc.E_ARG
    assert out.value is None and "format" in kvc.kv_last_error()


# ---- validation parity with the oracle (library checks via the host-only shim) ----

@pytest.fixture(scope="module")
def hc():
    if not os.path.exists(HOSTCHECK):
        pytest.skip("host-check shim not built")
    L = ctypes.CDLL(HOSTCHECK)
    p, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    L.hc_check_alloc.argtypes = [i32] * 6
    L.hc_check_append.argtypes = [p, i32, i32, p, p, p, i32, i32, p, p, f32, f32, i32]
    L.hc_check_prefill.argtypes = [p, i32, i32, i32, p, p, i32, i32, f32, p]
    L.hc_check_decode.argtypes = [p, i32, i32, p, p, p, i32, i32, f32, p]
    L.hc_check_decode_runs.argtypes = [p, i32, i32, p, p, p, p, p, i32, i32, f32, p]
    L.hc_check_qkv.argtypes = [p, i32, i32, p, p, p, i32, p, p, p, p, p, p, i32, i32, p, f32, f32,
                               i32]
    L.hc_last_message.restype = ctypes.c_char_p
    return L


GEOM = (2, 2, 2, 16, 10)  # n_seq, n_layer, n_head_kv, hd_kv, capacity
FAKE = 0x1000             # a 16-byte-aligned stand-in for a device pointer (never touched)


def g5():
    a = np.array(GEOM, np.int32)
    return a, a.ctypes.data


def iarr(x):
    a = np.ascontiguousarray(np.asarray(x, np.int32))
    return a, a.ctypes.data


APPEND_CASES = [
    # (name, kwargs)
    ("ok", dict()),
    ("layer_range", dict(layer=2)),
    ("pos_at_capacity", dict(pos=[3, 10])),
    ("pos_negative", dict(pos=[-1, 3])),
    ("dup", dict(pos=[4, 4], seq=[1, 1])),
    ("dup_unsorted", dict(seq=[1, 0, 1], pos=[4, 2, 4])),
    ("decreasing_ok", dict(seq=[1, 1, 0], pos=[5, 3, 9])),
    ("dup_after_increasing_run", dict(seq=[0] * 6, pos=[0, 1, 2, 3, 4, 2])),
    ("range_beside_dup", dict(seq=[0, 0, 0], pos=[3, 3, 10])),
    ("seq_range", dict(seq=[0, 2])),
    ("hd_lt_hd_kv", dict(hd=8)),
    ("hd_odd", dict(hd=17)),
    ("hd_too_big", dict(hd=258)),
    ("heads_not_multiple", dict(n_head=3)),
    ("bad_style", dict(style=7)),
    ("bad_base", dict(base=0.0)),
    ("nan_scale", dict(fscale=float("nan"))),
    ("no_q_ok", dict(q=False, n_head=0, hd=0)),
    ("none_style_ignores_base", dict(style=2, base=-1.0)),
    ("nt_zero", dict(pos=[], seq=[])),
]


@pytest.mark.parametrize("name,kw", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_append_checks_match_oracle(hc, name, kw):
    seq = kw.get("seq", [0, 1])
    pos = kw.get("pos", [4, 4])
    n_head, hd = kw.get("n_head", 4), kw.get("hd", 16)
    layer, style = kw.get("layer", 1), kw.get("style", 0)
    base, fscale = kw.get("base", 1e6), kw.get("fscale", 1.0)
    has_q = kw.get("q", True)
    g, gp = g5()
    s, sp = iarr(seq)
    p, pp = iarr(pos)
    st_lib = hc.hc_check_append(gp, layer, len(pos), sp, pp, FAKE if has_q else None, n_head, hd,
                                FAKE, FAKE, base, fscale, style)
    c = OracleCache(*GEOM)
    nt = len(pos)
    q = custom(1, (nt, max(n_head, 1), max(hd, 2))) if has_q else None
    k = custom(2, (nt, 2, 16))
    st_orc, _ = c.append_rope(layer, seq, pos, q, n_head, hd, k, k, base, fscale, style)
    c.close()
    assert st_lib == st_orc, (name, st_lib, st_orc, hc.hc_last_message())


def test_append_rejects_misaligned_pointers(hc):
    g, gp = g5()
    s, sp = iarr([0])
    p, pp = iarr([1])
    assert hc.hc_check_append(gp, 0, 1, sp, pp, None, 0, 0, FAKE + 4, FAKE, 1e6, 1.0, 0) == kvc.E_ARG


PREFILL_CASES = [
    ("ok", dict()),
    ("seq_range", dict(seq=2)),
    ("layer_range", dict(layer=-1)),
    ("pos_range", dict(pos=[0, 10])),
    ("hd_lt_hd_kv", dict(hd=8)),
    ("heads", dict(n_head=5)),
    ("scale_inf", dict(scale=float("inf"))),
    ("nt_zero", dict(pos=[])),
]


@pytest.mark.parametrize("name,kw", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_checks_match_oracle(hc, name, kw):
    seq, layer = kw.get("seq", 1), kw.get("layer", 0)
    pos = kw.get("pos", [0, 9])
    n_head, hd, scale = kw.get("n_head", 4), kw.get("hd", 16), kw.get("scale", 0.25)
    g, gp = g5()
    p, pp = iarr(pos)
    st_lib = hc.hc_check_prefill(gp, seq, layer, len(pos), pp, FAKE, n_head, hd, scale, FAKE)
    c = OracleCache(*GEOM)
    st_orc, _ = c.attn_prefill(seq, layer, pos, custom(3, (len(pos), n_head, hd)), n_head, hd,
                               scale)
    c.close()
    assert st_lib == st_orc, (name, st_lib, st_orc)


DECODE_CASES = [
    ("ok", dict()),
    ("same_seq_twice_ok", dict(seq=[1, 1])),
    ("seq_range", dict(seq=[0, 9])),
    ("pos_range", dict(pos=[3, 11])),
    ("hd_lt_hd_kv", dict(hd=14)),
    ("heads", dict(n_head=0)),
    ("n_zero", dict(seq=[], pos=[])),
]


@pytest.mark.parametrize("name,kw", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_checks_match_oracle(hc, name, kw):
    seq, pos = kw.get("seq", [0, 1]), kw.get("pos", [3, 9])
    n_head, hd = kw.get("n_head", 2), kw.get("hd", 16)
    g, gp = g5()
    s, sp = iarr(seq)
    p, pp = iarr(pos)
    st_lib = hc.hc_check_decode(gp, 0, len(pos), sp, pp, FAKE, n_head, hd, 0.25, FAKE)
    c = OracleCache(*GEOM)
    st_orc, _ = c.attn_decode(0, seq, pos, custom(4, (len(pos), max(n_head, 1), hd)), n_head, hd,
                              0.25)
    c.close()
    assert st_lib == st_orc, (name, st_lib, st_orc)


def test_alloc_checks(hc):
    for dt in (kvc.KV_F32, kvc.KV_F16, kvc.KV_Q8_0):
        assert hc.hc_check_alloc(1, 1, 8, 128, 40960, dt) == kvc.OK
        for bad in [(0, 1, 1, 32, 8), (1, 0, 1, 32, 8), (1, 1, 0, 32, 8), (1, 1, 1, 24, 8),
                    (1, 1, 1, 32, 0), (1, 1, 1, 32, (1 << 24) + 1)]:
            assert hc.hc_check_alloc(*bad, dt) == kvc.E_ARG, (bad, dt)
    assert hc.hc_check_alloc(1, 1, 2, 16, 8, 3) == kvc.E_ARG
    # The oracle accepts and refuses the same formats and geometries: Q8_0 blocks must
    # lie inside one kv head (hd_kv a multiple of 32).
    from oracle import Oracle
    L = Oracle().L
    for hdk in (16, 32, 64, 80, 96, 112, 128, 160, 192, 256):
        for dt in (kvc.KV_F32, kvc.KV_F16, kvc.KV_Q8_0):
            lib_ok = hc.hc_check_alloc(1, 1, 2, hdk, 8, dt) == kvc.OK
            h = L.orc_cache_new_typed(1, 1, 2, hdk, 8, dt)
            if dt == kvc.KV_Q8_0 and hdk in (96, 160, 192):
                # The oracle's Q8_0 takes any multiple of 32; the library's kernels only
                # the power-of-two head dims (a documented limit).
                assert bool(h) and not lib_ok, hdk
                assert hc.hc_check_alloc(1, 1, 2, hdk, 8, dt) == kvc.E_GEOMETRY
            else:
                assert lib_ok == bool(h), (hdk, dt)
            if h:
                L.orc_cache_free(h)
    assert hc.hc_check_alloc(1, 1, 2, 16, 8, kvc.KV_Q8_0) == kvc.E_GEOMETRY
    # Head dims the library does not run (the oracle takes any even one up to 256).
    for hdk in (24, 48, 144, 208, 240, 250):
        assert hc.hc_check_alloc(1, 1, 2, hdk, 8, kvc.KV_F32) == kvc.E_ARG, hdk


RUNS_CASES = [
    ("ok", dict()),
    ("adjacent_runs_ok", dict(runs=[[(0, 3), (3, 2)], [(9, 1)]])),
    ("out_of_order_ok", dict(runs=[[(6, 2), (0, 3)], [(0, 10)]])),
    ("same_seq_twice_ok", dict(seq=[1, 1])),
    ("seq_range", dict(seq=[0, 2])),
    ("no_run", dict(runs=[[(0, 3)], []])),
    ("empty_run", dict(runs=[[(0, 0)], [(1, 2)]])),
    ("negative_start", dict(runs=[[(-1, 2)], [(1, 2)]])),
    ("past_capacity", dict(runs=[[(8, 3)], [(1, 2)]])),
    ("last_row_ok", dict(runs=[[(9, 1)], [(0, 10)]])),
    ("overlap", dict(runs=[[(0, 4), (3, 2)], [(1, 2)]])),
    ("same_run_twice", dict(runs=[[(2, 2), (2, 2)], [(1, 2)]])),
    ("hd_lt_hd_kv", dict(hd=14)),
    ("heads", dict(n_head=3)),
    ("n_zero", dict(seq=[], runs=[])),
]


@pytest.mark.parametrize("name,kw", RUNS_CASES, ids=[c[0] for c in RUNS_CASES])
def test_decode_runs_checks_match_oracle(hc, name, kw):
    from oracle import runs_csr
    seq = kw.get("seq", [0, 1])
    runs = kw.get("runs", [[(0, 4), (6, 2)], [(2, 5)]])
    n_head, hd = kw.get("n_head", 2), kw.get("hd", 16)
    g, gp = g5()
    s, sp = iarr(seq)
    off, starts, lens = runs_csr(runs)
    o, op = iarr(off)
    st_, stp = iarr(starts if starts.size else [0])
    ln, lnp = iarr(lens if lens.size else [0])
    st_lib = hc.hc_check_decode_runs(gp, 0, len(seq), sp, op, stp, lnp, FAKE, n_head, hd, 0.25,
                                     FAKE)
    c = OracleCache(*GEOM)
    st_orc, _ = c.attn_decode_runs(0, seq, runs, custom(5, (len(seq), max(n_head, 1), hd)),
                                   n_head, hd, 0.25)
    c.close()
    assert st_lib == st_orc, (name, st_lib, st_orc, hc.hc_last_message())


QKV_CASES = [
    ("ok", dict()),
    ("no_bias_ok", dict(bias=False)),
    ("dup", dict(pos=[3, 3], seq=[1, 1])),
    ("pos_range", dict(pos=[3, 10])),
    ("seq_range", dict(seq=[0, 2])),
    ("hd_lt_hd_kv", dict(hd=8)),
    ("heads", dict(n_head=3)),
    ("hd_odd", dict(hd=17)),
    ("style", dict(style=7)),
    ("base", dict(base=0.0)),
    ("base_ignored_for_none", dict(base=0.0, style=2)),
    ("hd_lt_hd_kv_and_bad_style", dict(hd=8, style=9)),
    ("nt_zero", dict(pos=[], seq=[])),
    ("x_null", dict(x_null=True)),
]


@pytest.mark.parametrize("name,kw", QKV_CASES, ids=[c[0] for c in QKV_CASES])
def test_qkv_checks_match_oracle(hc, name, kw):
    seq, pos = kw.get("seq", [0, 1]), kw.get("pos", [3, 9])
    n_head, hd, d = kw.get("n_head", 4), kw.get("hd", 16), 8
    style, base = kw.get("style", 0), kw.get("base", 1e4)
    nkt = GEOM[2] * GEOM[3]
    g, gp = g5()
    s_, sp = iarr(seq)
    p_, pp = iarr(pos)
    bias = FAKE if kw.get("bias", True) else None
    xp = None if kw.get("x_null") else FAKE
    st_lib = hc.hc_check_qkv(gp, 0, len(pos), sp, pp, xp, d, FAKE, bias, FAKE, bias, FAKE, bias,
                             n_head, hd, FAKE, base, 1.0, style)
    c = OracleCache(*GEOM)
    nt = len(pos)
    rng = np.random.default_rng(6)
    x = None if kw.get("x_null") else rng.standard_normal((max(nt, 1), d)).astype(np.float32)
    wq = rng.standard_normal((max(n_head * hd, 1), d)).astype(np.float32)
    wkv = rng.standard_normal((nkt, d)).astype(np.float32)
    bq = rng.standard_normal(max(n_head * hd, 1)).astype(np.float32) if bias else None
    bkv = rng.standard_normal(nkt).astype(np.float32) if bias else None
    st_orc, _ = c.qkv_rope_append(0, seq, pos, x, wq, bq, wkv, bkv, wkv, bkv, n_head, hd, base,
                                  1.0, style)
    c.close()
    assert st_lib == st_orc, (name, st_lib, st_orc, hc.hc_last_message())


def test_qkv_library_limits(hc):
    """Limits the library adds (the oracle has none): d_model a multiple of 4, at most 64
    tokens per call."""
    g, gp = g5()
    s_, sp = iarr([0])
    p_, pp = iarr([1])
    assert hc.hc_check_qkv(gp, 0, 1, sp, pp, FAKE, 6, FAKE, None, FAKE, None, FAKE, None, 4, 16,
                           FAKE, 1e4, 1.0, 0) == kvc.E_ARG
    s_, sp = iarr(list(range(2)) * 33)
    p_, pp = iarr([i // 2 for i in range(66)])
    geom = np.array((2, 2, 2, 16, 100), np.int32)
    assert hc.hc_check_qkv(geom.ctypes.data, 0, 65, sp, pp, FAKE, 8, FAKE, None, FAKE, None,
                           FAKE, None, 4, 16, FAKE, 1e4, 1.0, 0) == kvc.E_ARG
    assert hc.hc_check_qkv(geom.ctypes.data, 0, 64, sp, pp, FAKE, 8, FAKE, None, FAKE, None,
                           FAKE, None, 4, 16, FAKE, 1e4, 1.0, 0) == kvc.OK
