"""Pins that tie the oracle to something other than itself.

Each pin takes an `oracle.Oracle` (the real one, or a deliberately broken copy built by
the mutant test) and raises AssertionError if the oracle disagrees with what the pages
and the mathematics fix: the pages' worked examples (tests/golden/), closed forms,
arbitrary-precision values (mpmath), invariants the pages state, and an f64 brute force
on tiny shapes.

Sources: "11 · Attention, vec ops, and the KV cache" (§2.1 attention, §2.3 RoPE, §2.4
GQA, §3.2.2 RoPE, §3.2.3 KV store, §3.2.4 attention, §3.2.5 softmax, §3.4 invariants)
and "IV.2: Zero-copy KV cache" (append in place, no copy of existing rows).
"""
from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np

from oracle import (E_ARG, E_DUP, E_GEOMETRY, E_RANGE, KV_F16, KV_Q8_0, OK, ROPE_INTERLEAVED,
                    ROPE_NEOX, ROPE_NONE, Oracle, OracleCache, q8_split)
from tests import bruteforce as bf
from tests.workloads import custom, custom_positions

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rn32(x: mpmath.mpf) -> np.float32:
    """Round an arbitrary-precision value to the nearest f32 (ties to even)."""
    with mpmath.workprec(24):
        y = +x
    return np.float32(float(y))


def f32bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# ------------------------------------------------------------------------------------
# RoPE
# ------------------------------------------------------------------------------------

def pin_inv_freq_correctly_rounded(o: Oracle):
    """Every frequency equals freq_scale / base^(2i/hd) computed to 60 digits, then
    rounded once to f32 (the reading of the pages' powf that no libm changes)."""
    mpmath.mp.dps = 60
    for hd in (4, 16, 64, 128, 256):
        for base in (1.0e4, 1.0e6, 5.0e5):
            for fs in (1.0, 0.25):
                got = o.rope_inv_freq(hd, base, fs)
                want = [rn32(mpmath.mpf(float(np.float32(fs))) /
                             mpmath.power(mpmath.mpf(float(np.float32(base))),
                                          mpmath.mpf(2 * i) / hd)) for i in range(hd // 2)]
                assert np.array_equal(f32bits(got), f32bits(want)), (hd, base, fs)


def pin_rope_worked_example(o: Oracle):
    """§3.2.2 worked example: hd = 4, base = 1e4, pos = 2.  Pair 0 turns by 2 rad;
    pair 1's speed is 1e4^(-1/2) = 0.01 by the formula (the page prints 0.1)."""
    g = golden("rope_hd4_base1e4_pos2.json")["what_the_page_states"]
    hd, base, p = g["hd"], g["freq_base"], g["pos"]
    inv = o.rope_inv_freq(hd, base, 1.0)
    assert inv[0] == np.float32(1.0)
    assert inv[1] == np.float32(0.01)
    cs, sn = o.rope_cos_sin(hd, base, 1.0, p)
    assert np.float32(p) * inv[0] == np.float32(g["pair0_angle_rad"])
    mpmath.mp.dps = 40
    assert cs[0] == rn32(mpmath.cos(2)) and sn[0] == rn32(mpmath.sin(2))
    th1 = mpmath.mpf(float(np.float32(2.0) * np.float32(0.01)))
    assert cs[1] == rn32(mpmath.cos(th1)) and sn[1] == rn32(mpmath.sin(th1))
    # Closed-form rotation of basis vectors (NEOX pairs (0,2), (1,3)).
    e0 = np.array([[[1.0, 0.0, 0.0, 0.0]]], np.float32)
    # (Values compared with ==, so a zero's sign does not matter; nonzero entries are
    # exact because one factor of every product is 0 or 1.)
    r = o.rope(e0, [p], base, 1.0, ROPE_NEOX)[0, 0]
    assert np.array_equal(r, np.array([cs[0], 0.0, sn[0], 0.0], np.float32))
    e3 = np.array([[[0.0, 0.0, 0.0, 1.0]]], np.float32)
    r = o.rope(e3, [p], base, 1.0, ROPE_NEOX)[0, 0]
    assert np.array_equal(r, np.array([0.0, -sn[1], 0.0, cs[1]], np.float32))
    # Interleaved pairs (0,1), (2,3).
    r = o.rope(e0, [p], base, 1.0, ROPE_INTERLEAVED)[0, 0]
    assert np.array_equal(r, np.array([cs[0], sn[0], 0.0, 0.0], np.float32))


def pin_cos_sin_correctly_rounded(o: Oracle):
    """cos/sin of the f32 angle, correctly rounded: sampled against mpmath at the
    long-context positions and both ends of the frequency range."""
    mpmath.mp.dps = 40
    rng = np.random.default_rng(11)
    for hd in (16, 64, 128):
        inv = o.rope_inv_freq(hd, 1.0e6, 1.0)
        ps = np.concatenate([[0, 1, 2, 511, 32767, 40959], rng.integers(0, 40960, 6)])
        for p in ps:
            cs, sn = o.rope_cos_sin(hd, 1.0e6, 1.0, int(p))
            for i in (0, 1, hd // 4, hd // 2 - 1):
                th = mpmath.mpf(float(np.float32(p) * inv[i]))
                assert cs[i] == rn32(mpmath.cos(th)), (hd, p, i)
                assert sn[i] == rn32(mpmath.sin(th)), (hd, p, i)


# Head dims and positions of every RoPE table the workloads and the GPU tests build:
# kv head dims 16, 64, 128 and query head dims above them (48, 96, 192), positions up to
# the long-context capacity 40,960 (which covers the 520, 1,023 and 12,800 of the others).
ROPE_GRID_HDS = (16, 48, 64, 96, 128, 192)
ROPE_GRID_POSITIONS = 40960


def rn32_f64_certified(y: np.ndarray, ulps: float = 8.0):
    """Round f64 approximations y of exact values to f32, and say where that is certainly
    the correctly rounded f32 of the exact value: y within `ulps` f64 ulps of it and no
    f32 rounding boundary (midpoint of two neighbouring f32) that close to y."""
    f = y.astype(np.float32)
    lo = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    fd = f.astype(np.float64)
    margin = np.minimum(y - (fd + lo) / 2, (fd + hi) / 2 - y)
    return f, margin > ulps * np.spacing(np.abs(y))


def pin_cos_sin_exhaustive_grid(o: Oracle):
    """Every cos/sin entry of every table on the workload grid (all positions below
    40,960, all pairs of head dims 16 to 192, base 1e6) is the correctly rounded f32 of
    cos/sin of the f32 angle: against numpy's f64 cos/sin where that rounding is certain
    (8 ulps of slack for the f64 functions), else against mpmath at 40 digits."""
    mpmath.mp.dps = 40
    P = np.arange(ROPE_GRID_POSITIONS, dtype=np.float32)[:, None]
    for hd in ROPE_GRID_HDS:
        inv = o.rope_inv_freq(hd, 1.0e6, 1.0)
        th = P * inv[None, :]                      # f32 products, as in the definition
        assert th.dtype == np.float32
        got_c = np.empty(th.shape, np.float32)
        got_s = np.empty(th.shape, np.float32)
        for p in range(ROPE_GRID_POSITIONS):
            got_c[p], got_s[p] = o.rope_cos_sin(hd, 1.0e6, 1.0, p)
        for name, fn, mfn, got in (("cos", np.cos, mpmath.cos, got_c),
                                   ("sin", np.sin, mpmath.sin, got_s)):
            want, sure = rn32_f64_certified(fn(th.astype(np.float64)))
            bad = sure & (f32bits(got) != f32bits(want))
            assert not bad.any(), (hd, name, np.argwhere(bad)[:4].tolist())
            for p, i in np.argwhere(~sure):
                w = rn32(mfn(mpmath.mpf(float(th[p, i]))))
                assert f32bits(got[p, i]) == f32bits(w), (hd, name, int(p), int(i))


def pin_cos_sin_mpmath_sample(o: Oracle):
    """10,000 seeded (position, pair) entries of the grid's tables against mpmath
    correct rounding (an arbitrary-precision check of the same entries)."""
    mpmath.mp.dps = 40
    rng = np.random.default_rng(12)
    for hd in ROPE_GRID_HDS:
        inv = o.rope_inv_freq(hd, 1.0e6, 1.0)
        n = 10000 // len(ROPE_GRID_HDS) + 1
        for p, i in zip(rng.integers(0, ROPE_GRID_POSITIONS, n), rng.integers(0, hd // 2, n)):
            cs, sn = o.rope_cos_sin(hd, 1.0e6, 1.0, int(p))
            th = mpmath.mpf(float(np.float32(p) * inv[i]))
            assert cs[i] == rn32(mpmath.cos(th)) and sn[i] == rn32(mpmath.sin(th)), (hd, p, i)


def pin_rope_near_ties(o: Oracle):
    """At angles and speeds whose exact cos, sin or speed lies within about 2^-53 of the
    midpoint of two f32 values (tests/golden/rope_near_ties.json, found by a seeded
    search), the oracle still gives the correctly rounded f32 (mpmath at 60 digits).
    An angle is read through pair 0 at position 1 (speed freq_scale, so the angle is
    freq_scale itself); a speed fs / base^(1/2) through pair 1 of head dim 4."""
    g = golden("rope_near_ties.json")
    with mpmath.workdps(60):
        for a in g["angles"]:
            th = np.uint32(a["theta_bits"]).view(np.float32)
            cs, sn = o.rope_cos_sin(2, 1.0e4, float(th), 1)
            t = mpmath.mpf(float(th))
            assert f32bits(cs[0]) == f32bits(rn32(mpmath.cos(t))), float(th)
            assert f32bits(sn[0]) == f32bits(rn32(mpmath.sin(t))), float(th)
        for sp in g["speeds"]:
            fs = np.uint32(sp["freq_scale_bits"]).view(np.float32)
            base = np.uint32(sp["base_bits"]).view(np.float32)
            inv = o.rope_inv_freq(4, float(base), float(fs))
            want = rn32(mpmath.mpf(float(fs)) / mpmath.sqrt(mpmath.mpf(float(base))))
            assert f32bits(inv[1]) == f32bits(want), (float(fs), float(base))


def pin_rope_pos0_identity(o: Oracle):
    """Position 0 turns every pair by 0 rad: RoPE is the identity, bit for bit, on
    N(0,1) data (which never holds a signed zero)."""
    x = custom(1, (3, 4, 64))
    for style in (ROPE_NEOX, ROPE_INTERLEAVED):
        r = o.rope(x, [0, 0, 0], 1.0e6, 1.0, style)
        assert np.array_equal(f32bits(r), f32bits(x))


def pin_rope_brute_force(o: Oracle):
    """Explicit f64 rotation matrices (their own pair lists and angles) agree with the
    oracle within a few f32 ulps, for both layouts and a spread of positions."""
    for style in (ROPE_NEOX, ROPE_INTERLEAVED):
        for hd in (4, 16, 64):
            x = custom(2 + hd, (5, 3, hd))
            pos = [0, 1, 7, 300, 4095]
            got = o.rope(x, pos, 1.0e4, 1.0, style).astype(np.float64)
            want = bf.rope_bf(x, pos, 1.0e4, 1.0, style)
            err = np.abs(got - want)
            bound = 4 * np.finfo(np.float32).eps * (np.abs(x).max() + 1e-30)
            assert err.max() <= bound, (style, hd, err.max())


def pin_rope_norm_and_relative_position(o: Oracle):
    """Rotation keeps each vector's norm, and <R(m)q, R(n)k> depends only on m - n."""
    q = custom(3, (1, 1, 64))
    k = custom(4, (1, 1, 64))
    for style in (ROPE_NEOX, ROPE_INTERLEAVED):
        r = o.rope(q, [1234], 1.0e4, 1.0, style)
        n0, n1 = np.linalg.norm(q.astype(np.float64)), np.linalg.norm(r.astype(np.float64))
        assert abs(n0 - n1) <= 1e-6 * n0
        scale = np.linalg.norm(q) * np.linalg.norm(k)
        for (m, n, d) in ((5, 2, 3), (10, 10, 7), (3, 9, 20)):
            a = float(np.dot(o.rope(q, [m], 1.0e4, 1.0, style).ravel().astype(np.float64),
                             o.rope(k, [n], 1.0e4, 1.0, style).ravel().astype(np.float64)))
            b = float(np.dot(o.rope(q, [m + d], 1.0e4, 1.0, style).ravel().astype(np.float64),
                             o.rope(k, [n + d], 1.0e4, 1.0, style).ravel().astype(np.float64)))
            assert abs(a - b) <= 1e-5 * scale, (style, m, n, d, a, b)


# ------------------------------------------------------------------------------------
# Append (KV store)
# ------------------------------------------------------------------------------------

def pin_append_rows_land_in_place(o: Oracle):
    """A store writes row t at offset pos[t] * row width of its (seq, layer) region and
    nothing else; regions never move; the high-water mark is max(pos) + 1."""
    c = OracleCache(2, 2, 2, 16, 20, o)
    nkt = 32
    k0 = c.k(1, 1).ctypes.data
    k = custom(5, (3, 2, 16))
    v = custom(6, (3, 2, 16))
    st, _ = c.append_rope(1, [1, 1, 0], [4, 9, 2], None, 0, 0, k, v, 1.0e6, 1.0, ROPE_NONE)
    assert st == OK
    assert c.k(1, 1).ctypes.data == k0
    K, V = c.k(1, 1), c.v(1, 1)
    assert np.array_equal(f32bits(K[4]), f32bits(k[0].ravel()))
    assert np.array_equal(f32bits(K[9]), f32bits(k[1].ravel()))
    assert np.array_equal(f32bits(V[9]), f32bits(v[1].ravel()))
    assert np.array_equal(f32bits(c.k(0, 1)[2]), f32bits(k[2].ravel()))
    others = [r for r in range(20) if r not in (4, 9)]
    assert not K[others].any() and not V[others].any()
    assert not c.k(0, 0).any() and not c.k(1, 0).any()
    assert c.seq_len(1, 1) == 10 and c.seq_len(0, 1) == 3 and c.seq_len(1, 0) == 0
    assert K.shape == (20, nkt)
    c.close()


def pin_append_rotates_k_not_v(o: Oracle):
    """The stored K row is k rotated at its position with the kv head dim's own
    frequencies; the stored V row is v unchanged; q comes back rotated with hd's."""
    c = OracleCache(1, 1, 2, 16, 8, o)
    q = custom(7, (2, 4, 32))       # hd = 32 > hd_kv = 16
    k = custom(8, (2, 2, 16))
    v = custom(9, (2, 2, 16))
    st, qr = c.append_rope(0, [0, 0], [3, 5], q, 4, 32, k, v, 1.0e4, 1.0, ROPE_NEOX)
    assert st == OK
    want_k = bf.rope_bf(k, [3, 5], 1.0e4, 1.0, bf.NEOX)
    want_q = bf.rope_bf(q, [3, 5], 1.0e4, 1.0, bf.NEOX)
    assert np.abs(c.k(0, 0)[[3, 5]].reshape(2, 2, 16) - want_k).max() < 1e-5
    assert np.abs(qr - want_q).max() < 1e-5
    assert np.array_equal(f32bits(c.v(0, 0)[[3, 5]]), f32bits(v.reshape(2, 32)))


def pin_append_errors_write_nothing(o: Oracle):
    """Position out of range -> error, never a clamp; duplicate (seq, pos) -> error;
    bad sequence -> error; hd < hd_kv -> geometry error.  No error writes anything."""
    c = OracleCache(2, 1, 2, 16, 10, o)
    k = custom(10, (2, 2, 16))
    v = custom(11, (2, 2, 16))
    q = custom(12, (2, 4, 16))
    cases = [
        (dict(seq=[0, 0], pos=[3, 10]), E_RANGE),
        (dict(seq=[0, 0], pos=[-1, 3]), E_RANGE),
        (dict(seq=[0, 0], pos=[4, 4]), E_DUP),
        (dict(seq=[0, 2], pos=[4, 5]), E_ARG),
        (dict(seq=[0, 1], pos=[4, 4], hd=8), E_GEOMETRY),
        (dict(seq=[0, 1], pos=[4, 4], hd=15), E_ARG),
        (dict(seq=[0, 1], pos=[4, 4], n_head=3, q=custom(13, (2, 3, 16))), E_ARG),
    ]
    for kw, want in cases:
        qq = kw.get("q", q)
        hd = kw.get("hd", 16)
        if hd != 16:
            qq = custom(14, (2, 4, hd))
        st, _ = c.append_rope(0, kw["seq"], kw["pos"], qq, kw.get("n_head", 4), hd, k, v,
                              1.0e6, 1.0, ROPE_NEOX)
        assert st == want, (kw, st, want)
        assert not c.k(0, 0).any() and not c.k(1, 0).any() and not c.v(0, 0).any()
        assert c.seq_len(0, 0) == 0 and c.seq_len(1, 0) == 0
    # Distinct sequences may share a position.
    st, _ = c.append_rope(0, [0, 1], [4, 4], q, 4, 16, k, v, 1.0e6, 1.0, ROPE_NEOX)
    assert st == OK
    c.close()


# ------------------------------------------------------------------------------------
# Attention
# ------------------------------------------------------------------------------------

def _cache_with_rows(o, K, V, n_head_kv, hd_kv, capacity):
    c = OracleCache(1, 1, n_head_kv, hd_kv, capacity, o)
    rows = len(K)
    st, _ = c.append_rope(0, [0] * rows, list(range(rows)), None, 0, 0,
                          np.asarray(K, np.float32).reshape(rows, n_head_kv, hd_kv),
                          np.asarray(V, np.float32).reshape(rows, n_head_kv, hd_kv),
                          1.0e6, 1.0, ROPE_NONE)
    assert st == OK
    return c


def pin_attn_worked_example_1(o: Oracle):
    """§3.2.4 first example: q = [1,1,0,0] at pos 1 blends v0 and v1 equally:
    out = [2, 3, 0, 0] exactly; the third (masked) slot adds nothing."""
    g = golden("attn_example1.json")
    i = g["inputs"]
    c = _cache_with_rows(o, i["k_rows"], i["v_rows"], 1, 4, i["capacity"])
    st, out = c.attn_prefill(0, 0, [i["pos"]], np.array([[i["q"]]], np.float32), 1, 4,
                             i["scale"])
    assert st == OK
    assert np.array_equal(out[0, 0], np.array(g["page_values"]["out"], np.float32))
    c.close()


def pin_attn_worked_example_2(o: Oracle):
    """§3.2.4 variation: q = [1,0,0,0] scores [0.5, 0]; weights are the closed form
    [1/(1+e^-0.5), 1/(1+e^0.5)] (the page's [0.73, 0.27] is softmax([1, 0]))."""
    g = golden("attn_example2.json")
    i = g["inputs"]
    c = _cache_with_rows(o, i["k_rows"], i["v_rows"], 1, 4, i["capacity"])
    st, out = c.attn_prefill(0, 0, [i["pos"]], np.array([[i["q"]]], np.float32), 1, 4,
                             i["scale"])
    assert st == OK
    w0 = 1.0 / (1.0 + math.exp(-0.5))
    want = [w0 * 1 + (1 - w0) * 3, w0 * 2 + (1 - w0) * 4, 0.0, 0.0]
    assert np.abs(out[0, 0] - want).max() <= 1e-6
    # The page's printed weights are those of the unscaled scores.
    assert abs(1.0 / (1.0 + math.exp(-1.0)) - 0.73) < 0.005
    c.close()


def pin_attn_worked_example_3(o: Oracle):
    """§3.2.4 decode step: append k2/v2 at pos 2, then tokens at pos 0, 1, 2 see 1, 2, 3
    rows.  Token 2's output is the closed form; token 0 returns v0 exactly."""
    g = golden("attn_example3.json")
    i = g["inputs"]
    c = _cache_with_rows(o, i["k_rows"][:2], i["v_rows"][:2], 1, 4, i["capacity"])
    a = i["append"]
    st, _ = c.append_rope(0, [0], [a["pos"]], None, 0, 0, np.array([[a["k"]]], np.float32),
                          np.array([[a["v"]]], np.float32), 1.0e6, 1.0, ROPE_NONE)
    assert st == OK and c.seq_len(0, 0) == 3
    e = math.exp(0.5)
    w0, w1 = 1 / (1 + 2 * e), e / (1 + 2 * e)
    want2 = [w0 * 1 + w1 * 3 + w1 * 5, w0 * 2 + w1 * 4, 0.0, 0.0]
    st, out = c.attn_decode(0, [0], [i["pos2"]], np.array([[i["q2"]]], np.float32), 1, 4, 0.5)
    assert st == OK
    assert np.abs(out[0, 0] - want2).max() <= 1e-6
    # Windows: token 0 sees only row 0 -> exactly v0, whatever its query.
    q3 = np.array([[[0, 1, 1, 0]], [[0, 1, 1, 0]], [[0, 1, 1, 0]]], np.float32)
    st, out = c.attn_prefill(0, 0, [0, 1, 2], q3, 1, 4, 0.5)
    assert st == OK
    assert np.array_equal(out[0, 0], np.array(i["v_rows"][0], np.float32))
    assert np.abs(out[2, 0] - want2).max() <= 1e-6
    c.close()


def pin_attn_brute_force(o: Oracle):
    """Random tiny shapes against the f64 mask-matrix brute force: GQA groups 1, 2, 3,
    hd > hd_kv, non-contiguous and repeated positions, ragged windows."""
    shapes = [
        # nt, n_head, n_head_kv, hd, hd_kv, capacity
        (5, 2, 2, 8, 8, 9),
        (7, 4, 2, 16, 16, 13),
        (6, 6, 2, 24, 16, 11),
        (4, 3, 1, 10, 6, 40),
    ]
    for si, (nt, nh, nkv, hd, hdk, cap) in enumerate(shapes):
        K = custom(100 + si, (cap, nkv * hdk))
        V = custom(200 + si, (cap, nkv * hdk))
        c = _cache_with_rows(o, K.reshape(cap, nkv, hdk), V.reshape(cap, nkv, hdk), nkv, hdk,
                             cap)
        q = custom(300 + si, (nt, nh, hd))
        pos = custom_positions(400 + si, nt, 0, cap, unique=False)
        scale = 0.37
        st, out = c.attn_prefill(0, 0, pos, q, nh, hd, scale)
        assert st == OK
        want = bf.attention_bf(q, K, V, pos, nkv, scale)
        err = np.abs(out - want)
        assert err.max() <= 1e-6 + 1e-5 * np.abs(want).max(), (si, err.max())
        st, outd = c.attn_decode(0, [0] * nt, pos, q, nh, hd, scale)
        assert st == OK and np.array_equal(f32bits(outd), f32bits(out))
        c.close()


def pin_attn_invariants(o: Oracle):
    """Weights sum to 1 (constant V rows come back unchanged); one cached row returns
    its V exactly; equal scores give the mean of V; rows past pos[t] never matter."""
    nkv, hdk, cap = 2, 16, 12
    q = custom(20, (3, 4, 16))
    K = custom(21, (cap, nkv, hdk))
    # Constant V: any convex combination returns the constant.
    Vc = np.full((cap, nkv, hdk), 0.75, np.float32)
    c = _cache_with_rows(o, K, Vc, nkv, hdk, cap)
    st, out = c.attn_prefill(0, 0, [2, 7, 11], q, 4, 16, 0.25)
    assert st == OK and np.abs(out - 0.75).max() <= 1e-6
    c.close()
    # Single row: weight exactly 1.
    V = custom(22, (cap, nkv, hdk))
    c = _cache_with_rows(o, K, V, nkv, hdk, cap)
    st, out = c.attn_prefill(0, 0, [0, 0, 0], q, 4, 16, 0.25)
    assert st == OK
    for h in range(4):
        assert np.array_equal(f32bits(out[:, h]), f32bits(np.repeat(V[0:1, h // 2], 3, 0)))
    # Causality: rewriting rows beyond every window changes nothing.
    st, before = c.attn_prefill(0, 0, [2, 5, 6], q, 4, 16, 0.25)
    k2 = custom(23, (5, nkv, hdk))
    st2, _ = c.append_rope(0, [0] * 5, [7, 8, 9, 10, 11], None, 0, 0, k2, k2, 1.0e6, 1.0,
                           ROPE_NONE)
    st3, after = c.attn_prefill(0, 0, [2, 5, 6], q, 4, 16, 0.25)
    assert st == st2 == st3 == OK and np.array_equal(f32bits(before), f32bits(after))
    c.close()
    # Equal scores (zero keys): the plain mean of the window's V rows.
    c = _cache_with_rows(o, np.zeros_like(K), V, nkv, hdk, cap)
    st, out = c.attn_prefill(0, 0, [4], q[:1], 4, 16, 0.25)
    assert st == OK
    assert np.abs(out[0, 0] - V[:5, 0].astype(np.float64).mean(0)).max() <= 1e-6
    assert np.abs(out[0, 3] - V[:5, 1].astype(np.float64).mean(0)).max() <= 1e-6
    c.close()


def pin_attn_large_scores_stable(o: Oracle):
    """Scores in the hundreds must not overflow: the max is subtracted before exp
    (§3.2.5), so the result still matches the brute force and holds no NaN/inf."""
    cap, nkv, hdk = 6, 1, 8
    K = custom(30, (cap, nkv * hdk)) * 20
    V = custom(31, (cap, nkv * hdk))
    c = _cache_with_rows(o, K.reshape(cap, 1, 8), V.reshape(cap, 1, 8), 1, 8, cap)
    q = custom(32, (2, 1, 8)) * 20
    st, out = c.attn_prefill(0, 0, [3, 5], q, 1, 8, 1.0)
    assert st == OK and np.isfinite(out).all()
    want = bf.attention_bf(q, K, V, [3, 5], 1, 1.0)
    assert np.abs(out - want).max() <= 1e-5
    c.close()


def pin_attn_thread_invariance(o: Oracle):
    """Heads never reduce against each other: 1 thread and many give the same bits."""
    cap, nkv, hdk = 64, 2, 16
    K = custom(40, (cap, nkv, hdk))
    V = custom(41, (cap, nkv, hdk))
    c = _cache_with_rows(o, K, V, nkv, hdk, cap)
    q = custom(42, (9, 6, 16))
    pos = custom_positions(43, 9, 0, cap)
    st1, a = c.attn_prefill(0, 0, pos, q, 6, 16, 0.25, nthreads=1)
    st4, b = c.attn_prefill(0, 0, pos, q, 6, 16, 0.25, nthreads=4)
    assert st1 == st4 == OK and np.array_equal(f32bits(a), f32bits(b))
    c.close()


def pin_attn_errors(o: Oracle):
    """Attention rejects hd < hd_kv, a position beyond the region, a bad sequence and a
    head count the kv heads do not divide."""
    c = OracleCache(2, 1, 2, 16, 10, o)
    q = custom(50, (1, 4, 16))
    assert c.attn_prefill(0, 0, [3], custom(51, (1, 4, 8)), 4, 8, 0.25)[0] == E_GEOMETRY
    assert c.attn_prefill(0, 0, [10], q, 4, 16, 0.25)[0] == E_RANGE
    assert c.attn_prefill(2, 0, [3], q, 4, 16, 0.25)[0] == E_ARG
    assert c.attn_prefill(0, 0, [3], custom(52, (1, 3, 16)), 3, 16, 0.25)[0] == E_ARG
    assert c.attn_decode(0, [0, 5], [1, 2], custom(53, (2, 4, 16)), 4, 16, 0.25)[0] == E_ARG
    assert c.attn_decode(0, [0, 1], [1, 10], custom(53, (2, 4, 16)), 4, 16, 0.25)[0] == E_RANGE
    c.close()


# ------------------------------------------------------------------------------------
# Half-precision cache ("11 · Attention, vec ops, and the KV cache" §2.5 and §3.3: the GPU
# backends may keep K/V in f16 to halve the bytes; arithmetic stays f32)
# ------------------------------------------------------------------------------------

def f16_edge_values():
    """f32 values at every kind of binary16 rounding boundary."""
    h = np.arange(0, 0x7c00, dtype=np.uint32)              # every finite positive half
    lo = h[:-1].astype(np.uint16).view(np.float16).astype(np.float64)
    hi = h[1:].astype(np.uint16).view(np.float16).astype(np.float64)
    mids = ((lo + hi) / 2)                                 # exact ties (representable in f32)
    sel = np.linspace(0, len(mids) - 1, 4000).astype(int)
    vals = np.concatenate([mids[sel], np.nextafter(mids[sel], 0), np.nextafter(mids[sel], 1),
                           [0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                            1.5 * 2.0 ** -24, 2.0 ** -26, 2.0 ** -14, 1e-30, 3.1e-5, 6.1e-5]])
    vals = vals.astype(np.float32)
    return np.concatenate([vals, -vals, [np.inf, -np.inf]]).astype(np.float32)


def pin_f16_round_to_nearest_even(o: Oracle):
    """f32 -> binary16 equals IEEE round-to-nearest-even (numpy's float16 conversion) on
    every tie and its neighbours, overflow, subnormals, zeros and a wide random sample."""
    x = np.concatenate([f16_edge_values(),
                        (np.random.default_rng(3).standard_normal(6000) *
                         np.repeat([1e-7, 1e-4, 1.0, 1e3, 3e4, 7e4], 1000)).astype(np.float32)])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = o.f32_to_f16(x)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])


def pin_f16_widening_exact(o: Oracle):
    """binary16 -> f32 is exact for all 63,488 finite patterns (and keeps inf)."""
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = (h & 0x7c00) != 0x7c00
    hs = np.concatenate([h[finite], np.array([0x7c00, 0xfc00], np.uint16)])
    want = hs.view(np.float16).astype(np.float32)
    got = o.f16_to_f32(hs)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def pin_f16_cache_store_and_attention(o: Oracle):
    """An f16 cache stores binary16(rot(k)) and binary16(v) (rot pinned above), and its
    attention equals the f64 brute force over the widened rows."""
    cap, nkv, hdk = 24, 2, 16
    k = custom(60, (cap, nkv, hdk)) * 3
    v = custom(61, (cap, nkv, hdk))
    c32 = OracleCache(1, 1, nkv, hdk, cap, o)
    c16 = OracleCache(1, 1, nkv, hdk, cap, o, dtype=KV_F16)
    for c in (c32, c16):
        st, _ = c.append_rope(0, [0] * cap, np.arange(cap), None, 0, 0, k, v, 1e4, 1.0, ROPE_NEOX)
        assert st == OK
    assert np.array_equal(c16.k(0, 0), c32.k(0, 0).astype(np.float16).view(np.uint16))
    assert np.array_equal(c16.v(0, 0), v.reshape(cap, -1).astype(np.float16).view(np.uint16))
    K = c16.k(0, 0).view(np.float16).astype(np.float64)
    V = c16.v(0, 0).view(np.float16).astype(np.float64)
    q = custom(62, (6, 4, 16))
    pos = [0, 5, 9, 17, 23, 23]
    st, out = c16.attn_prefill(0, 0, pos, q, 4, 16, 0.3)
    assert st == OK
    want = bf.attention_bf(q, K, V, pos, nkv, 0.3)
    assert np.abs(out - want).max() <= 1e-6 + 1e-5 * np.abs(want).max()
    st, outd = c16.attn_decode(0, [0] * 6, pos, q, 4, 16, 0.3)
    assert st == OK and np.array_equal(outd.view(np.uint32), out.view(np.uint32))
    c32.close()
    c16.close()


# ------------------------------------------------------------------------------------
# Q8_0 cache ("11 · Attention, vec ops, and the KV cache" §2.5 "Storage": 34 bytes per 32
# values; the block arithmetic is the reading stated in tests/golden/q8_0_blocks.json)
# ------------------------------------------------------------------------------------

def pin_q8_worked_blocks(o: Oracle):
    """Hand-derived blocks: unit and half scales, a scale that binary16 cannot hold (and
    which separates the f32-reciprocal reading from a binary16-reciprocal one), a
    subnormal scale, an all-zero block; ties go away from zero."""
    g = golden("q8_0_blocks.json")
    for blk in g["blocks"]:
        x = np.array(blk["x"], np.float32)
        scales, codes = q8_split(o.q8_quantize(x))
        assert int(scales[0]) == blk["scale_bits"], (blk["name"], hex(int(scales[0])))
        assert codes[0].tolist() == blk["codes"], (blk["name"], codes[0].tolist())
        deq = o.q8_dequantize(o.q8_quantize(x))
        for i, want in blk.get("dequantized", {}).items():
            assert deq[int(i)] == np.float32(want), (blk["name"], i, deq[int(i)], want)
        if blk["scale_bits"] in (0x3C00,):   # unit scale: values are the codes
            assert np.array_equal(deq, np.array(blk["codes"], np.float32))


def pin_q8_block_invariants(o: Oracle):
    """On seeded blocks of many magnitudes: the largest-magnitude value gets code +-127
    with its sign; codes stay in [-127, 127]; negating the block negates the codes and
    keeps the scale; scaling by 2^k keeps the codes and moves the scale's exponent by k;
    blocks of a row are quantized independently; the stored scale is the binary16
    nearest to max|x| / 127 (checked in f64 against numpy's binary16); the dequantization
    error is within d/2 plus the scale's own rounding."""
    x = custom(70, (64, 32)) * np.float32(3)
    x *= np.float32(2.0) ** np.repeat(np.arange(-6, 10, dtype=np.float32), 4)[:, None]
    b = o.q8_quantize(x.ravel())
    scales, codes = q8_split(b)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    for r in range(x.shape[0]):
        i = int(np.argmax(np.abs(x[r])))
        assert codes[r, i] == (127 if x[r, i] > 0 else -127), (r, codes[r, i])
        one_s, one_c = q8_split(o.q8_quantize(x[r]))
        assert one_s[0] == scales[r] and np.array_equal(one_c[0], codes[r])
        amax = np.abs(x[r].astype(np.float64)).max()
        d16 = np.float64(scales[r:r + 1].view(np.float16)[0])
        # d/2^11 bounds binary16 rounding of a normal scale; the exact quotient sits
        # within an f32 rounding of the f32 d.
        assert abs(d16 - amax / 127) <= (amax / 127) * (2.0 ** -11 + 2.0 ** -23), r
        deq = o.q8_dequantize(b[r:r + 1]).astype(np.float64)
        bound = (amax / 127) * (0.5 + 2.0 ** -16) + 127 * abs(d16 - amax / 127)
        assert np.abs(deq - x[r]).max() <= bound, r
    neg_s, neg_c = q8_split(o.q8_quantize(-x.ravel()))
    assert np.array_equal(neg_s, scales) and np.array_equal(neg_c, -codes)
    y = x[16:48]   # scales well inside the binary16 normal range
    ys, yc = q8_split(o.q8_quantize(y.ravel()))
    ys2, yc2 = q8_split(o.q8_quantize((y * np.float32(8)).ravel()))
    assert np.array_equal(yc2, yc)
    assert np.array_equal(ys2.view(np.float16).astype(np.float64),
                          ys.view(np.float16).astype(np.float64) * 8)


def pin_q8_cache_store_and_attention(o: Oracle):
    """A Q8_0 cache stores the blocks of rot(k) and of v at each row (rot pinned above,
    blocks pinned by the two pins before), and its attention is the f32 attention of
    the dequantized rows (values built here from the stored bytes with numpy's
    binary16), so it equals the f64 brute force within the f32 bar.  hd_kv must be a
    multiple of 32."""
    cap, nkv, hdk = 20, 2, 32
    k = custom(63, (cap, nkv, hdk)) * 3
    v = custom(64, (cap, nkv, hdk))
    c32 = OracleCache(1, 1, nkv, hdk, cap, o)
    cq = OracleCache(1, 1, nkv, hdk, cap, o, dtype=KV_Q8_0)
    for c in (c32, cq):
        st, _ = c.append_rope(0, [0] * cap, np.arange(cap), None, 0, 0, k, v, 1e4, 1.0, ROPE_NEOX)
        assert st == OK
    for which, src in ((0, c32.k(0, 0)), (1, v.reshape(cap, -1))):
        reg = cq.region(which, 0, 0)
        for r in range(cap):
            assert np.array_equal(reg[r].ravel(), o.q8_quantize(src[r]).ravel()), (which, r)
    deq = []
    for which in (0, 1):
        sc, cd = q8_split(cq.region(which, 0, 0))
        deq.append((sc.view(np.float16).astype(np.float32)[..., None] *
                    cd.astype(np.float32)).reshape(cap, nkv * hdk))
    cd32 = OracleCache(1, 1, nkv, hdk, cap, o)
    st, _ = cd32.append_rope(0, [0] * cap, np.arange(cap), None, 0, 0, deq[0], deq[1], 0, 0,
                             ROPE_NONE)
    assert st == OK
    q = custom(65, (5, 4, 32))
    pos = [0, 3, 11, 19, 19]
    st, out = cq.attn_prefill(0, 0, pos, q, 4, 32, 0.2)
    st2, want32 = cd32.attn_prefill(0, 0, pos, q, 4, 32, 0.2)
    assert st == OK and st2 == OK
    assert np.array_equal(out.view(np.uint32), want32.view(np.uint32))
    want = bf.attention_bf(q, deq[0].astype(np.float64), deq[1].astype(np.float64), pos, nkv, 0.2)
    assert np.abs(out - want).max() <= 1e-6 + 1e-5 * np.abs(want).max()
    st, outd = cq.attn_decode(0, [0] * 5, pos, q, 4, 32, 0.2)
    assert st == OK and np.array_equal(outd.view(np.uint32), out.view(np.uint32))
    for c in (c32, cq, cd32):
        c.close()
    try:
        OracleCache(1, 1, 2, 16, 8, o, dtype=KV_Q8_0)
    except ValueError:
        pass
    else:
        raise AssertionError("a Q8_0 cache with hd_kv = 16 was accepted")


# ------------------------------------------------------------------------------------
# Explicit windows ("13 · The decode loop and graph reuse" §2.2 Budget 3: a query's
# allowed cells are an input, a list of runs; §3.4 item 4: stale cells past a
# rolled-back cursor are never read)
# ------------------------------------------------------------------------------------

def _runs_cache(o, seed, n_seq=2, cap=48, nkv=2, hdk=16):
    c = OracleCache(n_seq, 1, nkv, hdk, cap, o)
    for s in range(n_seq):
        k = custom(seed + s, (cap, nkv, hdk)) * 2
        v = custom(seed + 10 + s, (cap, nkv, hdk))
        st, _ = c.append_rope(0, [s] * cap, np.arange(cap), None, 0, 0, k, v, 1e4, 1.0, ROPE_NEOX)
        assert st == OK
    return c


def pin_runs_single_run_is_the_causal_window(o: Oracle):
    """A window of one run [0, pos] (or of consecutive runs covering it in order) is the
    position-derived window: bit-identical to the pinned decode."""
    c = _runs_cache(o, 100)
    q = custom(102, (5, 4, 16))
    seqs, pos = [0, 1, 0, 1, 0], [0, 7, 31, 47, 20]
    st, want = c.attn_decode(0, seqs, pos, q, 4, 16, 0.3)
    assert st == OK
    st, got = c.attn_decode_runs(0, seqs, [[(0, p + 1)] for p in pos], q, 4, 16, 0.3)
    assert st == OK and np.array_equal(got.view(np.uint32), want.view(np.uint32))
    split = [[(0, 1)], [(0, 3), (3, 5)], [(0, 10), (10, 1), (11, 21)], [(0, 47), (47, 1)],
             [(0, 20), (20, 1)]]
    st, got = c.attn_decode_runs(0, seqs, split, q, 4, 16, 0.3)
    assert st == OK and np.array_equal(got.view(np.uint32), want.view(np.uint32))
    c.close()


def pin_runs_brute_force(o: Oracle):
    """Scattered, out-of-order runs against an f64 brute force whose mask is built from
    the runs (cell j is allowed iff some run holds it), GQA groups of 2."""
    c = _runs_cache(o, 110)
    q = custom(112, (4, 4, 16))
    runs = [[(40, 8), (3, 5), (20, 1)], [(0, 48)], [(47, 1)], [(10, 10), (0, 2), (30, 6)]]
    seqs = [1, 0, 0, 1]
    st, got = c.attn_decode_runs(0, seqs, runs, q, 4, 16, 0.27)
    assert st == OK
    for b in range(4):
        allowed = np.zeros(48, bool)
        for s0, ln in runs[b]:
            allowed[s0:s0 + ln] = True
        K = c.k(seqs[b], 0).astype(np.float64)[allowed]
        V = c.v(seqs[b], 0).astype(np.float64)[allowed]
        want = bf.attention_bf(q[b:b + 1], K, V, [K.shape[0] - 1], 2, 0.27)
        assert np.abs(got[b] - want[0]).max() <= 1e-6 + 1e-5 * np.abs(want).max(), b
    # Run order changes only the summation order.
    st, rev = c.attn_decode_runs(0, seqs, [r[::-1] for r in runs], q, 4, 16, 0.27)
    assert st == OK and np.abs(rev - got).max() <= 1e-6
    c.close()


def pin_runs_stale_cells_and_shared_region(o: Oracle):
    """Cells outside a window are never read (rewriting them changes nothing, bit for
    bit), and rows stored at any cells of a region -- e.g. a second sequence's rows after
    the first's -- attend exactly as the same rows at the start of a region of their own."""
    c = _runs_cache(o, 120, n_seq=1)
    q = custom(122, (2, 4, 16))
    runs = [[(0, 20)], [(24, 10)]]
    st, before = c.attn_decode_runs(0, [0, 0], runs, q, 4, 16, 0.3)
    assert st == OK
    junk = np.full((4, 2, 16), 1e30, np.float32)
    st, _ = c.append_rope(0, [0] * 4, [20, 21, 22, 23], None, 0, 0, junk, junk, 0, 0, ROPE_NONE)
    assert st == OK
    st, after = c.attn_decode_runs(0, [0, 0], runs, q, 4, 16, 0.3)
    assert st == OK and np.array_equal(after.view(np.uint32), before.view(np.uint32))
    alone = OracleCache(1, 1, 2, 16, 10, o)
    rows = c.k(0, 0)[24:34].reshape(10, 2, 16), c.v(0, 0)[24:34].reshape(10, 2, 16)
    st, _ = alone.append_rope(0, [0] * 10, np.arange(10), None, 0, 0, rows[0], rows[1], 0, 0,
                              ROPE_NONE)
    assert st == OK
    st, want = alone.attn_decode(0, [0], [9], q[1:], 4, 16, 0.3)
    assert st == OK and np.array_equal(after[1:].view(np.uint32), want.view(np.uint32))
    alone.close()
    c.close()


def pin_runs_errors(o: Oracle):
    """Malformed windows are refused before anything is computed."""
    c = _runs_cache(o, 130)
    q = custom(131, (2, 4, 16))
    L = c.L

    def call(off, starts, lens, seqs=(0, 1)):
        seqs = np.asarray(seqs, np.int32)
        off, starts, lens = (np.asarray(a, np.int32) for a in (off, starts, lens))
        out = np.zeros((len(seqs), 4, 16), np.float32)
        return L.orc_attn_decode_runs(c.h, 0, len(seqs), seqs.ctypes.data, off.ctypes.data,
                                      starts.ctypes.data, lens.ctypes.data,
                                      np.ascontiguousarray(q[:len(seqs)]).ctypes.data, 4, 16,
                                      0.3, out.ctypes.data, 0)

    assert call([0, 1, 2], [0, 5], [3, 4]) == OK
    assert call([0, 1, 3], [0, 5, 9], [3, 4, 1]) == OK          # adjacent runs
    assert call([1, 2, 3], [0, 5, 0], [3, 4, 1]) == E_ARG       # offsets must start at 0
    assert call([0, 1, 1], [0], [3]) == E_ARG                   # a query with no run
    assert call([0, 1, 2], [0, 5], [3, 0]) == E_ARG             # empty run
    assert call([0, 1, 2], [0, -1], [3, 2]) == E_RANGE          # before the region
    # Past the capacity (48); on sequence 0, so that a broken check reads only memory of
    # the next region.
    assert call([0, 1, 2], [0, 40], [3, 9], seqs=(1, 0)) == E_RANGE
    assert call([0, 1, 2], [0, 47], [3, 1]) == OK               # the last cell
    assert call([0, 2, 3], [0, 2, 7], [3, 4, 1]) == E_DUP       # overlapping runs
    assert call([0, 2, 3], [6, 6, 7], [1, 1, 1]) == E_DUP       # the same cell twice
    assert call([0, 1, 2], [0, 5], [3, 4], seqs=(0, 2)) == E_ARG
    c.close()


# ------------------------------------------------------------------------------------
# Fused decode projections ("13 · The decode loop and graph reuse" §2.3: q/k/v matmuls,
# biases, two RoPEs and two KV stores as one operation; §3.4 item 5: fused and unfused
# paths bit-identical)
# ------------------------------------------------------------------------------------

def rn32_fraction(r):
    """The f32 nearest to the rational r (ties to even), by integer arithmetic."""
    from fractions import Fraction
    if r == 0:
        return np.float32(0.0)
    sign = -1 if r < 0 else 1
    a = abs(Fraction(r))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    quantum_exp = max(e - 23, -149)          # spacing of f32 values near a
    m = a / Fraction(2) ** quantum_exp
    q = m.numerator // m.denominator
    rem = m - q
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and q % 2 == 1):
        q += 1
    return np.float32(sign * float(Fraction(q) * Fraction(2) ** quantum_exp))


def pin_project_exact_rational(o: Oracle):
    """Each projection output is the f32 nearest to the exact rational dot product, then
    plus the bias in f32: against exact Fraction arithmetic, on rows with wide magnitude
    ranges and heavy cancellation (where any f32 or f64 running sum goes wrong)."""
    from fractions import Fraction
    rng = np.random.default_rng(140)
    nt, rows, d = 3, 6, 37
    x = (rng.standard_normal((nt, d)) * 10.0 ** rng.integers(-6, 7, (nt, d))).astype(np.float32)
    w = (rng.standard_normal((rows, d)) * 10.0 ** rng.integers(-6, 7, (rows, d))).astype(np.float32)
    x[0, :4] = [1e20, 1.0, -1e20, 0.5]     # row 0 of w below: exact result 1.5 (an f64
    #                                          running sum loses the 1 next to 1e20)
    w[0, :] = 0.0
    w[0, :4] = 1.0
    w[1] = -w[2] * np.float32(1.0)          # rows 1 and 2 cancel term by term
    b = rng.standard_normal(rows).astype(np.float32)
    got = o.project(x, w)
    gotb = o.project(x, w, b)
    for t in range(nt):
        for j in range(rows):
            exact = sum(Fraction(float(x[t, i])) * Fraction(float(w[j, i])) for i in range(d))
            want = rn32_fraction(exact)
            assert got[t, j].view(np.uint32) == want.view(np.uint32), (t, j, got[t, j], want)
            assert gotb[t, j].view(np.uint32) == (want + b[j]).view(np.uint32), (t, j)
    assert got[0, 0] == 1.5
    assert np.array_equal(got[:, 1], -got[:, 2])


def pin_fused_equals_unfused(o: Oracle):
    """The fused step's rotated q, cache rows and high-water marks are those of the
    projections (pinned above) followed by the pinned append, bit for bit, with and
    without biases, in the three RoPE styles and the three region formats."""
    from oracle import KV_F16 as F16, KV_Q8_0 as Q8
    rng = np.random.default_rng(150)
    d, nh, nkv, hd, hdk, cap = 96, 4, 2, 32, 32, 16
    for style in (ROPE_NEOX, ROPE_INTERLEAVED, ROPE_NONE):
        for dt in (0, F16, Q8):
            for with_bias in (True, False):
                x = rng.standard_normal((3, d)).astype(np.float32)
                wq, wk, wv = (rng.standard_normal((r, d)).astype(np.float32) * np.float32(0.1)
                              for r in (nh * hd, nkv * hdk, nkv * hdk))
                bq, bk, bv = ((rng.standard_normal(r).astype(np.float32) if with_bias else None)
                              for r in (nh * hd, nkv * hdk, nkv * hdk))
                seqs, pos = [0, 1, 0], [3, 3, 15]
                fused = OracleCache(2, 1, nkv, hdk, cap, o, dtype=dt)
                st, qf = fused.qkv_rope_append(0, seqs, pos, x, wq, bq, wk, bk, wv, bv, nh, hd,
                                               1e4, 1.0, style)
                assert st == OK
                plain = OracleCache(2, 1, nkv, hdk, cap, o, dtype=dt)
                q = o.project(x, wq, bq).reshape(3, nh, hd)
                k = o.project(x, wk, bk).reshape(3, nkv, hdk)
                v = o.project(x, wv, bv).reshape(3, nkv, hdk)
                st, qp = plain.append_rope(0, seqs, pos, q, nh, hd, k, v, 1e4, 1.0, style)
                assert st == OK
                assert np.array_equal(qf.view(np.uint32), qp.view(np.uint32))
                for s_ in (0, 1):
                    assert np.array_equal(fused.k(s_, 0), plain.k(s_, 0))
                    assert np.array_equal(fused.v(s_, 0), plain.v(s_, 0))
                    assert fused.seq_len(s_, 0) == plain.seq_len(s_, 0)
                fused.close()
                plain.close()
    # Errors come from the same checks as the append: nothing is written.  (Two sequences:
    # a broken range check then writes into the second region, not past the allocation.)
    c = OracleCache(2, 1, nkv, hdk, cap, o)
    x = rng.standard_normal((2, d)).astype(np.float32)
    w = rng.standard_normal((nh * hd, d)).astype(np.float32)
    wkv = rng.standard_normal((nkv * hdk, d)).astype(np.float32)
    st, _ = c.qkv_rope_append(0, [0, 0], [1, 1], x, w, None, wkv, None, wkv, None, nh, hd, 1e4)
    assert st == E_DUP and not c.k(0, 0).any() and c.seq_len(0, 0) == 0
    st, _ = c.qkv_rope_append(0, [0, 0], [1, 16], x, w, None, wkv, None, wkv, None, nh, hd, 1e4)
    assert st == E_RANGE and not c.k(0, 0).any()
    c.close()


# Pins too slow to repeat for each planted mistake of the mutant test (seconds each):
# run once by tests/test_oracle_pins.py.  The mutants they would catch are caught by the
# sampled pins above as well.
SWEEP_PINS = [
    pin_cos_sin_exhaustive_grid,
    pin_cos_sin_mpmath_sample,
]

ALL_PINS = [
    pin_inv_freq_correctly_rounded,
    pin_rope_worked_example,
    pin_cos_sin_correctly_rounded,
    pin_rope_near_ties,
    pin_rope_pos0_identity,
    pin_rope_brute_force,
    pin_rope_norm_and_relative_position,
    pin_append_rows_land_in_place,
    pin_append_rotates_k_not_v,
    pin_append_errors_write_nothing,
    pin_attn_worked_example_1,
    pin_attn_worked_example_2,
    pin_attn_worked_example_3,
    pin_attn_brute_force,
    pin_attn_invariants,
    pin_attn_large_scores_stable,
    pin_attn_thread_invariance,
    pin_attn_errors,
    pin_f16_round_to_nearest_even,
    pin_f16_widening_exact,
    pin_f16_cache_store_and_attention,
    pin_q8_worked_blocks,
    pin_q8_block_invariants,
    pin_q8_cache_store_and_attention,
    pin_runs_single_run_is_the_causal_window,
    pin_runs_brute_force,
    pin_runs_stale_cells_and_shared_region,
    pin_runs_errors,
    pin_project_exact_rational,
    pin_fused_equals_unfused,
]
