"""GPU edge cases through the C ABI: every supported kv head dim, GQA group sizes that
leave idle waves or need several passes, hd > hd_kv, single-row windows, positions out of
order / repeated / at the end of the region, ragged tiles, the three RoPE styles, errors
that must leave the cache untouched, and the no-copy/no-move contract."""
import numpy as np
import pytest

import kv_cache_causal_amd as kvc
from tests.gpu_util import Pair, assert_bitwise, assert_close, compare_cache, dev, host, say
from tests.workloads import custom, custom_positions

pytestmark = pytest.mark.gpu


def build(seed, n_seq, n_head, n_head_kv, hd, hd_kv, capacity, rows, style=0, base=1e6, kv=0):
    """A cache pair with rows [0, rows) of sequence 0 (and 1 if present) written."""
    p = Pair(n_seq, 1, n_head_kv, hd_kv, capacity, dtype=kv)
    for s in range(n_seq):
        k = custom(seed * 10 + s, (rows, n_head_kv, hd_kv))
        v = custom(seed * 10 + 5 + s, (rows, n_head_kv, hd_kv))
        p.append(0, [s] * rows, np.arange(rows), None, n_head, hd, k, v, base, 1.0, style)
    return p


HEADS = [
    # n_head, n_head_kv, hd, hd_kv
    (2, 2, 16, 16),
    (4, 1, 32, 32),
    (6, 2, 64, 64),     # G = 3: one idle wave / lane of heads
    (14, 2, 64, 64),    # G = 7
    (16, 8, 128, 128),  # G = 2
    (16, 1, 128, 128),  # G = 16: two decode passes, four prefill head subsets
    (8, 4, 256, 256),
    (4, 2, 48, 32),     # hd > hd_kv
    (4, 2, 160, 128),   # hd > hd_kv, not a multiple of 4 only in the tail
]


FORMATS = pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])


def v_row(pair, kv, seq, row):
    """Row `row` of the oracle's V region as f32 values (widened or dequantized)."""
    v = pair.o.v(seq, 0)[row]
    if kv == 1:
        return v.view(np.float16).astype(np.float32)
    if kv == 2:
        from oracle import q8_split
        sc, cd = q8_split(v)
        return (sc.view(np.float16).astype(np.float32)[:, None] * cd.astype(np.float32)).ravel()
    return v


@FORMATS
@pytest.mark.parametrize("nh,nkv,hd,hdk", HEADS, ids=[f"h{a}kv{b}d{c}dk{d}" for a, b, c, d in HEADS])
def test_decode_and_prefill_shapes(nh, nkv, hd, hdk, kv):
    if kv == 2 and hdk % 32:
        pytest.skip("Q8_0 needs hd_kv a multiple of 32")
    say(f"shape n_head={nh} n_head_kv={nkv} hd={hd} hd_kv={hdk} kv={kv}")
    cap, rows = 300, 300
    p = build(1, 2, nh, nkv, hd, hdk, cap, rows, kv=kv)
    # Decode: two sequences, long and short windows, one at the last row.
    q = custom(2, (3, nh, hd))
    seqs, pos = [0, 1, 0], [299, 0, 137]
    got, want = p.decode(0, seqs, pos, dev(q), q, nh, hd, 0.31)
    assert_close(got, want, "decode")
    # A one-row window returns that V row exactly (widened from binary16 or dequantized
    # from Q8_0 if stored so).
    v0 = v_row(p, kv, 1, 0)
    for h in range(nh):
        assert_bitwise(got[1, h], v0[(h // (nh // nkv)) * hdk:][:hdk], "pos 0 = v0")
    # Prefill: 77 tokens (ragged tile), positions out of order with repeats.
    nt = 77
    q = custom(3, (nt, nh, hd))
    pos = custom_positions(4, nt, 0, rows, unique=False)
    got, want = p.prefill(0, 0, pos, dev(q), q, nh, hd, 0.29)
    assert_close(got, want, "prefill")
    p.close()


@FORMATS
@pytest.mark.parametrize("style", [0, 1, 2], ids=["neox", "interleaved", "none"])
def test_rope_styles_and_hd_gt_hd_kv(style, kv):
    say(f"rope style {style} kv={kv}")
    p = Pair(2, 3, 2, 32, 64, dtype=kv)
    nt = 40
    q = custom(10, (nt, 4, 48))
    k = custom(11, (nt, 2, 32))
    v = custom(12, (nt, 2, 32))
    seqs = np.array([0, 1] * (nt // 2), np.int32)
    pos = np.concatenate([custom_positions(13, nt // 2, 0, 64), custom_positions(14, nt // 2, 0, 64)])
    pos = pos.reshape(2, -1).T.reshape(-1)   # interleave the two sequences' positions
    qd, qo = p.append(1, seqs, pos, q, 4, 48, k, v, 5e5, 0.5, style)
    for s in range(2):
        for layer in range(3):
            compare_cache(p.g, p.o, s, layer, f"style {style}")
    p.close()


def test_positions_to_the_last_row_and_tiles_past_capacity():
    say("capacity 100 (not a tile multiple), tokens at 98/99")
    p = build(20, 1, 4, 2, 64, 64, 100, 100)
    q = custom(21, (5, 4, 64))
    pos = [99, 98, 0, 64, 63]
    got, want = p.prefill(0, 0, pos, dev(q), q, 4, 64, 0.125)
    assert_close(got, want, "prefill at the region's end")
    got, want = p.decode(0, [0] * 5, pos, dev(q), q, 4, 64, 0.125)
    assert_close(got, want, "decode at the region's end")
    p.close()


def test_unwritten_rows_read_as_zero():
    """Rows inside a window that were never appended hold +0.0 and take part as zeros."""
    say("unwritten rows")
    p = Pair(1, 1, 2, 64, 256)
    k = custom(30, (10, 2, 64))
    p.append(0, [0] * 10, np.arange(0, 200, 20), None, 4, 64, k, k, 1e6, 1.0, 0)
    q = custom(31, (3, 4, 64))
    got, want = p.decode(0, [0, 0, 0], [199, 250, 5], dev(q), q, 4, 64, 0.125)
    assert_close(got, want, "decode over gaps")
    got, want = p.prefill(0, 0, [199, 250, 5], dev(q), q, 4, 64, 0.125)
    assert_close(got, want, "prefill over gaps")
    compare_cache(p.g, p.o, 0, 0, "gappy cache")
    p.close()


def test_errors_leave_everything_untouched():
    say("error paths")
    p = build(40, 2, 4, 2, 64, 64, 50, 20)
    k = custom(41, (2, 2, 64))
    q = custom(42, (2, 4, 64))
    qd = dev(q)
    kp0 = kvc.kv_view(p.g, 1, 0)
    cases = [
        (dict(seq=[0, 1], pos=[5, 50]), kvc.E_RANGE),
        (dict(seq=[1, 1], pos=[7, 7]), kvc.E_DUP),
        (dict(seq=[0, 2], pos=[1, 2]), kvc.E_ARG),
        (dict(seq=[0, 1], pos=[1, 2], hd=32), kvc.E_GEOMETRY),
    ]
    for kw, code in cases:
        hd = kw.get("hd", 64)
        qq = qd if hd == 64 else dev(custom(43, (2, 4, hd)))
        with pytest.raises(kvc.KvcError) as ei:
            kvc.kv_append_rope(p.g, 0, kw["seq"], kw["pos"], qq, 4, hd, dev(k), dev(k), 1e6)
        assert ei.value.status == code, (kw, ei.value)
    assert_bitwise(host(qd), q, "q untouched by failed appends")
    for s in range(2):
        compare_cache(p.g, p.o, s, 0, "after failed appends")
    import torch
    out = torch.full((1, 4, 64), 7.0, device="cuda")
    with pytest.raises(kvc.KvcError) as ei:
        kvc.gqa_attn_decode(p.g, 0, [0], [50], qd[:1], 4, 64, 0.125, out)
    assert ei.value.status == kvc.E_RANGE
    with pytest.raises(kvc.KvcError) as ei:
        kvc.gqa_attn_prefill(p.g, 0, 0, [3], dev(custom(44, (1, 4, 32))), 4, 32, 0.125, out)
    assert ei.value.status == kvc.E_GEOMETRY
    assert (host(out) == 7.0).all()
    # Regions never move; a later good append still works.
    assert kvc.kv_view(p.g, 1, 0) == kp0
    p.append(0, [1], [49], q[:1], 4, 64, k[:1], k[:1])
    compare_cache(p.g, p.o, 1, 0, "after recovery")
    assert kvc.kv_view(p.g, 1, 0) == kp0
    p.close()


def test_binding_refuses_short_tensors():
    """The binding checks each tensor's size against the call before the library sees
    it (a short tensor would be read or written past its end): ValueError, nothing
    written."""
    import torch
    say("binding size checks")
    p = build(45, 1, 4, 2, 64, 64, 32, 8)
    q = dev(custom(46, (2, 4, 64)))
    k = dev(custom(47, (2, 2, 64)))
    out = torch.full((2, 4, 64), 7.0, device="cuda")
    with pytest.raises(ValueError):
        kvc.kv_append_rope(p.g, 0, [0, 0], [8, 9], q, 4, 64, k[:1], k, 1e6)
    with pytest.raises(ValueError):
        kvc.kv_append_rope(p.g, 0, [0, 0], [8, 9], q[:1], 4, 64, k, k, 1e6)
    with pytest.raises(ValueError):
        kvc.gqa_attn_decode(p.g, 0, [0, 0], [3, 4], q, 4, 64, 0.125, out[:1])
    with pytest.raises(ValueError):
        kvc.gqa_attn_prefill(p.g, 0, 0, [3, 4], q[:1], 4, 64, 0.125, out)
    with pytest.raises(ValueError):
        kvc.gqa_attn_decode_runs(p.g, 0, [0, 0], [[(0, 4)], [(2, 3)]], q, 4, 64, 0.125, out[:1])
    assert (host(out) == 7.0).all()
    compare_cache(p.g, p.o, 0, 0, "after refused calls")
    p.close()


def test_empty_calls_are_noops():
    say("nt = 0")
    p = Pair(1, 1, 2, 16, 8)
    kvc.kv_append_rope(p.g, 0, [], [], None, 0, 0, None, None, 1e6)
    kvc.gqa_attn_prefill(p.g, 0, 0, [], None, 2, 16, 0.25, None)
    kvc.gqa_attn_decode(p.g, 0, [], [], None, 2, 16, 0.25, None)
    assert kvc.kv_seq_len(p.g, 0, 0) == 0
    compare_cache(p.g, p.o, 0, 0, "untouched")
    p.close()


def test_overwrite_below_high_water_and_isolation():
    """Rewriting an earlier position (a rollback) replaces exactly that row; other
    sequences and layers never change."""
    say("overwrite + isolation")
    p = Pair(3, 2, 2, 32, 40)
    for s in range(3):
        k = custom(50 + s, (30, 2, 32))
        p.append(1, [s] * 30, np.arange(30), None, 0, 0, k, k)
    k = custom(60, (3, 2, 32))
    p.append(1, [1, 1, 1], [3, 29, 10], custom(61, (3, 4, 32)), 4, 32, k, k)
    for s in range(3):
        for layer in range(2):
            compare_cache(p.g, p.o, s, layer, "overwrite")
    p.close()


def test_long_window_many_chunks_matches_single_chunk_shape():
    """A window split into many chunks (K3 merge) and a short one-chunk window."""
    say("split-K long window")
    p = build(70, 1, 16, 8, 128, 128, 9000, 9000)
    q = custom(71, (2, 16, 128))
    got, want = p.decode(0, [0, 0], [8999, 40], dev(q), q, 16, 128, 0.0883883461356163)
    assert_close(got, want, "split-K")
    p.close()


@pytest.mark.parametrize("style,hd", [(0, 20), (1, 18), (0, 40), (1, 36)],
                         ids=["neox20", "inter18", "neox40", "inter36"])
def test_rope_query_widths_scalar_and_vector_paths(style, hd):
    """Query head dims that rule out (20, 18) or allow (40, 36) whole-float4 access."""
    say(f"rope q width {hd} style {style}")
    p = Pair(1, 1, 2, 16, 96)
    nt = 70  # more than the 64 that travel in kernel arguments: positions go via memory
    q = custom(80 + hd, (nt, 4, hd))
    k = custom(81, (nt, 2, 16))
    v = custom(82, (nt, 2, 16))
    pos = custom_positions(83, nt, 0, 96)
    qd, qo = p.append(0, [0] * nt, pos, q, 4, hd, k, v, 1e4, 1.0, style)
    compare_cache(p.g, p.o, 0, 0, f"width {hd}")
    got, want = p.prefill(0, 0, pos, qd, qo, 4, hd, 0.2)
    assert_close(got, want, f"prefill width {hd}")
    p.close()


@pytest.mark.parametrize("style", [0, 2], ids=["neox", "none"])
def test_f16_store_rounding_edges(style):
    """binary16 stores of values that round to subnormals, to zero, across ties, to the
    largest finite half and to infinity: bit-identical to the oracle's rounding."""
    say(f"f16 store edges style {style}")
    p = Pair(1, 1, 2, 64, 128, dtype=1)
    rng = np.random.default_rng(90)
    scales = np.array([1e-9, 3e-8, 6e-8, 1e-6, 6.1e-5, 1.0, 2049.0, 65504.0, 65520.0, 1e5],
                      np.float32)
    k = (rng.standard_normal((100, 2, 64)) * scales[rng.integers(0, len(scales), (100, 2, 64))])
    v = (rng.standard_normal((100, 2, 64)) * scales[rng.integers(0, len(scales), (100, 2, 64))])
    k, v = k.astype(np.float32), v.astype(np.float32)
    p.append(0, [0] * 100, np.arange(100), None, 4, 64, k, v, 1e6, 1.0, style)
    compare_cache(p.g, p.o, 0, 0, "f16 edges")
    p.close()


@pytest.mark.parametrize("style", [0, 1, 2], ids=["neox", "interleaved", "none"])
def test_q8_store_edges(style):
    """Q8_0 stores bit-identical to the oracle's blocks: the hand-derived blocks (ties
    away from zero, a scale binary16 cannot hold, a subnormal scale, zero blocks) and
    random blocks spanning tiny (zero or subnormal scale) to huge (infinite scale)
    magnitudes; then attention over them."""
    import json
    import os
    say(f"q8 store edges style {style}")
    p = Pair(1, 1, 2, 64, 128, dtype=2)
    with open(os.path.join(os.path.dirname(__file__), "golden", "q8_0_blocks.json")) as f:
        blocks = [np.array(b["x"], np.float32) for b in json.load(f)["blocks"]]
    rng = np.random.default_rng(91)
    mags = np.array([1e-12, 1e-9, 1e-7, 1e-5, 1e-3, 1.0, 300.0, 1e5, 1e7], np.float32)
    k = rng.standard_normal((100, 4, 32)) * mags[rng.integers(0, len(mags), (100, 4, 1))]
    v = rng.standard_normal((100, 4, 32)) * mags[rng.integers(0, len(mags), (100, 4, 1))]
    k, v = k.astype(np.float32), v.astype(np.float32)
    for i, b in enumerate(blocks):      # rows 0..4: the worked blocks, in both regions
        k[i, :] = b
        v[i, :] = b[::-1]
    k, v = k.reshape(100, 2, 64), v.reshape(100, 2, 64)
    p.append(0, [0] * 100, np.arange(100), None, 4, 64, k, v, 1e6, 1.0, style)
    compare_cache(p.g, p.o, 0, 0, "q8 edges")
    # Attention over the worked rows only (a 1e7 block's scale overflows to infinity; the
    # rows past the windows hold such blocks, and must not leak into the results).
    q = custom(92, (3, 4, 64))
    got, want = p.decode(0, [0, 0, 0], [0, 2, 4], dev(q), q, 4, 64, 0.125)
    assert_close(got, want, "q8 decode over edge blocks")
    q5 = custom(93, (5, 4, 64))
    got, want = p.prefill(0, 0, np.arange(5, dtype=np.int32), dev(q5), q5, 4, 64, 0.125)
    assert_close(got, want, "q8 prefill over edge blocks")
    p.close()


@pytest.mark.parametrize("kv", [0, 1], ids=["f32", "f16"])
def test_non_finite_rows_outside_every_window(kv):
    """Rows past every query's window holding inf, -inf and NaN (written at later
    positions): attention sums only over [0, pos], so decode and prefill results stay
    finite and match the oracle, including the prefill's last key tile, which holds
    such rows beside the window's own."""
    say(f"non-finite rows outside the windows, kv {kv}")
    nh, nkv, hd = 4, 2, 64
    p = Pair(1, 1, nkv, hd, 128, dtype=kv)
    k, v = custom(94, (100, nkv, hd)), custom(95, (100, nkv, hd))
    bad = np.array([np.inf, -np.inf, np.nan], np.float32)
    rng = np.random.default_rng(96)
    for a in (k, v):
        a[40:] = bad[rng.integers(0, 3, a[40:].shape)]
    p.append(0, [0] * 100, np.arange(100, dtype=np.int32), None, nh, hd, k, v)
    q = custom(97, (3, nh, hd))
    got, want = p.decode(0, [0, 0, 0], [0, 17, 39], dev(q), q, nh, hd, 0.125)
    assert_close(got, want, "decode beside non-finite rows")
    for nt in (40, 8):
        qp = custom(98 + nt, (nt, nh, hd))
        got, want = p.prefill(0, 0, np.arange(nt, dtype=np.int32), dev(qp), qp, nh, hd, 0.125)
        assert_close(got, want, f"prefill of {nt} beside non-finite rows")
    p.close()


@pytest.mark.parametrize("nt,first_bad,seg", [(48, 30, 0), (200, 150, 0), (200, 150, 1)],
                         ids=["48_tokens", "200_tokens", "200_tokens_split"])
@pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])
def test_non_finite_values_inside_the_prompt(monkeypatch, kv, nt, first_bad, seg):
    """A prompt whose later tokens' v rows hold inf, -inf and NaN: the earlier queries
    share those rows' key tile (the causal diagonal) but not their windows, so their
    results stay finite and match the oracle; the later queries' results are non-finite
    exactly where the oracle's are (same inf / -inf / NaN).  Also with every key tile a
    segment of its own (split-K records and their merge carrying the values)."""
    say(f"non-finite values inside the prompt, kv {kv}, nt {nt}, seg {seg}")
    monkeypatch.setenv("KVC_PREFILL_SEG", str(seg))
    nh, nkv, hd = 4, 2, 64
    p = Pair(1, 1, nkv, hd, 256, dtype=kv)
    k, v = custom(110, (nt, nkv, hd)), custom(111, (nt, nkv, hd))
    big = 1e7 if kv == 2 else np.inf      # Q8_0: a block whose scale overflows
    rng = np.random.default_rng(112)
    pick = rng.integers(0, 4, v[first_bad:].shape)
    v[first_bad:] = np.where(pick == 0, big, np.where(pick == 1, -big, v[first_bad:]))
    if kv != 2:
        v[first_bad + 3, 0, 5] = np.nan
    p.append(0, [0] * nt, np.arange(nt, dtype=np.int32), None, nh, hd, k, v)
    qp = custom(113, (nt, nh, hd))
    got, want = p.prefill(0, 0, np.arange(nt, dtype=np.int32), dev(qp), qp, nh, hd, 0.125)
    assert_close(got[:first_bad], want[:first_bad], "queries before the non-finite rows")
    g, w = got[first_bad:], want[first_bad:]
    assert not np.isfinite(w).all(), "the case must reach non-finite results"
    assert np.array_equal(np.isnan(g), np.isnan(w)), "NaN pattern"
    assert np.array_equal(np.isposinf(g), np.isposinf(w)) and np.array_equal(np.isneginf(g), np.isneginf(w)), "inf pattern"
    fin = np.isfinite(w)
    assert_close(np.where(fin, g, 0.0), np.where(fin, w, 0.0), "finite part of the later queries")
    p.close()


def assert_same_nonfinite(got, want, what):
    """Non-finite results equal the oracle's kind for kind (NaN, +inf, -inf); the finite
    ones pass the allclose bar."""
    assert not np.isfinite(want).all(), f"{what}: the case must reach non-finite results"
    assert np.array_equal(np.isnan(got), np.isnan(want)), f"{what}: NaN pattern"
    assert np.array_equal(np.isposinf(got), np.isposinf(want)), f"{what}: +inf pattern"
    assert np.array_equal(np.isneginf(got), np.isneginf(want)), f"{what}: -inf pattern"
    fin = np.isfinite(want)
    assert_close(np.where(fin, got, 0.0), np.where(fin, want, 0.0), f"{what} (finite part)")


@pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])
def test_decode_non_finite_value_at_a_chunk_start(monkeypatch, kv):
    """A V row holding +inf, -inf and NaN at the first row of a decode chunk whose window
    ends inside a step: the chunk's last step reads rows past its end (masked, weight 0),
    and 0 * inf must not turn the result into NaN where the oracle has +inf or -inf.
    Position windows (chunks of 128 rows over a 300-row window: the last chunk starts at
    row 256 and holds 44 rows) and explicit windows (runs cut into the same chunks, one
    starting at the non-finite row)."""
    say(f"non-finite V at a decode chunk's first row, kv {kv}")
    monkeypatch.setenv("KVC_SPLIT_ROWS", "128")
    nh, nkv, hd = 4, 2, 64
    p = Pair(1, 1, nkv, hd, 320, dtype=kv)
    k, v = custom(120, (300, nkv, hd)), custom(121, (300, nkv, hd))
    if kv == 2:
        # Q8_0 holds finite inputs only; a block whose scale overflows binary16 decodes to
        # +inf, -inf (codes of either sign) and NaN (code 0).
        for row in (256, 278):
            v[row, 0, :32] = np.float32(1e7) * np.sign(custom(122 + row, (32,)))
            v[row, 0, 5] = 0.0
    else:
        for row in (256, 278):
            v[row, 0, 3], v[row, 0, 7], v[row, 0, 11] = np.inf, -np.inf, np.nan
            v[row, 1, 20] = -np.inf
    p.append(0, [0] * 300, np.arange(300, dtype=np.int32), None, nh, hd, k, v)
    q = custom(123, (2, nh, hd))
    got, want = p.decode(0, [0, 0], [299, 255], dev(q), q, nh, hd, 0.125)
    assert_same_nonfinite(got[0], want[0], "decode, window [0, 299]")
    assert_close(got[1], want[1], "decode, window [0, 255] (before the non-finite rows)")
    # Runs [150, 300) then [0, 100): pieces [150, 278), [278, 300), [0, 100).
    got, want = p.decode_runs(0, [0], [[(150, 150), (0, 100)]], dev(q[:1]), q[:1], nh, hd, 0.125)
    assert_same_nonfinite(got, want, "decode over runs")
    p.close()


def test_q8_geometry_is_checked():
    with pytest.raises(kvc.KvcError) as e:
        kvc.kv_alloc(1, 1, 2, 16, 64, dtype=kvc.KV_Q8_0)
    assert e.value.status == kvc.E_GEOMETRY


def test_maximum_capacity_and_last_position():
    """The largest supported region (capacity 2^24 rows) with rows written at its first,
    middle and last positions: RoPE table rows at the end, the stores, a decode whose
    window is all 2^24 rows (split into thousands of chunks, unwritten rows reading as 0)
    and a 3-token prefill at the last positions (split into hundreds of key segments)."""
    cap = 1 << 24
    say(f"maximum capacity {cap}")
    nh, nkv, hd, hdk = 2, 1, 16, 16
    p = Pair(1, 1, nkv, hdk, cap)
    pos = np.array([0, 1, 1 << 23, cap - 3, cap - 2, cap - 1], np.int32)
    q = custom(60, (len(pos), nh, hd))
    k = custom(61, (len(pos), nkv, hdk))
    v = custom(62, (len(pos), nkv, hdk))
    p.append(0, [0] * len(pos), pos, q, nh, hd, k, v)
    compare_cache(p.g, p.o, 0, 0, "max capacity", rows=pos)
    qd = custom(63, (1, nh, hd))
    got, want = p.decode(0, [0], [cap - 1], dev(qd), qd, nh, hd, 0.25)
    assert_close(got, want, "decode over 2^24 rows")
    qp = custom(64, (3, nh, hd))
    got, want = p.prefill(0, 0, pos[-3:], dev(qp), qp, nh, hd, 0.25)
    assert_close(got, want, "prefill at the last positions")
    p.close()
