"""Launch planning on the host (plan.cpp through the host-only shim, no GPU): how a
prefill's query tiles are cut into workgroup units, and the decode chunk length.

The prefill kernel trusts the unit table completely (which key tiles a workgroup scans,
whether it writes the output or a segment record, how many records the merge folds), so
the properties here are the ones its correctness rests on: every query tile's key tiles
[0, tiles) are covered exactly once, in segment order, each segment knows its index and
its tile's segment count, and the key-tile count of a tile follows from its largest
position."""
import ctypes
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOSTCHECK = os.path.join(ROOT, "kv_cache_causal_amd", "lib", "libkvc_hostcheck.so")


@pytest.fixture(scope="module")
def hc():
    if not os.path.exists(HOSTCHECK):
        pytest.skip("host-check shim not built")
    L = ctypes.CDLL(HOSTCHECK)
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.hc_plan_prefill.argtypes = [p, i32, i32, i32, i32, i32, p, p, i32]
    L.hc_decode_chunk_rows.argtypes = [i64, i32, i32, i64]
    L.hc_decode_chunk_rows.restype = i64
    L.hc_decode_one_round_rows.argtypes = [p, i32, i32, i32, i64, i32, i64, i32]
    L.hc_decode_one_round_rows.restype = i64
    L.hc_decode_one_round_excess.argtypes = [i32]
    L.hc_decode_one_round_excess.restype = i32
    L.hc_max_part_bytes.restype = i64
    return L


def seg_length(hc, tiles, hgroups, nt, n_head, hd_kv, force=0):
    """The documented segment length: tiles spread over ~512 units, at least 3 (or the
    forced length), grown until max_seg records per query row fit the scratch cap."""
    s = force if force > 0 else max(3, -(-sum(tiles) * hgroups // 512))
    max_recs = max(1, hc.hc_max_part_bytes() // (nt * n_head * (hd_kv + 4) * 4))
    return max(s, -(-max(tiles) // max_recs))


UNIT_INTS = 8


def plan(hc, pos, n_head, n_head_kv, hd_kv, force=0):
    pos = np.ascontiguousarray(np.asarray(pos, np.int32))
    meta = np.zeros(9, np.int32)
    cap = 1 << 20
    units = np.zeros(cap, np.int32)
    assert hc.hc_plan_prefill(pos.ctypes.data, len(pos), n_head, n_head_kv, hd_kv, force,
                              meta.ctypes.data, units.ctypes.data, cap) == 0
    keys = ("GB", "TQ", "n_qtiles", "n_hsub", "KT", "units_per_hgroup", "max_seg", "n_units",
            "contiguous")
    m = dict(zip(keys, (int(x) for x in meta)))
    return m, units[:m["n_units"]].reshape(-1, UNIT_INTS)


def tiles_of(pos, TQ, KT):
    """Key tiles each query tile must scan: up to its largest position."""
    return [int(pos[q:q + TQ].max()) // KT + 1 for q in range(0, len(pos), TQ)]


def check_units(m, u, pos, seg_len):
    """The unit table: every query tile's key tiles covered exactly once, in segment order
    (one whole-tile unit per query tile when nothing is split), heavy tiles first, and
    each unit carrying its query tile's largest and smallest position."""
    pos = np.asarray(pos)
    tiles = tiles_of(pos, m["TQ"], m["KT"])
    assert m["n_qtiles"] == len(tiles)
    assert m["units_per_hgroup"] == len(u)
    assert m["contiguous"] == int(bool(np.all(np.diff(pos) == 1)))
    if m["max_seg"] == 1:
        seg_len = max(tiles)
        assert len(u) == m["n_qtiles"]
    seen = {}
    for qt, k0, nk, code, kmax, kmin, z0, z1 in u:
        seg, nseg = code >> 16, code & 0xFFFF
        toks = pos[qt * m["TQ"]:(qt + 1) * m["TQ"]]
        assert kmax == toks.max() and kmin == toks.min() and z0 == 0 and z1 == 0
        seen.setdefault(int(qt), []).append((int(k0), int(nk), int(seg), int(nseg)))
    assert sorted(seen) == list(range(len(tiles)))          # every query tile has units
    order = [int(q) for q in u[:, 0]]
    assert order == sorted(order, reverse=True)             # heavy (late) tiles first
    for qt, segs in seen.items():
        nseg = len(segs)
        assert [s[2] for s in segs] == list(range(nseg))    # segment indices in order
        assert all(s[3] == nseg for s in segs)              # each knows the count
        assert nseg <= m["max_seg"]
        k = 0
        for k0, nk, _, _ in segs:                           # contiguous, exact cover
            assert k0 == k and 1 <= nk <= seg_len
            k += nk
        assert k == tiles[qt]
        if m["max_seg"] > 1:
            assert all(nk == seg_len for _, nk, _, _ in segs[:-1])
    assert m["max_seg"] == max(len(s) for s in seen.values())


GEOMS = [  # n_head, n_head_kv, hd_kv
    (16, 8, 128),   # Qwen3-0.6B: G = 2 -> 2 heads x 32 tokens per tile
    (14, 2, 64),    # Qwen2.5-0.5B: G = 7 -> 4 heads x 16 tokens, two head subsets
    (8, 4, 256),    # 32-key tiles
    (4, 4, 16),     # G = 1 -> 64 tokens per tile
    (16, 1, 128),   # G = 16 -> four head subsets
]


@pytest.mark.parametrize("g", GEOMS, ids=[f"h{a}kv{b}d{c}" for a, b, c in GEOMS])
def test_tile_shape(hc, g):
    n_head, n_head_kv, hd_kv = g
    m, _ = plan(hc, np.arange(100), n_head, n_head_kv, hd_kv, force=-1)
    G = n_head // n_head_kv
    assert m["GB"] == min(4, 1 << (G.bit_length() - 1)) and m["GB"] * m["TQ"] == 64
    assert m["n_hsub"] * m["GB"] >= G > (m["n_hsub"] - 1) * m["GB"]
    assert m["KT"] == (32 if hd_kv >= 256 else 64)
    assert m["n_qtiles"] == -(-100 // m["TQ"])


@pytest.mark.parametrize("g", GEOMS, ids=[f"h{a}kv{b}d{c}" for a, b, c in GEOMS])
def test_short_causal_prompts_split_with_the_documented_length(hc, g):
    n_head, n_head_kv, hd_kv = g
    for nt in (1, 40, 200, 511):
        pos = np.arange(nt, dtype=np.int32)
        m, u = plan(hc, pos, n_head, n_head_kv, hd_kv)
        hgroups = n_head_kv * m["n_hsub"]
        tiles = tiles_of(pos, m["TQ"], m["KT"])
        if hgroups * m["n_qtiles"] >= 512:
            assert m["max_seg"] == 1
            check_units(m, u, pos, 0)
            continue
        seg_len = seg_length(hc, tiles, hgroups, nt, n_head, hd_kv)
        check_units(m, u, pos, seg_len)
        assert (m["max_seg"] > 1) == (max(tiles) > seg_len)


def test_continuation_and_scattered_positions(hc):
    rng = np.random.default_rng(7)
    cases = [np.arange(8000, 8064), np.arange(4000, 4256),
             rng.integers(0, 3000, 90), np.array([0, 1, 2999, 2, 2500] + list(range(40)))]
    for pos in cases:
        for g in GEOMS:
            m, u = plan(hc, pos, *g)
            hgroups = g[1] * m["n_hsub"]
            tiles = tiles_of(pos, m["TQ"], m["KT"])
            seg_len = seg_length(hc, tiles, hgroups, len(pos), g[0], g[2])
            check_units(m, u, pos, seg_len)


def test_forced_segment_lengths_and_no_split(hc):
    pos = np.arange(3000, 3040, dtype=np.int32)
    for force in (1, 2, 3, 7, 1000):
        m, u = plan(hc, pos, 16, 8, 128, force)
        check_units(m, u, pos, force)
    m, u = plan(hc, pos, 16, 8, 128, -1)
    assert m["max_seg"] == 1
    check_units(m, u, pos, 0)
    # Large prompts fill the chip unsplit, unless a length is forced.
    big = np.arange(4096, dtype=np.int32)
    m, u = plan(hc, big, 16, 8, 128)
    assert m["max_seg"] == 1 and m["units_per_hgroup"] == 128
    check_units(m, u, big, 0)
    m, u = plan(hc, big, 16, 8, 128, 16)
    check_units(m, u, big, 16)


def test_partial_records_stay_within_the_cap(hc):
    """One late position among thousands of early ones: the late query tile alone would
    want hundreds of segments; they grow until max_seg x nt x n_head x (hd_kv + 4) floats
    fit the scratch cap, and the cover stays exact."""
    cap = hc.hc_max_part_bytes()
    for n_head, n_head_kv, hd_kv, nt in ((4, 1, 256, 8000), (16, 8, 128, 1000), (4, 4, 16, 4000)):
        pos = np.arange(nt, dtype=np.int32) % 64
        pos[-1] = (1 << 24) - 1
        m, u = plan(hc, pos, n_head, n_head_kv, hd_kv)
        hgroups = n_head_kv * m["n_hsub"]
        if hgroups * m["n_qtiles"] >= 512:
            continue
        tiles = tiles_of(pos, m["TQ"], m["KT"])
        check_units(m, u, pos, seg_length(hc, tiles, hgroups, nt, n_head, hd_kv))
        assert m["max_seg"] * nt * n_head * (hd_kv + 4) * 4 <= cap


def test_decode_chunk_rows(hc):
    f = hc.hc_decode_chunk_rows
    for br in (16, 32, 64, 128):
        for hpb in (1, 2, 4):
            prev = 0
            for work in (1, 100, 10_000, 131_072, 131_073, 500_000, 1 << 20, (1 << 20) + 1,
                         1 << 26):
                r = f(work, br, hpb, 0)
                assert r >= br and r % br == 0
                assert r >= prev                              # never shrinks with work
                prev = r
            up = lambda x: max(br, -(-x // br) * br)          # noqa: E731 (round up to br)
            assert f(131_073, br, hpb, 0) == up(512 // hpb)        # middle range: 512 rows
            assert f(1 << 26, br, hpb, 0) == up((1 << 26) // 2048 // hpb)   # ~2048 workgroups
            assert f(512 * 40, br, hpb, 0) == up(40 // hpb)        # small: ~512 workgroups
            assert f(10_000, br, hpb, 100) == up(100)              # forced, rounded up to br


def one_round(hc, lens, n_head_kv, hpb, slots, br, rows, excess=15):
    a = np.ascontiguousarray(np.asarray(lens, np.int64))
    return hc.hc_decode_one_round_rows(a.ctypes.data, len(a), n_head_kv, hpb, slots, br, rows,
                                       excess)


def test_decode_one_round_rows(hc):
    """The one-round chunk length: the shortest multiple of br (from the rule's length up)
    whose chunks x head blocks fit the resident workgroups, taken only above the small
    range (131,072 row-heads) and within the format's limit above a perfect balance (20%
    for binary16, 15% for f32 and Q8_0); anything else keeps the rule's length."""
    assert [hc.hc_decode_one_round_excess(f) for f in (0, 1, 2)] == [15, 20, 15]
    from tests.workloads import batch_n_past
    lens = batch_n_past().astype(np.int64) + 1         # the 32-sequence batch's windows
    blocks = lambda r, nkv, hpb: int(np.sum((lens + r - 1) // r)) * (nkv // hpb)  # noqa: E731
    # binary16 / Q8_0 at 2 kv heads per workgroup, 3 resident workgroups per CU: 768 rows
    # (748 workgroups), 12% above the balance of 685 rows per workgroup.
    assert one_round(hc, lens, 8, 2, 768, 32, 288) == 768
    assert blocks(768, 8, 2) <= 768 < blocks(736, 8, 2)
    # One kv head per workgroup (1,664 rows: 21.4% above the balance) and f32 at 2 resident
    # workgroups per CU (2,944 rows: 43% above): the rule's length stays.
    assert one_round(hc, lens, 8, 1, 768, 64, 576) == 576
    assert one_round(hc, lens, 8, 1, 768, 64, 576, 20) == 576
    assert one_round(hc, lens, 8, 1, 512, 128, 640) == 640
    assert one_round(hc, lens, 8, 1, 768, 64, 576, 22) == 1664   # within a 22% limit
    # Small work, unknown occupancy, or no length that fits: unchanged.
    assert one_round(hc, [16384], 8, 2, 768, 32, 256) == 256   # 131,072 row-heads: small
    assert one_round(hc, [16385], 8, 2, 768, 32, 256) == 256   # the rule's 260 fit already
    assert one_round(hc, [8193] * 8, 8, 2, 768, 32, 256) == 352   # 8 x 24 chunks x 4 blocks
    assert one_round(hc, lens, 8, 2, 0, 32, 288) == 288
    assert one_round(hc, lens, 8, 2, 100, 32, 288) == 288
    # Random cases against a direct search.
    rng = np.random.default_rng(11)
    for _ in range(300):
        m = int(rng.integers(1, 65))
        ls = rng.integers(1, 40000, m).astype(np.int64)
        nkv, hpb = [(8, 2), (8, 1), (2, 2), (4, 1), (16, 2)][int(rng.integers(0, 5))]
        br = int(rng.choice([16, 32, 64, 128]))
        slots = int(rng.choice([256, 512, 768, 1024, 2048]))
        rows = br * int(rng.integers(1, 40))
        excess = int(rng.choice([15, 20]))
        got = one_round(hc, ls, nkv, hpb, slots, br, rows, excess)
        if int(ls.sum()) * nkv <= 131072:
            assert got == rows
            continue
        wg = lambda r: int(np.sum((ls + r - 1) // r)) * (nkv // hpb)  # noqa: E731
        want = rows
        top = max(rows, -(-int(ls.max()) // br) * br)
        if wg(top) <= slots:
            r = rows
            while wg(r) > slots:
                r += br
            if r * slots * 100 <= int(ls.sum()) * (nkv // hpb) * (100 + excess):
                want = r
        assert got == want, (m, nkv, hpb, br, slots, rows, got, want)
        assert got % br == 0 and got >= rows


def test_rope_exact_evaluation_constants(hc):
    """The digits of 2/pi and the double-double pi/2 and ln 2 the RoPE table's exact path
    uses, against 400-bit values: every word, and hi/lo the nearest doubles to the value
    and to its remainder."""
    import mpmath
    hc.hc_rope_consts.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hc.hc_rope_consts.restype = ctypes.c_int32
    words = np.zeros(16, np.uint32)
    dd = np.zeros(4, np.float64)
    n = hc.hc_rope_consts(words.ctypes.data, dd.ctypes.data)
    with mpmath.workprec(400):
        digits = int(mpmath.floor(2 / mpmath.pi * mpmath.mpf(2) ** (32 * n)))
        want = [(digits >> (32 * (n - 1 - k))) & 0xFFFFFFFF for k in range(n)]
        assert [int(w) for w in words[:n]] == want
        for (hi, lo), x in (((dd[0], dd[1]), mpmath.pi / 2), ((dd[2], dd[3]), mpmath.log(2))):
            assert hi == float(x) and lo == float(x - mpmath.mpf(float(x)))
