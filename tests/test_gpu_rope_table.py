"""The device RoPE tables read out entry by entry, through the C ABI, against the oracle.

A k (or q) row whose pairs are (1, 0) comes out of the rotation as exactly (cos, sin) of
its table row: 1 * c - 0 * s = c and 1 * s + 0 * c = s, each step exact.  Appending such
rows at every position below a cache's capacity therefore writes every entry of the
k table into the K region, and rotating such q rows (query head dim above the kv head
dim: a table of its own) every entry of the q table into q; both are compared bit for
bit with the oracle's correctly rounded tables.  A second pass appends N(0,1) rows at
every position (the rotation's own arithmetic over the whole table).

Grids: the workloads' kv head dims with their capacities (16 / 520, 64 / 1,023,
128 / 40,960), query head dims 48, 96 and 192, base 1e6, NEOX and interleaved pairs
("11 · Attention, vec ops, and the KV cache" §2.3, §3.2.2).
"""
import numpy as np
import pytest

from tests.gpu_util import Pair, compare_cache, say
from tests.workloads import custom

pytestmark = pytest.mark.gpu

GRIDS = [(16, 520, 48), (64, 1023, 96), (128, 40960, 192)]


def unit_pairs(n, heads, width, style):
    x = np.zeros((n, heads, width), np.float32)
    if style == 0:
        x[..., : width // 2] = 1.0      # NEOX pairs (i, i + width/2)
    else:
        x[..., 0::2] = 1.0              # interleaved pairs (2i, 2i + 1)
    return x


@pytest.mark.parametrize("style", [0, 1], ids=["neox", "interleaved"])
@pytest.mark.parametrize("hd_kv,cap,hd", GRIDS, ids=[f"dk{a}_cap{b}_dq{c}" for a, b, c in GRIDS])
def test_every_table_entry(hd_kv, cap, hd, style):
    say(f"rope tables: hd_kv {hd_kv} (capacity {cap}), hd {hd}, style {style}")
    p = Pair(1, 1, 1, hd_kv, cap)
    pos = np.arange(cap, dtype=np.int32)
    seqs = np.zeros(cap, np.int32)
    k = unit_pairs(cap, 1, hd_kv, style)
    q = unit_pairs(cap, 1, hd, style)
    v = custom(130 + hd_kv, (cap, 1, hd_kv))
    # The q rows come back bit for bit (Pair.append checks them): every q-table entry.
    p.append(0, seqs, pos, q, 1, hd, k, v, 1.0e6, 1.0, style)
    compare_cache(p.g, p.o, 0, 0, "k-table readout")
    q = custom(131 + hd_kv, (cap, 1, hd))
    k = custom(132 + hd_kv, (cap, 1, hd_kv))
    p.append(0, seqs, pos, q, 1, hd, k, v, 1.0e6, 1.0, style)
    compare_cache(p.g, p.o, 0, 0, "N(0,1) rows at every position")
    p.close()


@pytest.mark.parametrize("hd_kv,cap,hd", GRIDS, ids=[f"dk{a}_cap{b}_dq{c}" for a, b, c in GRIDS])
def test_every_table_entry_through_the_exact_path(monkeypatch, hd_kv, cap, hd):
    """KVC_ROPE_EXACT=1: every entry evaluated in double-double (argument reduction by the
    digits of 2/pi, Taylor series, exp / log for the speeds) instead of only the f64
    values the bound cannot certify -- the same bits as the oracle everywhere."""
    monkeypatch.setenv("KVC_ROPE_EXACT", "1")
    say(f"rope tables, exact path: hd_kv {hd_kv} (capacity {cap}), hd {hd}")
    p = Pair(1, 1, 1, hd_kv, cap)
    pos = np.arange(cap, dtype=np.int32)
    p.append(0, np.zeros(cap, np.int32), pos, unit_pairs(cap, 1, hd, 0), 1, hd,
             unit_pairs(cap, 1, hd_kv, 0), custom(133, (cap, 1, hd_kv)), 1.0e6, 1.0, 0)
    compare_cache(p.g, p.o, 0, 0, "exact-path table readout")
    p.close()


def near_ties():
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "rope_near_ties.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("exact", [0, 1], ids=["certified", "exact"])
def test_near_tie_angles_and_speeds(monkeypatch, exact):
    """Angles and speeds whose exact cos, sin or speed lies within about 2^-53 of an f32
    midpoint (tests/golden/rope_near_ties.json, angles from 8e-4 to 3e35): the tables
    hold the oracle's correctly rounded values.  An angle is freq_scale itself at pair 0,
    position 1; a speed fs / base^(1/2) is pair 4 of head dim 16 (exponent 8/16), and at
    position 1 its angle is below 2^-12, where the sin entry is the angle itself."""
    monkeypatch.setenv("KVC_ROPE_EXACT", str(exact))
    g = near_ties()
    say(f"near-tie angles ({len(g['angles'])}) and speeds ({len(g['speeds'])}), exact {exact}")
    p = Pair(1, 1, 1, 16, 2)
    k = unit_pairs(1, 1, 16, 0)
    q = unit_pairs(1, 1, 32, 0)
    v = custom(134, (1, 1, 16))
    for a in g["angles"]:
        th = float(np.uint32(a["theta_bits"]).view(np.float32))
        p.append(0, [0], [1], q, 1, 32, k, v, 1.0e4, th, 0)
        compare_cache(p.g, p.o, 0, 0, f"angle {th!r}", rows=[1])
    for sp in g["speeds"]:
        fs = float(np.uint32(sp["freq_scale_bits"]).view(np.float32))
        base = float(np.uint32(sp["base_bits"]).view(np.float32))
        p.append(0, [0], [1], q, 1, 32, k, v, base, fs, 0)
        compare_cache(p.g, p.o, 0, 0, f"speed {fs!r} / {base!r}^(1/2)", rows=[1])
    p.close()
