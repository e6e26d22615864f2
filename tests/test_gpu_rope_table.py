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
