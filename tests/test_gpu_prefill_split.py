"""GPU prefill with the key range of each query tile cut into segments (split-K prefill).

A short prompt gives too few query tiles to fill the chip, so the library scans each
tile's keys in segments on separate workgroups and merges their (m, l, O) records.
KVC_PREFILL_SEG forces the segment length (or forbids the split), so every case here
runs both paths on the same inputs and checks each against the oracle: segments of one
tile (the most records per query), of a few tiles, the library's own choice, and no
split.  Cases cover the shapes the split has to get right: queries whose window ends
before a segment starts (that segment sees no key of theirs), positions out of order
with gaps, a continuation prompt far into the cache (many segments per tile), idle
heads of a GQA group, 32-key tiles (hd_kv 256) and the three region formats."""
import numpy as np
import pytest

from tests.gpu_util import Pair, assert_close, dev, say
from tests.workloads import custom, custom_positions

pytestmark = pytest.mark.gpu

SEGS = pytest.mark.parametrize("seg", [-1, 1, 3, 0], ids=["nosplit", "seg1", "seg3", "auto"])
FORMATS = pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])


def filled(seed, n_head, n_head_kv, hd, hd_kv, capacity, rows, kv):
    p = Pair(1, 1, n_head_kv, hd_kv, capacity, dtype=kv)
    k = custom(seed, (rows, n_head_kv, hd_kv))
    v = custom(seed + 1, (rows, n_head_kv, hd_kv))
    p.append(0, [0] * rows, np.arange(rows), None, n_head, hd, k, v)
    return p


def run(monkeypatch, seg, p, pos, nh, hd, seed, scale=0.27, sample=None):
    monkeypatch.setenv("KVC_PREFILL_SEG", str(seg))
    q = custom(seed, (len(pos), nh, hd))
    got, want = p.prefill(0, 0, pos, dev(q), q, nh, hd, scale, sample=sample)
    assert_close(got, want, f"prefill seg={seg}")


@FORMATS
@SEGS
def test_causal_prompt_qwen3_heads(monkeypatch, seg, kv):
    """A 200-token causal prompt at positions 0..199 (Qwen3-0.6B heads: G = 2)."""
    say(f"split prefill causal 200 seg={seg} kv={kv}")
    p = filled(100, 16, 8, 128, 128, 256, 200, kv)
    run(monkeypatch, seg, p, np.arange(200, dtype=np.int32), 16, 128, 101)
    p.close()


@FORMATS
@SEGS
def test_scattered_positions_leave_segments_empty(monkeypatch, seg, kv):
    """Positions out of order with gaps and repeats: a tile mixes early and late queries,
    so later segments hold no key of the early ones."""
    say(f"split prefill scattered seg={seg} kv={kv}")
    p = filled(110, 14, 2, 64, 64, 700, 700, kv)
    pos = custom_positions(111, 90, 0, 700, unique=False)
    pos[:5] = [0, 1, 699, 2, 640]
    run(monkeypatch, seg, p, pos, 14, 64, 112)
    p.close()


@FORMATS
@SEGS
def test_continuation_far_into_the_cache(monkeypatch, seg, kv):
    """40 tokens continuing at position 3000 (tens of segments per query tile)."""
    say(f"split prefill continuation seg={seg} kv={kv}")
    p = filled(120, 16, 8, 128, 128, 3072, 3040, kv)
    pos = np.arange(3000, 3040, dtype=np.int32)
    run(monkeypatch, seg, p, pos, 16, 128, 121, sample=[0, 7, 19, 31, 32, 39])
    p.close()


@pytest.mark.parametrize("geom", [(16, 1, 128, 128), (8, 4, 256, 256), (6, 2, 64, 64), (4, 2, 16, 16),
                                  (4, 2, 160, 128)],
                         ids=["g16", "hd256", "g3", "hd16", "hd_gt_hd_kv"])
@SEGS
def test_head_geometries(monkeypatch, seg, geom):
    nh, nkv, hd, hdk = geom
    say(f"split prefill geometry {geom} seg={seg}")
    p = filled(130, nh, nkv, hd, hdk, 400, 400, 0)
    pos = np.concatenate([np.arange(300, 333), custom_positions(131, 30, 0, 400)]).astype(np.int32)
    run(monkeypatch, seg, p, pos, nh, hd, 132)
    p.close()
