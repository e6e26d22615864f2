"""GPU parity for the kv head dims between the powers of two: 80, 96, 112, 160 and 192
(f32 and binary16 regions; Q8_0 regions keep 32, 64, 128, 256).  The decode lays its
lanes out for the next power of two, and the lanes past the head dim load nothing; the
prefill's K/V tiles, swizzle and output grouping take any multiple of 16.  Each case
checks against the oracle: the cache rows and the rotated q bit for bit, the prefill
(key ranges split and unsplit) and the decode (one chunk, many chunks, explicit runs)
within the attention tolerance, and the fused projection step bit for bit."""
import numpy as np
import pytest

from tests.gpu_util import Pair, assert_bitwise, assert_close, compare_cache, dev, say
from tests.test_gpu_qkv import weights
from tests.workloads import custom, custom_positions

pytestmark = pytest.mark.gpu

DIMS = [80, 96, 112, 160, 192]
FORMATS = pytest.mark.parametrize("kv", [0, 1], ids=["f32", "f16"])


@FORMATS
@pytest.mark.parametrize("hdk", DIMS, ids=[f"hdkv{d}" for d in DIMS])
@pytest.mark.parametrize("G,extra", [(2, 0), (3, 16)], ids=["g2", "g3_hd_gt_hdkv"])
def test_append_prefill_decode(monkeypatch, hdk, kv, G, extra):
    nkv, cap, rows = 2, 700, 600
    nh, hd = nkv * G, hdk + extra
    say(f"head dim hd_kv={hdk} hd={hd} G={G} kv={kv}")
    p = Pair(2, 1, nkv, hdk, cap, dtype=kv)
    for s in range(2):
        q = custom(500 + s, (rows, nh, hd))
        k = custom(510 + s, (rows, nkv, hdk))
        v = custom(520 + s, (rows, nkv, hdk))
        p.append(0, [s] * rows, np.arange(rows), q, nh, hd, k, v, 1e6, 1.0, s % 2)
        compare_cache(p.g, p.o, s, 0, f"hd_kv {hdk} seq {s}")
    # Prefill of a 130-token continuation (ragged query tiles), the key ranges split as
    # the plan chooses, forced into 2-tile segments, and unsplit.
    nt = 130
    qp = custom(530, (nt, nh, hd))
    pos = np.arange(rows - nt, rows, dtype=np.int32)
    for seg in (0, 2, -1):
        monkeypatch.setenv("KVC_PREFILL_SEG", str(seg))
        got, want = p.prefill(0, 0, pos, dev(qp), qp, nh, hd, 0.2)
        assert_close(got, want, f"prefill seg={seg}")
    # Scattered positions with repeats (early and late queries in one tile).
    pos = custom_positions(531, 70, 0, rows, unique=False)
    got, want = p.prefill(1, 0, pos, dev(qp[:70]), qp[:70], nh, hd, 0.2)
    assert_close(got, want, "prefill scattered")
    # Decode: windows of 600, 18 and 321 rows; chunks as planned, then of 64 rows.
    qd = custom(540, (3, nh, hd))
    seqs, dpos = [0, 1, 0], [599, 17, 320]
    for split in ("0", "64"):
        monkeypatch.setenv("KVC_SPLIT_ROWS", split)
        got, want = p.decode(0, seqs, dpos, dev(qd), qd, nh, hd, 0.17)
        assert_close(got, want, f"decode split rows {split}")
    monkeypatch.setenv("KVC_SPLIT_ROWS", "0")
    runs = [[(300, 200), (0, 100)], [(5, 7)], [(599, 1), (0, 64)]]
    got, want = p.decode_runs(0, seqs, runs, dev(qd), qd, nh, hd, 0.17)
    assert_close(got, want, "decode runs")
    p.close()


@FORMATS
@pytest.mark.parametrize("hdk", DIMS, ids=[f"hdkv{d}" for d in DIMS])
@pytest.mark.parametrize("nt", [1, 6], ids=["nt1", "nt6"])
def test_fused_step(hdk, kv, nt):
    """The fused projection + RoPE + store: q and the cache rows equal the oracle's."""
    say(f"fused step hd_kv={hdk} kv={kv} nt={nt}")
    d, nh, nkv = 256, 4, 2
    p = Pair(2, 1, nkv, hdk, 64, dtype=kv)
    ws = weights(550 + hdk, d, nh, hdk, nkv, hdk)
    x = custom(551, (nt, d))
    seqs = np.arange(nt, dtype=np.int32) % 2
    pos = np.arange(nt, dtype=np.int32) // 2 + 5
    for style in (0, 1):
        qg, qo = p.qkv(0, seqs, pos, x, ws, nh, hdk, 1e6, 1.0, style)
        assert_bitwise(qg, qo, f"rotated q style {style}")
        for s in range(2):
            compare_cache(p.g, p.o, s, 0, f"fused hd_kv {hdk} seq {s}")
    p.close()
