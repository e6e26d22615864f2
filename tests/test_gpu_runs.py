"""Explicit attention windows on the GPU (gqa_attn_decode_runs) against the oracle.

"13 · The decode loop and graph reuse" §2.2 (Budget 3): a decode query's cells are an
input -- a list of runs -- not a bound derived from positions; §3.4 item 4: cells past a
rolled-back cursor are never read.  Cases: one run [0, pos] (bit-identical to the
position-derived decode, which cuts the window into the same chunks), scattered and
out-of-order runs, runs long enough to be cut into many chunks, batches of more than 64
entries (several launches), the three region formats, stale rows outside every window,
and malformed windows that must leave the output untouched."""
import numpy as np
import pytest

import kv_cache_causal_amd as kvc
from tests import workloads as W
from tests.gpu_util import Pair, assert_bitwise, assert_close, dev, host, say
from tests.workloads import custom

pytestmark = pytest.mark.gpu

FORMATS = pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])


def fill(pair, seed, n_seq, rows, nkv, hdk):
    for s in range(n_seq):
        k = custom(seed + s, (rows, nkv, hdk))
        v = custom(seed + 500 + s, (rows, nkv, hdk))
        pair.append(0, [s] * rows, np.arange(rows), None, 0, 0, k, v, 1e6, 1.0, 2)


def random_runs(rng, cap, n_runs, max_len):
    """Disjoint runs inside [0, cap), in random order."""
    cuts = np.sort(rng.choice(np.arange(1, cap), size=2 * n_runs, replace=False))
    runs = []
    for i in range(n_runs):
        a, b = int(cuts[2 * i]), int(cuts[2 * i + 1])
        runs.append((a, min(b - a, max_len)))
    rng.shuffle(runs)
    return runs


@FORMATS
def test_single_run_matches_position_window(kv):
    """The batch workload's 32 windows as one run each: bit-identical to gqa_attn_decode."""
    w = W.QWEN3_BATCH
    say(f"runs = causal windows, batch workload, kv={kv}")
    p = Pair(w.n_seq, 1, w.n_head_kv, w.hd_kv, w.capacity, dtype=kv)
    n_past = W.batch_n_past(w)
    for s in range(w.n_seq):
        rows = int(n_past[s])
        for ci, r0 in enumerate(range(0, rows, 4096)):
            r1 = min(rows, r0 + 4096)
            k, v = W.fill_rows(w, s, 0, ci, r1 - r0)
            p.append(0, [s] * (r1 - r0), np.arange(r0, r1), None, 0, 0,
                     k.reshape(r1 - r0, w.n_head_kv, w.hd_kv), v.reshape(r1 - r0, w.n_head_kv, w.hd_kv),
                     w.base, w.freq_scale, w.style)
    q, _, _ = W.decode_qkv(w, w.n_seq, 0, 0)
    seqs = np.arange(w.n_seq, dtype=np.int32)
    pos = n_past - 1
    import torch
    qd = dev(q)
    ref = torch.empty((w.n_seq, w.n_head, w.hd_kv), dtype=torch.float32, device="cuda")
    kvc.gqa_attn_decode(p.g, 0, seqs, pos, qd, w.n_head, w.hd, w.scale, ref)
    got, want = p.decode_runs(0, seqs, [[(0, int(x) + 1)] for x in pos], qd, q, w.n_head, w.hd,
                              w.scale)
    assert_bitwise(got, host(ref), "runs [0, pos] vs position window")
    assert_close(got, want, "runs vs oracle")
    p.close()


@FORMATS
def test_scattered_runs(kv):
    """70 entries (two launches), 1-6 runs each in random order, some long enough to be
    cut into several chunks, over 3 sequences of one layer."""
    say(f"scattered runs kv={kv}")
    cap, nkv, hdk, nh, hd = 6000, 4, 128, 8, 128
    p = Pair(3, 1, nkv, hdk, cap, dtype=kv)
    fill(p, 200, 3, cap, nkv, hdk)
    rng = np.random.default_rng(201)
    n = 70
    seqs = rng.integers(0, 3, n).astype(np.int32)
    runs = [random_runs(rng, cap, int(rng.integers(1, 7)), int(rng.choice([1, 7, 300, 5000])))
            for _ in range(n)]
    q = custom(202, (n, nh, hd))
    got, want = p.decode_runs(0, seqs, runs, dev(q), q, nh, hd, 0.0883883461356163)
    assert_close(got, want, "scattered runs")
    p.close()


@pytest.mark.parametrize("nh,nkv,hd,hdk", [(14, 2, 64, 64), (4, 2, 48, 32), (16, 1, 128, 128)],
                         ids=["g7", "hd_gt_hdkv", "g16"])
def test_runs_head_shapes(nh, nkv, hd, hdk):
    say(f"runs shapes n_head={nh} n_head_kv={nkv} hd={hd} hd_kv={hdk}")
    cap = 700
    p = Pair(2, 1, nkv, hdk, cap)
    fill(p, 210, 2, cap, nkv, hdk)
    runs = [[(650, 50), (0, 1)], [(10, 300), (400, 250)], [(699, 1)]]
    q = custom(211, (3, nh, hd))
    got, want = p.decode_runs(0, [0, 1, 1], runs, dev(q), q, nh, hd, 0.2)
    assert_close(got, want, "runs shapes")
    p.close()


@FORMATS
def test_stale_rows_outside_the_window_are_not_read(kv):
    """Rolled-back rows past the window are rewritten with huge values (infinite as
    binary16, an overflowed scale as Q8_0): the output is the same to the bit.  The run
    edges are not multiples of 4, so rewritten rows share a Q8_0 row quad with rows of
    the window."""
    say(f"runs rollback kv={kv}")
    cap, nkv, hdk, nh = 3000, 2, 64, 4
    p = Pair(1, 1, nkv, hdk, cap, dtype=kv)
    fill(p, 220, 1, cap, nkv, hdk)
    runs = [[(0, 1501)], [(0, 701), (2002, 998)]]
    q = custom(221, (2, nh, hdk))
    qd = dev(q)
    before, want = p.decode_runs(0, [0, 0], runs, qd, q, nh, hdk, 0.125)
    assert_close(before, want, "before rollback")
    junk = np.full((1301, nkv, hdk), 1e30, np.float32)
    p.append(0, [0] * 1301, np.arange(701, 2002), None, 0, 0, junk, junk, 1e6, 1.0, 2)
    after, _ = p.decode_runs(0, [0], [runs[1]], qd[1:], q[1:], nh, hdk, 0.125)
    assert_bitwise(after, before[1:], "window unchanged by stale rows")
    p.close()


def test_malformed_windows_leave_output_untouched():
    import torch
    say("runs errors")
    p = Pair(2, 1, 2, 32, 100)
    fill(p, 230, 2, 100, 2, 32)
    q = dev(custom(231, (2, 4, 32)))
    out = torch.full((2, 4, 32), 7.0, device="cuda")
    cases = [
        ([[(0, 10), (5, 3)], [(0, 1)]], kvc.E_DUP),
        ([[(95, 6)], [(0, 1)]], kvc.E_RANGE),
        ([[(0, 0)], [(0, 1)]], kvc.E_ARG),
        ([[], [(0, 1)]], kvc.E_ARG),
    ]
    for runs, want in cases:
        with pytest.raises(kvc.KvcError) as e:
            kvc.gqa_attn_decode_runs(p.g, 0, [0, 1], runs, q, 4, 32, 0.2, out)
        assert e.value.status == want, (runs, e.value.status)
    assert (host(out) == 7.0).all()
    p.close()
