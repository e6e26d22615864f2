"""gqa_attn_decode_noalloc through the C ABI: the decode whose split-K records live in
the library's fixed device scratch (no allocation, no wait) against gqa_attn_decode on
the same inputs -- bit for bit, since both queue the same kernels with the same chunks
-- and against the oracle within the attention bar; two calls in a row, the second
smaller (the fixed scratch keeps the first call's records, which the second must not
read); and a call whose records would not fit the scratch, refused before anything is
queued."""
import numpy as np
import pytest

import kv_cache_causal_amd as kvc
from tests.gpu_util import Pair, assert_bitwise, assert_close, dev, host, say
from tests.workloads import custom

pytestmark = pytest.mark.gpu

NH, NKV, HD = 16, 8, 128
SCALE = 0.0883883461356163


def filled_pair(n_seq, rows):
    p = Pair(n_seq, 1, NKV, HD, int(max(rows)) + 64)
    for s, r in enumerate(rows):
        k = custom(140 + s, (int(r), NKV, HD))
        v = custom(170 + s, (int(r), NKV, HD))
        p.append(0, [s] * int(r), np.arange(int(r), dtype=np.int32), None, NH, HD, k, v)
    return p


def both(p, seqs, pos, q):
    import torch
    n = len(seqs)
    a = torch.full((n, NH, HD), 3.0, device="cuda")
    b = torch.full((n, NH, HD), 5.0, device="cuda")
    kvc.gqa_attn_decode(p.g, 0, seqs, pos, dev(q), NH, HD, SCALE, a)
    kvc.gqa_attn_decode_noalloc(p.g, 0, seqs, pos, dev(q), NH, HD, SCALE, b)
    return host(a), host(b)


def test_noalloc_matches_decode_two_calls_second_smaller():
    rows = np.array([5000, 4100, 3000, 2500, 1800, 900, 300, 129])
    p = filled_pair(len(rows), rows)
    # Call 1: 70 entries (two launches of up to 64), windows of up to 5,000 rows.
    rng = np.random.default_rng(150)
    seqs = rng.integers(0, len(rows), 70).astype(np.int32)
    pos = np.array([rng.integers(0, rows[s]) for s in seqs], np.int32)
    pos[:8] = rows - 1
    q = custom(151, (70, NH, HD))
    say("no-alloc decode, call 1: 70 entries")
    a, b = both(p, seqs, pos, q)
    assert_bitwise(b, a, "noalloc vs gqa_attn_decode, call 1")
    st, want = p.o.attn_decode(0, seqs, pos, q, NH, HD, SCALE)
    assert st == 0
    assert_close(b, want, "noalloc vs oracle, call 1")
    # Call 2: fewer, shorter windows.
    seqs2 = np.array([6, 7, 5], np.int32)
    pos2 = np.array([299, 100, 777], np.int32)
    q2 = custom(152, (3, NH, HD))
    say("no-alloc decode, call 2: 3 entries")
    a, b = both(p, seqs2, pos2, q2)
    assert_bitwise(b, a, "noalloc vs gqa_attn_decode, call 2")
    st, want = p.o.attn_decode(0, seqs2, pos2, q2, NH, HD, SCALE)
    assert_close(b, want, "noalloc vs oracle, call 2")
    p.close()


def test_noalloc_refuses_a_call_beyond_its_scratch(monkeypatch):
    """64-row chunks over 64 windows of 5,000 rows need about 10.7 M floats of records,
    more than the 4 M the fixed scratch holds: KVC_E_ARG, output untouched.  The same
    call through gqa_attn_decode (handle scratch, grown on demand) still runs."""
    import torch
    monkeypatch.setenv("KVC_SPLIT_ROWS", "64")
    p = filled_pair(1, [5000])
    seqs = np.zeros(64, np.int32)
    pos = np.full(64, 4999, np.int32)
    q = custom(153, (64, NH, HD))
    out = torch.full((64, NH, HD), 7.0, device="cuda")
    with pytest.raises(kvc.KvcError) as ei:
        kvc.gqa_attn_decode_noalloc(p.g, 0, seqs, pos, dev(q), NH, HD, SCALE, out)
    assert ei.value.status == kvc.E_ARG and "fixed scratch" in ei.value.message
    assert (host(out) == 7.0).all()
    kvc.gqa_attn_decode(p.g, 0, seqs, pos, dev(q), NH, HD, SCALE, out)
    st, want = p.o.attn_decode(0, seqs[:1], pos[:1], q[:1], NH, HD, SCALE)
    assert_close(host(out)[:1], want, "handle-scratch decode of the same call")
    p.close()
