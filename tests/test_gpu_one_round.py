"""Decodes whose chunk plan fills one round of resident workgroups, against the oracle.

Above the small range (131,072 row-heads) a decode of one launch takes, where it balances,
the shortest chunk whose workgroups all fit the device at once (the plan is pinned on
the host in test_plan_host.py); binary16 and Q8_0 regions at query-head group 2 then run
two kv heads per workgroup.  The windows here are ragged (8 sequences of 6,793 to 8,193
rows, Qwen3-0.6B heads: ~470,000 row-heads): the plan takes 320-row chunks (764
workgroups of 768 resident) for binary16 and Q8_0 and 1,024-row chunks (504 of 512) for
f32, so the chunks of one entry end at different rows and the last chunk of each is
short.  Attention follows [MINFER-11] §3.2.4 (every
query attends to its window), explicit windows [MINFER-13] §2.2 (a query's cells are a
list of runs); outputs within max-abs 1e-4 / max-rel 1e-5 of the oracle."""
import numpy as np
import pytest

from tests import workloads as W
from tests.gpu_util import Pair, assert_close, compare_cache, say

pytestmark = pytest.mark.gpu
KV = pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])
N_PAST = [8192 - 200 * s for s in range(8)]


def filled_pair(kv):
    w = W.QWEN3_BATCH
    p = Pair(len(N_PAST), 1, w.n_head_kv, w.hd_kv, max(N_PAST) + 1, dtype=kv)
    for s, n in enumerate(N_PAST):
        for ci, r0 in enumerate(range(0, n, 4096)):
            r1 = min(n, r0 + 4096)
            k, v = W.fill_rows(w, s, 0, ci, r1 - r0)
            p.append(0, [s] * (r1 - r0), np.arange(r0, r1), None, 0, 0,
                     k.reshape(r1 - r0, w.n_head_kv, w.hd_kv),
                     v.reshape(r1 - r0, w.n_head_kv, w.hd_kv), w.base, w.freq_scale, w.style)
    seqs = np.arange(len(N_PAST), dtype=np.int32)
    lens = np.array(N_PAST, np.int32)
    q, k, v = W.decode_qkv(w, len(N_PAST), 0, 0)
    qd, qo = p.append(0, seqs, lens, q, w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
    return w, p, seqs, lens, qd, qo


@KV
def test_position_windows(kv):
    say(f"one-round decode, position windows, kv={kv}")
    w, p, seqs, lens, qd, qo = filled_pair(kv)
    got, want = p.decode(0, seqs, lens, qd, qo, w.n_head, w.hd, w.scale)
    assert_close(got, want, "one-round decode")
    for s in range(len(seqs)):
        compare_cache(p.g, p.o, s, 0, "one-round decode")
    p.close()


@KV
def test_explicit_runs(kv):
    """The same windows as two runs each, the later half first: the plan counts chunks
    per run."""
    say(f"one-round decode, explicit runs, kv={kv}")
    w, p, seqs, lens, qd, qo = filled_pair(kv)
    runs = [[((int(x) + 1) // 2, int(x) + 1 - (int(x) + 1) // 2), (0, (int(x) + 1) // 2)]
            for x in lens]
    got, want = p.decode_runs(0, seqs, runs, qd, qo, w.n_head, w.hd, w.scale)
    assert_close(got, want, "one-round decode over runs")
    ref, _ = p.decode(0, seqs, lens, qd, qo, w.n_head, w.hd, w.scale)
    assert_close(got, ref, "runs against position windows on the GPU")
    p.close()
