"""GPU parity on the five workloads, at full size, through the C ABI.

Each test drives the HIP library and the oracle with the same seeded inputs
(tests/workloads.py) and compares: caches, rotated q and high-water marks bit for bit,
attention outputs within the allclose bar of tests/gpu_util.py.  Every output of every
call is compared, including all 4,096 x 16 x 128 values of the batch workload's prefill
(in the benchmark's launch configuration; the oracle takes 10-30 s of host time for it).
"""
import time

import numpy as np
import pytest

from tests import workloads as W
from tests.gpu_util import Pair, assert_close, compare_cache, dev, say

pytestmark = pytest.mark.gpu

# Region formats: f32, the binary16 cache (store rounds to half, attention widens) and
# the Q8_0 cache (store quantizes 32-value blocks, attention dequantizes).
KV = pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])


def fill(pair, w, seq, layer, n_rows, chunk=4096):
    """Pre-fill rows [0, n_rows) of (seq, layer) on both sides (store only, q = None)."""
    for ci, r0 in enumerate(range(0, n_rows, chunk)):
        r1 = min(n_rows, r0 + chunk)
        k, v = W.fill_rows(w, seq, layer, ci, r1 - r0)
        k = k.reshape(r1 - r0, w.n_head_kv, w.hd_kv)
        v = v.reshape(r1 - r0, w.n_head_kv, w.hd_kv)
        pair.append(layer, [seq] * (r1 - r0), np.arange(r0, r1), None, 0, 0, k, v, w.base,
                    w.freq_scale, w.style)


@KV
def test_tiny(kv):
    w = W.TINY
    if kv == 2:
        pytest.skip("Q8_0 blocks need hd_kv a multiple of 32; this workload has hd_kv 16")
    say(f"{w.name} kv={kv}")
    p = Pair(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity, dtype=kv)
    nt = w.extra["prefill"]
    pos = np.arange(nt, dtype=np.int32)
    q, k, v = W.prefill_qkv(w, nt, 0)
    qd, qo = p.append(0, [0] * nt, pos, q, w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
    compare_cache(p.g, p.o, 0, 0, "tiny prefill")
    got, want = p.prefill(0, 0, pos, qd, qo, w.n_head, w.hd, w.scale)
    assert_close(got, want, "tiny prefill out")
    for step in range(w.extra["decode_steps"]):
        ps = [nt + step]
        q, k, v = W.decode_qkv(w, 1, step, 0)
        qd, qo = p.append(0, [0], ps, q, w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
        got, want = p.decode(0, [0], ps, qd, qo, w.n_head, w.hd, w.scale)
        assert_close(got, want, f"tiny decode step {step}")
    compare_cache(p.g, p.o, 0, 0, "tiny after decode")
    p.close()


@KV
def test_qwen25_layer(kv):
    w = W.QWEN25_LAYER
    say(f"{w.name} kv={kv}")
    p = Pair(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity, dtype=kv)
    n_past = w.extra["n_past"]
    fill(p, w, 0, 0, n_past)
    q, k, v = W.decode_qkv(w, 1, 0, 0)
    qd, qo = p.append(0, [0], [n_past], q, w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
    compare_cache(p.g, p.o, 0, 0, "qwen2.5 layer")
    got, want = p.decode(0, [0], [n_past], qd, qo, w.n_head, w.hd, w.scale)
    assert_close(got, want, "qwen2.5 layer decode")
    p.close()


@KV
def test_qwen3_stack(kv):
    w = W.QWEN3_STACK
    say(f"{w.name} kv={kv}")
    p = Pair(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity, dtype=kv)
    nt = w.extra["prefill"]
    pos = np.arange(nt, dtype=np.int32)
    worst = 0.0
    for layer in range(w.n_layer):
        q, k, v = W.prefill_qkv(w, nt, layer)
        qd, qo = p.append(layer, [0] * nt, pos, q, w.n_head, w.hd, k, v, w.base, w.freq_scale,
                          w.style)
        got, want = p.prefill(0, layer, pos, qd, qo, w.n_head, w.hd, w.scale)
        assert_close(got, want, f"qwen3 stack prefill layer {layer}")
    for step in range(w.extra["decode_steps"]):
        ps = [nt + step]
        for layer in range(w.n_layer):
            q, k, v = W.decode_qkv(w, 1, step, layer)
            qd, qo = p.append(layer, [0], ps, q, w.n_head, w.hd, k, v, w.base, w.freq_scale,
                              w.style)
            got, want = p.decode(layer, [0], ps, qd, qo, w.n_head, w.hd, w.scale)
            from tests.gpu_util import ATOL, RTOL
            err = np.abs(got.astype(np.float64) - want)
            assert (err <= ATOL + RTOL * np.abs(want)).all(), (step, layer, err.max())
            worst = max(worst, float(err.max()))
    say(f"  qwen3 stack decode 64 steps x 28 layers: max-abs {worst:.3e}")
    for layer in range(w.n_layer):
        compare_cache(p.g, p.o, 0, layer, "qwen3 stack")
    p.close()


@KV
def test_qwen3_long_context(kv):
    w = W.QWEN3_LONG
    say(f"{w.name} kv={kv}")
    p = Pair(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity, dtype=kv)
    n_past = w.extra["n_past"]
    fill(p, w, 0, 0, n_past, w.extra["fill_chunk"])
    q, k, v = W.decode_qkv(w, 1, 0, 0)
    qd, qo = p.append(0, [0], [n_past], q, w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
    compare_cache(p.g, p.o, 0, 0, "qwen3 long")
    got, want = p.decode(0, [0], [n_past], qd, qo, w.n_head, w.hd, w.scale)
    assert_close(got, want, "qwen3 long decode")
    p.close()


@KV
def test_qwen3_batch(kv):
    w = W.QWEN3_BATCH
    say(f"{w.name} kv={kv}")
    p = Pair(w.n_seq, w.n_layer, w.n_head_kv, w.hd_kv, w.capacity, dtype=kv)
    n_past = W.batch_n_past(w)
    say(f"  n_past {n_past.tolist()}")
    for s in range(w.n_seq):
        fill(p, w, s, 0, int(n_past[s]), w.extra["fill_chunk"])
    # Continuation prefill of 4096 tokens on sequence 0.
    nt = w.extra["prefill"]
    pos = np.arange(n_past[0], n_past[0] + nt, dtype=np.int32)
    q, k, v = W.prefill_qkv(w, nt, 0, 0)
    qd, qo = p.append(0, [0] * nt, pos, q, w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
    t0 = time.time()
    got, want = p.prefill(0, 0, pos, qd, qo, w.n_head, w.hd, w.scale)
    say(f"  prefill of {nt} tokens at {pos[0]}..{pos[-1]}: oracle and GPU done in "
        f"{time.time() - t0:.1f}s")
    assert_close(got, want, f"qwen3 batch prefill (all {nt} tokens)")
    # One decode step for all 32 sequences.
    lens = n_past.copy()
    lens[0] += nt
    q, k, v = W.decode_qkv(w, w.n_seq, 0, 0)
    seqs = np.arange(w.n_seq, dtype=np.int32)
    qd, qo = p.append(0, seqs, lens, q, w.n_head, w.hd, k, v, w.base, w.freq_scale, w.style)
    got, want = p.decode(0, seqs, lens, qd, qo, w.n_head, w.hd, w.scale)
    assert_close(got, want, "qwen3 batch batched decode")
    for s in range(w.n_seq):
        compare_cache(p.g, p.o, s, 0, "qwen3 batch")
    p.close()
