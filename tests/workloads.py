"""Seeded synthetic inputs and the five workload shapes.

This module only draws random numbers and names shapes; it holds none of the
attention, RoPE or cache arithmetic.  Both the oracle side and the HIP side of every
test (and the benchmark) take their inputs from here, so the two see identical bytes.

Every tensor is f32 N(0, 1) from numpy's PCG64.  The seed of a tensor is
SeedSequence(entropy=1000 + workload id, spawn_key=tag), where the tag names the
tensor's role (e.g. ("fill", seq, layer, chunk) or ("decode", step, layer)), so any one
tensor can be regenerated without drawing the others.

Workload shapes (the pages' model geometries: Qwen2.5-0.5B has 14 query heads of 64
over 2 KV heads; Qwen3-0.6B has 16 query heads of 128 over 8 KV heads, 28 layers,
a 40,960-token context; both use NEOX RoPE with base 1e6):

  TINY          1 layer, 2 q heads, 1 kv head, hd = hd_kv = 16; prefill of 8 tokens,
                then 4 decode steps.  Capacity 8 + 512.
  QWEN25_LAYER  one Qwen2.5-0.5B-shaped layer; rows 0..510 cached, one decode at 511.
                Capacity 511 + 512.
  QWEN3_STACK   28 Qwen3-0.6B-shaped layers; prefill of 511 tokens per layer, then 64
                decode steps, each appending one row per layer.  Capacity 511 + 512.
  QWEN3_LONG    one Qwen3-0.6B-shaped layer with 32,767 rows cached (context 40,960),
                one decode at position 32,767.
  QWEN3_BATCH   32 Qwen3-0.6B-shaped sequences with n_past drawn uniformly from
                [128, 8192]; a 4,096-token continuation prefill on sequence 0, then
                one decode step for all 32.  Capacity 8192 + 4096 + 512.

The integer id of each workload (1..5) only seeds its tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NEOX, INTERLEAVED, NONE = 0, 1, 2


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    n_seq: int
    n_layer: int
    n_head: int
    n_head_kv: int
    hd: int
    hd_kv: int
    capacity: int
    base: float = 1.0e6
    freq_scale: float = 1.0
    style: int = NEOX
    extra: dict = field(default_factory=dict)

    @property
    def nkt(self) -> int:
        return self.n_head_kv * self.hd_kv

    @property
    def scale(self) -> float:
        """Attention scale the models pass (one over the square root of the query head
        dim, as an f32), stated as literals per head dim."""
        return _SCALE[self.hd]


_SCALE = {16: 0.25, 64: 0.125, 128: float(np.float32(0.08838834764831845))}


TINY = Workload(1, "tiny", 1, 1, 2, 1, 16, 16, 8 + 512, extra=dict(prefill=8, decode_steps=4))
QWEN25_LAYER = Workload(2, "qwen2.5-0.5b-layer", 1, 1, 14, 2, 64, 64, 511 + 512, extra=dict(n_past=511))
QWEN3_STACK = Workload(3, "qwen3-0.6b-stack", 1, 28, 16, 8, 128, 128, 511 + 512,
                       extra=dict(prefill=511, decode_steps=64))
QWEN3_LONG = Workload(4, "qwen3-0.6b-long", 1, 1, 16, 8, 128, 128, 40960,
                      extra=dict(n_past=32767, fill_chunk=4096))
QWEN3_BATCH = Workload(5, "qwen3-0.6b-batch", 32, 1, 16, 8, 128, 128, 8192 + 4096 + 512,
                       extra=dict(prefill=4096, past_lo=128, past_hi=8192, fill_chunk=4096))

ALL = {w.cid: w for w in (TINY, QWEN25_LAYER, QWEN3_STACK, QWEN3_LONG, QWEN3_BATCH)}


def rng(cid: int, *tag: int) -> np.random.Generator:
    """Generator for one tensor of workload `cid`, identified by an integer tag."""
    ss = np.random.SeedSequence(entropy=1000 + cid, spawn_key=tuple(int(t) for t in tag))
    return np.random.Generator(np.random.PCG64(ss))


def normal(cid: int, shape, *tag: int) -> np.ndarray:
    """f32 N(0, 1) tensor of the given shape, seeded by (cid, tag)."""
    return rng(cid, *tag).standard_normal(size=shape, dtype=np.float32)


# Tag roots (first element of a tag) so roles never collide.
T_FILL_K, T_FILL_V, T_PRE_Q, T_PRE_K, T_PRE_V, T_DEC_Q, T_DEC_K, T_DEC_V, T_NPAST = range(1, 10)


def batch_n_past(w: Workload = QWEN3_BATCH) -> np.ndarray:
    """Ragged cached lengths of the batch workload, uniform in [lo, hi] inclusive."""
    g = rng(w.cid, T_NPAST)
    return g.integers(w.extra["past_lo"], w.extra["past_hi"], size=w.n_seq,
                      endpoint=True).astype(np.int32)


def fill_rows(w: Workload, seq: int, layer: int, chunk: int, nrows: int):
    """K and V rows ([nrows][nkt]) that pre-fill a cache before the timed work."""
    k = normal(w.cid, (nrows, w.nkt), T_FILL_K, seq, layer, chunk)
    v = normal(w.cid, (nrows, w.nkt), T_FILL_V, seq, layer, chunk)
    return k, v


def prefill_qkv(w: Workload, nt: int, layer: int, seq: int = 0):
    q = normal(w.cid, (nt, w.n_head, w.hd), T_PRE_Q, layer, seq)
    k = normal(w.cid, (nt, w.n_head_kv, w.hd_kv), T_PRE_K, layer, seq)
    v = normal(w.cid, (nt, w.n_head_kv, w.hd_kv), T_PRE_V, layer, seq)
    return q, k, v


def decode_qkv(w: Workload, n: int, step: int, layer: int):
    q = normal(w.cid, (n, w.n_head, w.hd), T_DEC_Q, step, layer)
    k = normal(w.cid, (n, w.n_head_kv, w.hd_kv), T_DEC_K, step, layer)
    v = normal(w.cid, (n, w.n_head_kv, w.hd_kv), T_DEC_V, step, layer)
    return q, k, v


def custom(seed: int, shape) -> np.ndarray:
    """f32 N(0, 1) for small hand-built test shapes (entropy 7000 + seed)."""
    ss = np.random.SeedSequence(entropy=7000 + int(seed))
    return np.random.Generator(np.random.PCG64(ss)).standard_normal(size=shape,
                                                                    dtype=np.float32)


def custom_positions(seed: int, n: int, lo: int, hi: int, unique: bool = True) -> np.ndarray:
    """n positions in [lo, hi) (distinct when `unique`), seeded; for ragged edge cases."""
    ss = np.random.SeedSequence(entropy=8000 + int(seed))
    g = np.random.Generator(np.random.PCG64(ss))
    if unique:
        return np.sort(g.choice(np.arange(lo, hi, dtype=np.int64), size=n,
                                replace=False)).astype(np.int32)
    return g.integers(lo, hi, size=n).astype(np.int32)
