"""Seeded random sweep over geometries, formats, RoPE styles and call patterns, each
case checked against the oracle through the C ABI: cache bits after appends at random
(non-repeating) positions, prefill over random positions, decode over random windows and
over random explicit runs, and the fused projection step.  The fixed seeds make every
case reproducible; each case prints its parameters first."""
import numpy as np
import pytest

from tests.gpu_util import Pair, assert_bitwise, assert_close, compare_cache, dev, say

pytestmark = pytest.mark.gpu

HD_KV = [16, 32, 64, 128, 256]
HD_KV_BETWEEN = [80, 96, 112, 160, 192]   # f32 and binary16 regions only
GROUPS = [1, 2, 3, 4, 7, 8]


def case(seed, dims=HD_KV):
    rng = np.random.default_rng(10_000 + seed)
    hdk = int(rng.choice(dims))
    nkv = int(rng.choice([1, 2, 4, 8] if hdk <= 128 else [1, 2]))
    g = int(rng.choice(GROUPS))
    hd = min(256, hdk + 2 * int(rng.integers(0, 3)) * int(rng.integers(0, 2)))   # sometimes > hd_kv
    fmts = [0, 1] + ([2] if hdk % 32 == 0 and (hdk & (hdk - 1)) == 0 else [])
    return dict(n_seq=int(rng.integers(1, 4)), n_layer=int(rng.integers(1, 3)), nkv=nkv,
                nh=nkv * g, hd=hd, hdk=hdk, cap=int(rng.integers(1, 1500)),
                kv=int(rng.choice(fmts)), style=int(rng.integers(0, 3)), rng=rng)


@pytest.mark.parametrize("seed", range(200))
def test_random_case(seed):
    run_case(seed, case(seed))


@pytest.mark.parametrize("seed", range(200, 260))
def test_random_case_between_dims(seed):
    """The same sweep over the kv head dims between the powers of two."""
    run_case(seed, case(seed, HD_KV_BETWEEN))


def run_case(seed, c):
    rng = c.pop("rng")
    say(f"random case {seed}: " + ", ".join(f"{k}={v}" for k, v in c.items()))
    n_seq, n_layer, nkv, nh, hd, hdk, cap = (c[k] for k in ("n_seq", "n_layer", "nkv", "nh", "hd",
                                                             "hdk", "cap"))
    p = Pair(n_seq, n_layer, nkv, hdk, cap, dtype=c["kv"])
    layer = int(rng.integers(0, n_layer))
    base = float(rng.choice([1e4, 5e5, 1e6]))
    # Appends: a few calls, each with distinct (seq, pos) pairs, positions anywhere.
    for call in range(3):
        nt = int(rng.integers(1, min(cap * n_seq, 90) + 1))
        flat = rng.choice(cap * n_seq, size=nt, replace=False)
        seqs, pos = (flat // cap).astype(np.int32), (flat % cap).astype(np.int32)
        q = rng.standard_normal((nt, nh, hd)).astype(np.float32)
        k = rng.standard_normal((nt, nkv, hdk)).astype(np.float32)
        v = rng.standard_normal((nt, nkv, hdk)).astype(np.float32)
        p.append(layer, seqs, pos, q, nh, hd, k, v, base, 1.0, c["style"])
    for s in range(n_seq):
        compare_cache(p.g, p.o, s, layer, f"case {seed}")
    scale = float(1.0 / np.sqrt(hd))
    # Prefill on one sequence: random positions (repeats allowed), ragged count.
    nt = int(rng.integers(1, 150))
    pos = rng.integers(0, cap, nt).astype(np.int32)
    q = rng.standard_normal((nt, nh, hd)).astype(np.float32)
    got, want = p.prefill(int(rng.integers(0, n_seq)), layer, pos, dev(q), q, nh, hd, scale)
    assert_close(got, want, f"case {seed} prefill")
    # Decode: random entries and windows.
    n = int(rng.integers(1, 80))
    seqs = rng.integers(0, n_seq, n).astype(np.int32)
    pos = rng.integers(0, cap, n).astype(np.int32)
    q = rng.standard_normal((n, nh, hd)).astype(np.float32)
    got, want = p.decode(layer, seqs, pos, dev(q), q, nh, hd, scale)
    assert_close(got, want, f"case {seed} decode")
    # Explicit windows: 1-4 disjoint runs per entry.
    runs = []
    for _ in range(n):
        k_runs = int(rng.integers(1, 5))
        if cap < 2 * k_runs:
            runs.append([(int(rng.integers(0, cap)), 1)])
            continue
        cuts = np.sort(rng.choice(np.arange(cap + 1), size=2 * k_runs, replace=False))
        rl = [(int(cuts[2 * i]), int(cuts[2 * i + 1] - cuts[2 * i])) for i in range(k_runs)]
        rng.shuffle(rl)
        runs.append(rl)
    got, want = p.decode_runs(layer, seqs, runs, dev(q), q, nh, hd, scale)
    assert_close(got, want, f"case {seed} runs")
    # Fused projection step for a few tokens at fresh positions.
    d = int(rng.choice([16, 64, 200]))
    nt = int(min(int(rng.integers(1, 10)), cap * n_seq))
    flat = rng.choice(cap * n_seq, size=nt, replace=False)
    seqs, pos = (flat // cap).astype(np.int32), (flat % cap).astype(np.int32)
    x = rng.standard_normal((nt, d)).astype(np.float32)
    ws = [rng.standard_normal((r, d)).astype(np.float32) * np.float32(d ** -0.5)
          for r in (nh * hd, nkv * hdk, nkv * hdk)]
    bs = [rng.standard_normal(r).astype(np.float32) if rng.integers(0, 2) else None
          for r in (nh * hd, nkv * hdk, nkv * hdk)]
    qg, qo = p.qkv(layer, seqs, pos, x, (ws[0], bs[0], ws[1], bs[1], ws[2], bs[2]), nh, hd, base,
                   1.0, c["style"])
    assert_bitwise(qg, qo, f"case {seed} fused q")
    for s in range(n_seq):
        compare_cache(p.g, p.o, s, layer, f"case {seed} after fused step")
    p.close()
