"""The fused decode step (kv_qkv_rope_append) on the GPU against the oracle.

"13 · The decode loop and graph reuse" §2.3: a one-token GPU step fuses the q/k/v
matmuls, their biases, the two RoPEs and the two KV stores; §3.4 item 5: fused and
unfused must agree bit for bit.  Every projection value is the f32 nearest to the exact
dot product (plus the bias in f32) on both sides, so the rotated q, the cache rows and
the high-water marks are compared bit for bit -- and against the GPU's own unfused path
(kv_append_rope on the same projections).  Weights and inputs are seeded N(0, 1)-scaled
synthetic values (no trained weights)."""
import numpy as np
import pytest

import kv_cache_causal_amd as kvc
from tests.gpu_util import Pair, assert_bitwise, compare_cache, dev, host, say
from tests.workloads import custom

pytestmark = pytest.mark.gpu


def weights(seed, d, n_head, hd, n_head_kv, hd_kv, bias=True):
    rng = np.random.default_rng(seed)
    s = np.float32(1.0 / np.sqrt(d))
    wq = (rng.standard_normal((n_head * hd, d)) * s).astype(np.float32)
    wk = (rng.standard_normal((n_head_kv * hd_kv, d)) * s).astype(np.float32)
    wv = (rng.standard_normal((n_head_kv * hd_kv, d)) * s).astype(np.float32)
    if not bias:
        return wq, None, wk, None, wv, None
    bq, bk, bv = (rng.standard_normal(r).astype(np.float32) for r in
                  (n_head * hd, n_head_kv * hd_kv, n_head_kv * hd_kv))
    return wq, bq, wk, bk, wv, bv


@pytest.mark.parametrize("nt", [1, 32], ids=["nt1", "nt32"])
def test_qwen3_shape(nt):
    """Qwen3-0.6B geometry (d_model 1024, 16 q / 8 kv heads of 128, no biases), one token
    and a 32-sequence decode batch."""
    say(f"fused qkv qwen3 nt={nt}")
    d, nh, nkv, hd = 1024, 16, 8, 128
    p = Pair(32, 2, nkv, hd, 300)
    ws = weights(300, d, nh, hd, nkv, hd, bias=False)
    x = custom(301, (nt, d))
    seqs = np.arange(nt, dtype=np.int32)
    pos = np.arange(nt, dtype=np.int32) * 7 + 11
    qg, qo = p.qkv(1, seqs, pos, x, ws, nh, hd)
    assert_bitwise(qg, qo, "rotated q")
    for s in range(nt):
        compare_cache(p.g, p.o, int(s), 1, f"fused row of seq {s}")
    p.close()


@pytest.mark.parametrize("kv", [0, 1, 2], ids=["f32", "f16", "q8_0"])
@pytest.mark.parametrize("style", [0, 1, 2], ids=["neox", "interleaved", "none"])
def test_styles_formats_biases(style, kv):
    """Qwen2.5-like geometry with biases (14 q / 2 kv heads of 64, d_model 896), 5 tokens
    over two sequences, every RoPE style and region format."""
    say(f"fused qkv style {style} kv={kv}")
    d, nh, nkv, hd = 896, 14, 2, 64
    p = Pair(2, 1, nkv, hd, 64, dtype=kv)
    ws = weights(310 + style, d, nh, hd, nkv, hd)
    x = custom(311, (5, d))
    seqs, pos = [0, 1, 0, 1, 0], [0, 0, 9, 63, 63]
    qg, qo = p.qkv(0, seqs, pos, x, ws, nh, hd, 1e6, 1.0, style)
    assert_bitwise(qg, qo, "rotated q")
    compare_cache(p.g, p.o, 0, 0, "fused seq 0")
    compare_cache(p.g, p.o, 1, 0, "fused seq 1")
    p.close()


@pytest.mark.parametrize("nh,nkv,hd,hdk,d,nt", [(4, 2, 48, 32, 64, 9), (4, 2, 18, 16, 40, 64),
                                                (16, 1, 256, 256, 512, 3)],
                         ids=["hd_gt_hdkv", "ragged_q_units_64_tokens", "hd256_g16"])
def test_odd_shapes(nh, nkv, hd, hdk, d, nt):
    say(f"fused qkv shape n_head={nh} n_head_kv={nkv} hd={hd} hd_kv={hdk} d={d} nt={nt}")
    p = Pair(1, 1, nkv, hdk, 80)
    ws = weights(320, d, nh, hd, nkv, hdk)
    x = custom(321, (nt, d))
    pos = np.arange(nt, dtype=np.int32)
    qg, qo = p.qkv(0, [0] * nt, pos, x, ws, nh, hd, 1e4, 1.0, 0)
    assert_bitwise(qg, qo, "rotated q")
    compare_cache(p.g, p.o, 0, 0, "fused")
    p.close()


def test_exact_dot_products():
    """Inputs whose exact dot products an f32 or f64 running sum gets wrong (a 1 next to
    +-1e20, wide magnitude ranges): the GPU's values are still the nearest f32."""
    say("fused qkv exactness")
    d, nh, nkv, hd = 256, 2, 1, 32
    rng = np.random.default_rng(330)
    x = (rng.standard_normal((2, d)) * 10.0 ** rng.integers(-8, 9, (2, d))).astype(np.float32)
    x[0, :4] = [1e20, 1.0, -1e20, 0.5]
    wq, bq, wk, bk, wv, bv = weights(331, d, nh, hd, nkv, hd)
    wq[0] = 0.0
    wq[0, :4] = 1.0                       # q value 0 of token 0: exactly 1.5 (+ bias)
    wk = (wk * 10.0 ** rng.integers(-8, 9, wk.shape)).astype(np.float32)
    p = Pair(1, 1, nkv, hd, 8)
    qg, qo = p.qkv(0, [0, 0], [0, 1], x, (wq, bq, wk, bk, wv, bv), nh, hd, 1e4, 1.0, 2)
    assert_bitwise(qg, qo, "q (no rotation)")
    assert qg[0, 0, 0] == np.float32(np.float32(1.5) + bq[0])
    compare_cache(p.g, p.o, 0, 0, "exact k/v")
    p.close()


@pytest.mark.parametrize("nt", [1, 3, 5], ids=["one_token", "three_tokens", "five_tokens"])
def test_rounding_boundaries(nt):
    """Dot products at or within 2^-80 of an f32 rounding boundary (a plain f64 sum cannot
    tell which way they round) and one comfortably inside an f32 interval, with values
    worked out by hand: x = (1, 2^-24, 2^-60, 0, ...) for every token (up to 4 tokens take
    a workgroup per token, more the fp64 matrix-core path)."""
    say(f"fused qkv rounding boundaries nt={nt}")
    d, nh, nkv, hd = 128, 2, 1, 16
    x = np.zeros((nt, d), np.float32)
    x[:, :3] = [1.0, 2.0 ** -24, 2.0 ** -60]
    wq, _, wk, _, wv, _ = weights(350, d, nh, hd, nkv, hd, bias=False)
    rows = {0: ([1, 1, 0], 1.0),                              # 1 + 2^-24: tie -> even (1)
            1: ([1, 1, 2.0 ** -20], 1.0 + 2.0 ** -23),        # tie + 2^-80 -> up
            2: ([-1, -1, -2.0 ** -20], -(1.0 + 2.0 ** -23)),   # mirrored
            3: ([1, 3, 0], 1.0 + 2.0 ** -22),                 # 1 + 3 * 2^-24: tie -> even
            4: ([1, -1, 2.0 ** -20], 1.0 - 2.0 ** -24)}        # inside an f32 interval
    for r, (w3, _) in rows.items():
        wq[r] = 0.0
        wq[r, :3] = w3
    p = Pair(1, 1, nkv, hd, 8)
    qg, qo = p.qkv(0, [0] * nt, list(range(nt)), x, (wq, None, wk, None, wv, None), nh, hd,
                   1e4, 1.0, 2)
    assert_bitwise(qg, qo, "q (no rotation)")
    for t in range(nt):
        for r, (_, want) in rows.items():
            assert qg[t, 0, r] == np.float32(want), (t, r, qg[t, 0, r], want)
    compare_cache(p.g, p.o, 0, 0, "k/v")
    p.close()


def test_fused_equals_unfused_on_the_gpu():
    """kv_append_rope on the (oracle's, bit-identical) projections writes the same cache
    and rotates q the same way as the fused kernel."""
    import torch
    say("fused vs unfused on the gpu")
    d, nh, nkv, hd = 512, 8, 4, 64
    ws = weights(340, d, nh, hd, nkv, hd)
    x = custom(341, (6, d))
    seqs, pos = [0, 1, 2, 0, 1, 2], [5, 5, 5, 6, 6, 6]
    fused = kvc.kv_alloc(3, 1, nkv, hd, 16)
    plain = kvc.kv_alloc(3, 1, nkv, hd, 16)
    qf = torch.empty((6, nh, hd), dtype=torch.float32, device="cuda")
    kvc.kv_qkv_rope_append(fused, 0, seqs, pos, dev(x), *[None if a is None else dev(a) for a in ws],
                           nh, hd, qf, 1e6)
    from oracle import Oracle
    o = Oracle()
    q = dev(o.project(x, ws[0], ws[1]).reshape(6, nh, hd))
    k = dev(o.project(x, ws[2], ws[3]).reshape(6, nkv, hd))
    v = dev(o.project(x, ws[4], ws[5]).reshape(6, nkv, hd))
    kvc.kv_append_rope(plain, 0, seqs, pos, q, nh, hd, k, v, 1e6)
    assert_bitwise(host(qf), host(q), "q")
    for s in range(3):
        fk, fv = kvc.kv_read(fused, s, 0)
        pk, pv = kvc.kv_read(plain, s, 0)
        assert_bitwise(host(fk), host(pk), f"K seq {s}")
        assert_bitwise(host(fv), host(pv), f"V seq {s}")
        assert kvc.kv_seq_len(fused, s, 0) == kvc.kv_seq_len(plain, s, 0) == 7
    fused.close()
    plain.close()


def test_errors_write_nothing():
    import torch
    say("fused qkv errors")
    d, nh, nkv, hd = 64, 2, 1, 32
    ws = weights(350, d, nh, hd, nkv, hd)
    c = kvc.kv_alloc(1, 1, nkv, hd, 8)
    q = torch.full((2, nh, hd), 3.0, device="cuda")
    dws = [dev(a) for a in ws]
    for pos, want in (([1, 1], kvc.E_DUP), ([1, 8], kvc.E_RANGE)):
        with pytest.raises(kvc.KvcError) as e:
            kvc.kv_qkv_rope_append(c, 0, [0, 0], pos, dev(custom(351, (2, d))), *dws, nh, hd, q,
                                   1e6)
        assert e.value.status == want
    k, v = kvc.kv_read(c, 0, 0)
    assert not host(k).any() and not host(v).any() and (host(q) == 3.0).all()
    assert kvc.kv_seq_len(c, 0, 0) == 0
    c.close()
