"""A decode step (kv_append_rope of a few tokens + gqa_attn_decode) captured into a HIP
graph and replayed: every replay must give the eager result bit for bit, with eager work
and synchronisation between replays, and match the oracle (output within the attention
tolerance, cache rows bit for bit).  Calls of up to 64 tokens/entries pass their integer
arrays in the kernel arguments and allocate nothing once warm, so they can be captured;
the graph replays the captured positions (the host-side high-water marks are updated only
when the calls are issued)."""
import numpy as np
import pytest

import kv_cache_causal_amd as kvc
from oracle import OracleCache
from tests.gpu_util import assert_bitwise, assert_close, compare_dense_cache, dev, host, say
from tests.workloads import custom

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replay():
    import torch
    say("graph replay of a decode step")
    nkv, hd, nh, cap = 2, 64, 8, 3000
    caches = [kvc.kv_alloc(2, 1, nkv, hd, cap) for _ in range(2)]
    orc = OracleCache(2, 1, nkv, hd, cap)
    k0h = custom(400, (2500, nkv, hd))
    k0 = dev(k0h)
    for c in caches:
        for s in range(2):
            kvc.kv_append_rope(c, 0, [s] * 2500, np.arange(2500), None, 0, 0, k0, k0, 1e6)
    for s in range(2):
        assert orc.append_rope(0, [s] * 2500, np.arange(2500), None, 0, 0, k0h, k0h, 1e6)[0] == 0
    seqs, pos = [0, 1], [2500, 2500]
    kh, vh, qh = custom(401, (2, nkv, hd)), custom(402, (2, nkv, hd)), custom(403, (2, nh, hd))
    k, v, q = dev(kh), dev(vh), dev(qh)
    assert orc.append_rope(0, seqs, pos, None, nh, hd, kh, vh, 1e6)[0] == 0
    st, want_orc = orc.attn_decode(0, seqs, pos, qh, nh, hd, 0.125)
    assert st == 0
    outs = [torch.empty((2, nh, hd), device="cuda") for _ in range(2)]

    def step(c, out):
        kvc.kv_append_rope(c, 0, seqs, pos, None, nh, hd, k, v, 1e6)
        kvc.gqa_attn_decode(c, 0, seqs, pos, q, nh, hd, 0.125, out)

    step(caches[0], outs[0])          # eager reference
    step(caches[1], outs[1])          # warm-up of the captured cache (tables, scratch)
    torch.cuda.synchronize()
    want = host(outs[0])
    want_k, want_v = (host(t) for t in kvc.kv_read(caches[0], 1, 0))
    outs[1].zero_()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(caches[1], outs[1])
    for r in range(4):
        outs[1].fill_(float(r + 1))
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise(host(outs[1]), want, f"replay {r} output")
        assert_close(host(outs[1]), want_orc, f"replay {r} output vs oracle")
        kk, vv = (host(t) for t in kvc.kv_read(caches[1], 1, 0))
        assert_bitwise(kk, want_k, f"replay {r} K")
        assert_bitwise(vv, want_v, f"replay {r} V")
        for s in range(2):
            compare_dense_cache(caches[1], orc, s, 0, f"replay {r} cache vs oracle")
        del junk
    for c in caches:
        c.close()
    orc.close()
