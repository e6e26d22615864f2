"""The C ABI from a plain C program (tests/c_abi/abi_demo.c, built by build() with gcc
against include/kvc.h and the HIP runtime): no Python binding and no torch in that
process.  It appends a prompt with RoPE, runs its prefill, appends and decodes one more
token, and makes one call that must fail; its outputs are checked against the oracle on
the same inputs (cache rows and rotated q bit for bit, attention within tolerance)."""
import os
import subprocess

import numpy as np
import pytest

from tests.gpu_util import assert_bitwise, assert_close, say
from tests.workloads import custom

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "kv_cache_causal_amd", "lib", "abi_demo")


def test_c_program_matches_the_oracle(tmp_path):
    if not os.path.exists(DEMO):
        pytest.fail("abi_demo is not built: run __graft_entry__.build()")
    from oracle import OracleCache
    import kv_cache_causal_amd as kvc
    nh, hd, nkv, hdk, cap, nt = 14, 64, 2, 64, 300, 150   # Qwen2.5-0.5B heads
    say(f"C program: n_head={nh} hd={hd} n_head_kv={nkv} hd_kv={hdk} capacity={cap} nt={nt}")
    q, k, v = custom(700, (nt, nh, hd)), custom(701, (nt, nkv, hdk)), custom(702, (nt, nkv, hdk))
    q1, k1, v1 = custom(703, (1, nh, hd)), custom(704, (1, nkv, hdk)), custom(705, (1, nkv, hdk))
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([nh, hd, nkv, hdk, cap, nt], np.int32).tobytes())
        for a in (q, k, v, q1, k1, v1):
            f.write(np.ascontiguousarray(a, np.float32).tobytes())
    r = subprocess.run([DEMO, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr

    raw = np.fromfile(outp, np.uint8)
    sizes = [nt * nh * hd, nt * nh * hdk, nh * hd, nh * hdk, (nt + 1) * nkv * hdk,
             (nt + 1) * nkv * hdk]
    parts, off = [], 0
    for n in sizes:
        parts.append(raw[off:off + 4 * n].view(np.float32))
        off += 4 * n
    status, said = raw[off:off + 8].view(np.int32)
    gq, gout, gq1, gout1, gK, gV = parts

    o = OracleCache(1, 1, nkv, hdk, cap)
    pos = np.arange(nt, dtype=np.int32)
    st, oq = o.append_rope(0, np.zeros(nt, np.int32), pos, q, nh, hd, k, v, 1e6, 1.0, 0)
    assert st == 0
    st, oout = o.attn_prefill(0, 0, pos, oq, nh, hd, 0.125)
    assert st == 0
    st, oq1 = o.append_rope(0, [0], [nt], q1, nh, hd, k1, v1, 1e6, 1.0, 0)
    assert st == 0
    st, oout1 = o.attn_decode(0, [0], [nt], oq1, nh, hd, 0.125)
    assert st == 0

    assert_bitwise(gq.reshape(oq.shape), oq, "rotated prompt q")
    assert_bitwise(gq1.reshape(oq1.shape), oq1, "rotated decode q")
    assert_bitwise(gK.reshape(nt + 1, -1), o.k(0, 0)[:nt + 1], "K rows")
    assert_bitwise(gV.reshape(nt + 1, -1), o.v(0, 0)[:nt + 1], "V rows")
    assert_close(gout.reshape(oout.shape), oout, "prefill from C")
    assert_close(gout1.reshape(oout1.shape), oout1, "decode from C")
    assert status == kvc.E_RANGE and said == 1
    o.close()
