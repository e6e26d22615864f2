"""Write rope_near_ties.json: f32 angles whose cos or sin lies unusually close to the
midpoint of two neighbouring f32 values, and RoPE speeds freq_scale / base^(2i/hd) that do.

These are inputs for tests of the correctly rounded RoPE tables ("11 · Attention, vec
ops, and the KV cache" §2.3 and §3.2.2: speed_i = freq_scale / base^(2i/d), angle =
position x speed, each pair rotated by cos and sin of its angle).  An evaluation that is
accurate to a few double-precision ulps rounds such values to f32 the wrong way unless it
detects the near-tie.  The expected table entries are not stored: the tests compute them
with the oracle, and a CPU pin checks the oracle at these inputs against mpmath.

Search: seeded random f32 angles (bit patterns uniform over exponents) and random
(freq_scale, base) pairs; numpy's f64 functions shortlist the candidates within a few
f64 ulps of a midpoint; mpmath at 60 digits measures the true distance, and the closest
are kept.  Run once:  python tests/golden/gen_rope_near_ties.py
"""
import json
import multiprocessing as mp
import os

import mpmath
import numpy as np

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rope_near_ties.json")


def rel_gap(x):
    """|x - nearest f32 midpoint| / |x| for an mpmath value x (60 digits)."""
    f = np.float32(float(x))
    best = None
    for nb in (np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))):
        m = (mpmath.mpf(float(f)) + mpmath.mpf(float(nb))) / 2
        d = abs(x - m)
        best = d if best is None or d < best else best
    return float(best / abs(x))


def shortlist(y):
    """Indices where the f64 values y are within 4 f64 ulps of an f32 midpoint."""
    f = y.astype(np.float32)
    fd = f.astype(np.float64)
    lo = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    margin = np.minimum(np.abs(y - (fd + lo) / 2), np.abs((fd + hi) / 2 - y))
    return np.nonzero(margin <= 4 * np.spacing(np.abs(y)))[0]


def search_angles(args):
    seed, n, e_lo, e_hi = args
    rng = np.random.default_rng(seed)
    e = rng.integers(e_lo, e_hi, n)
    man = rng.integers(0, 1 << 23, n)
    th = ((e + 127).astype(np.uint32) << 23 | man.astype(np.uint32)).view(np.float32)
    out = []
    with mpmath.workdps(60):
        for name, fn, mfn in (("cos", np.cos, mpmath.cos), ("sin", np.sin, mpmath.sin)):
            for i in shortlist(fn(th.astype(np.float64))):
                t = float(th[i])
                out.append((rel_gap(mfn(mpmath.mpf(t))), name, t))
    return out


def search_speeds(args):
    seed, n = args
    rng = np.random.default_rng(seed)
    # hd 4, i = 1: speed = fs / base^(1/2); fs small enough that the angle at position 1
    # (the speed itself) is below 2^-12, where the table's sin entry equals the angle.
    fs = np.exp2(rng.uniform(-20, -13, n)).astype(np.float32)
    base = rng.uniform(2.0, 1.0e6, n).astype(np.float32)
    y = fs.astype(np.float64) / np.sqrt(base.astype(np.float64))
    out = []
    with mpmath.workdps(60):
        for i in shortlist(y):
            x = mpmath.mpf(float(fs[i])) / mpmath.sqrt(mpmath.mpf(float(base[i])))
            out.append((rel_gap(x), float(fs[i]), float(base[i])))
    return out


def main():
    with mp.Pool(8) as pool:
        small = pool.map(search_angles, [(100 + k, 10_000_000, -12, 17) for k in range(40)])
        large = pool.map(search_angles, [(200 + k, 10_000_000, 17, 127) for k in range(20)])
        speeds = pool.map(search_speeds, [(300 + k, 10_000_000) for k in range(40)])
    ang = sorted(set(x for part in small + large for x in part))   # seeds can repeat a value
    spd = sorted(set(x for part in speeds for x in part))
    doc = {
        "what": "inputs for the correctly rounded RoPE table tests (see the generator's docstring)",
        "generator": "tests/golden/gen_rope_near_ties.py",
        "angles": [{"theta_bits": int(np.float32(t).view(np.uint32)), "fn": fn,
                    "rel_gap_to_midpoint": g} for g, fn, t in ang[:40]],
        "speeds": [{"freq_scale_bits": int(np.float32(f).view(np.uint32)),
                    "base_bits": int(np.float32(b).view(np.uint32)), "hd": 4, "i": 1,
                    "rel_gap_to_midpoint": g} for g, f, b in spd[:20]],
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=1)
    print(f"{len(ang)} angle and {len(spd)} speed candidates; kept {len(doc['angles'])} and "
          f"{len(doc['speeds'])}; closest {ang[0][0]:.3g} / {spd[0][0]:.3g}")


if __name__ == "__main__":
    main()
