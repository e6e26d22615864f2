"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pins
catch every one: a pin set that a dropped term, a flipped sign, a wrong index or a
transposed operand can slip past is not a pin set.

Each mutant is oracle.c with one textual substitution, built with the oracle's own
flags into a temporary directory.  The real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle as oracle_pkg
from oracle import Oracle
from tests.oracle_pins import ALL_PINS

MUTANTS = {
    # RoPE
    "rotation_sign": ("x[i0] = a - b;", "x[i0] = a + b;"),
    "rotation_swap_cos_sin": ("float a = x0 * cs[i];", "float a = x0 * sn[i];"),
    "neox_pair_index": ("{ i0 = i; i1 = i + half; }", "{ i0 = i; i1 = hd - 1 - i; }"),
    "freq_exponent_drops_2": ("(long double)(2 * i) / (long double)hd",
                              "(long double)(i) / (long double)hd"),
    "freq_scale_ignored": ("(long double)freq_scale / powl", "1.0L / powl"),
    "angle_in_f64": ("cs[i] = (float)cosl((long double)theta);",
                     "cs[i] = (float)cosl((long double)p * (long double)inv[i]);"),
    # Store
    "store_v_from_k": ("off, v + (size_t)t * nkt, nkt);", "off, k + (size_t)t * nkt, nkt);"),
    "store_off_by_one_row": ("const size_t off = (size_t)pos[t] * nkt;",
                             "const size_t off = (size_t)(pos[t] > 0 ? pos[t] - 1 : 0) * nkt;"),
    "k_not_rotated": ("int st = orc_rope(row, 1,", "int st = 0 * orc_rope(row, 0,"),
    "high_water_off": ("if (pos[t] + 1 > *hw) *hw = pos[t] + 1;", "if (pos[t] > *hw) *hw = pos[t];"),
    "no_range_check": ("if (pos[t] < 0 || pos[t] >= c->capacity) return ORC_E_RANGE;\n    int64_t",
                       "if (pos[t] < 0 || pos[t] > c->capacity) return ORC_E_RANGE;\n    int64_t"),
    # Attention
    "gqa_modulo": ("int32_t hk = h / gqa;", "int32_t hk = h % n_head_kv;"),
    "window_drops_current_row": ("int32_t vl = cells ? ncell[t] : pos[t] + 1;",
                                 "int32_t vl = cells ? ncell[t] : (pos[t] > 0 ? pos[t] : 1);"),
    "no_scale": ("float s = dot_f32(hd_kv, qrow, kr) * scale;", "float s = dot_f32(hd_kv, qrow, kr);"),
    "no_max_subtraction": ("float e = expf(scr[j] - mx);", "float e = expf(scr[j]);"),
    "v_from_k_region": ("const float *vr = head_row(vreg,", "const float *vr = head_row(kreg,"),
    "row_stride": ("const size_t off = j * (size_t)nkt + (size_t)hk * hd_kv;",
                   "const size_t off = j * (size_t)hd_kv + (size_t)hk * hd_kv;"),
    "no_normalisation": ("for (int32_t j = 0; j < vl; j++) scr[j] *= inv;", ""),
    # Half-precision cache
    "f16_truncates": ("if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++;", ""),
    "f16_ties_away": ("(rem == 0x1000u && (h & 1u))", "(rem == 0x1000u)"),
    "f16_subnormal_shift": ("const int32_t shift = 14 - e;", "const int32_t shift = 13 - e;"),
    "f16_widen_bias": ("x = sign | ((exp - 15 + 127) << 23) | (man << 13);",
                       "x = sign | ((exp - 16 + 127) << 23) | (man << 13);"),
    "f16_store_skipped": ("for (int32_t i = 0; i < n; i++) d[i] = orc_f32_to_f16(src[i]);",
                          "for (int32_t i = 0; i < n; i++) d[i] = orc_f32_to_f16(src[0]);"),
    # Q8_0 cache
    "q8_ties_to_even": ("const float r = roundf(xb[i] * id);", "const float r = rintf(xb[i] * id);"),
    "q8_truncates": ("const float r = roundf(xb[i] * id);", "const float r = truncf(xb[i] * id);"),
    "q8_divides_by_128": ("const float d = amax / 127.0f;", "const float d = amax / 128.0f;"),
    "q8_reciprocal_of_half_scale": (
        "const float id = d != 0.0f ? 1.0f / d : 0.0f;",
        "const float id = d != 0.0f ? 1.0f / orc_f16_to_f32(orc_f32_to_f16(d)) : 0.0f;"),
    "q8_signed_max": ("const float a = fabsf(xb[i]);", "const float a = xb[i];"),
    "q8_stores_amax": ("b[blk].d = orc_f32_to_f16(d);", "b[blk].d = orc_f32_to_f16(amax);"),
    "q8_dequant_drops_scale": ("out[(size_t)blk * ORC_Q8_BLOCK + i] = d * (float)b[blk].qs[i];",
                               "out[(size_t)blk * ORC_Q8_BLOCK + i] = (float)b[blk].qs[i];"),
    "q8_head_offset_dropped": (
        "orc_q8_dequantize_row((const orc_q8_block *)reg + off / ORC_Q8_BLOCK, hd_kv, buf);",
        "orc_q8_dequantize_row((const orc_q8_block *)reg + j * (size_t)nkt / ORC_Q8_BLOCK, hd_kv, buf);"),
    # Explicit windows
    "runs_start_ignored": ("for (int32_t i = 0; i < run_len[r]; i++) cells[b][j++] = run_start[r] + i;",
                           "for (int32_t i = 0; i < run_len[r]; i++) cells[b][j++] = i;"),
    "runs_v_window_ignored": ("const size_t vrow = cells ? (size_t)cells[j] : (size_t)j;",
                              "const size_t vrow = (size_t)j;"),
    "runs_overlap_allowed": ("if ((int64_t)tmp[2 * (r - 1)] + tmp[2 * (r - 1) + 1] > tmp[2 * r]) st = ORC_E_DUP;",
                             "if ((int64_t)tmp[2 * (r - 1)] + tmp[2 * (r - 1) + 1] > tmp[2 * r] + 1) st = ORC_E_DUP;"),
    "runs_range_off_by_one": ("(int64_t)run_start[r] + run_len[r] > c->capacity) return ORC_E_RANGE;",
                              "(int64_t)run_start[r] + run_len[r] > c->capacity + 1) return ORC_E_RANGE;"),
    # Fused decode projections
    "project_products_rounded": ("acc += (__float128)xr[i] * (__float128)wr[i];",
                                 "acc += (__float128)(xr[i] * wr[i]);"),
    "project_f64_sum": ("__float128 acc = 0;", "double acc = 0;"),
    "project_bias_dropped": ("if (b) y = y + b[j];", "(void)b;"),
    "fused_k_from_wv": ("st = orc_project(x, wk, bk, nt, nkt, d_model, k);",
                        "st = orc_project(x, wv, bk, nt, nkt, d_model, k);"),
    "fused_q_unrotated": ("if (st == ORC_OK) memcpy(q_out, q, sizeof(float) * (size_t)nt * n_head * hd);",
                          "if (st == ORC_OK) orc_project(x, wq, bq, nt, n_head * hd, d_model, q_out);"),
    "q8_store_skipped": ("orc_q8_quantize_row(src, n, (orc_q8_block *)region + off / ORC_Q8_BLOCK);",
                         "(void)src;"),
}


@pytest.fixture(scope="module")
def src():
    with open(oracle_pkg._SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, src, name):
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *oracle_pkg.CFLAGS, str(path), "-o", str(lib), "-lm"], check=True)
    o = Oracle(str(lib))
    failed = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
