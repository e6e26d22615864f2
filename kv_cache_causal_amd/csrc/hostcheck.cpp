// Host-only shim over validate.cpp and plan.cpp, built with g++ into
// libkvc_hostcheck.so.  It lets the CPU test suite drive every argument check and every
// launch-planning decision of the library without HIP or a GPU; the library itself calls
// the same functions from kvc_api.cpp.
#include <algorithm>
#include <cstring>
#include <string>

#include "plan.hpp"
#include "rope_consts.hpp"
#include "validate.hpp"

namespace {
thread_local std::string g_msg;

kvc::Geometry geom(const int32_t *g5)
{
    kvc::Geometry g;
    g.n_seq = g5[0];
    g.n_layer = g5[1];
    g.n_head_kv = g5[2];
    g.hd_kv = g5[3];
    g.capacity = g5[4];
    return g;
}
}  // namespace

extern "C" {

const char *hc_last_message(void) { return g_msg.c_str(); }

int hc_check_alloc(int32_t n_seq, int32_t n_layer, int32_t n_head_kv, int32_t hd_kv,
                   int32_t capacity, int32_t dtype)
{
    return kvc::check_alloc(n_seq, n_layer, n_head_kv, hd_kv, capacity, dtype, g_msg);
}

int hc_check_append(const int32_t *g5, int32_t layer, int32_t nt, const int32_t *seq_ids,
                    const int32_t *pos, const void *q, int32_t n_head, int32_t hd, const void *k,
                    const void *v, float freq_base, float freq_scale, int32_t style)
{
    return kvc::check_append(geom(g5), layer, nt, seq_ids, pos, q, n_head, hd, k, v, freq_base,
                             freq_scale, style, g_msg);
}

int hc_check_prefill(const int32_t *g5, int32_t seq, int32_t layer, int32_t nt,
                     const int32_t *pos, const void *q, int32_t n_head, int32_t hd, float scale,
                     const void *out)
{
    return kvc::check_prefill(geom(g5), seq, layer, nt, pos, q, n_head, hd, scale, out, g_msg);
}

int hc_check_decode(const int32_t *g5, int32_t layer, int32_t n_seq, const int32_t *seq_ids,
                    const int32_t *pos, const void *q, int32_t n_head, int32_t hd, float scale,
                    const void *out)
{
    return kvc::check_decode(geom(g5), layer, n_seq, seq_ids, pos, q, n_head, hd, scale, out,
                             g_msg);
}

int hc_check_decode_runs(const int32_t *g5, int32_t layer, int32_t n_seq, const int32_t *seq_ids,
                         const int32_t *run_off, const int32_t *run_start, const int32_t *run_len,
                         const void *q, int32_t n_head, int32_t hd, float scale, const void *out)
{
    return kvc::check_decode_runs(geom(g5), layer, n_seq, seq_ids, run_off, run_start, run_len, q,
                                  n_head, hd, scale, out, g_msg);
}

int hc_check_qkv(const int32_t *g5, int32_t layer, int32_t nt, const int32_t *seq_ids,
                 const int32_t *pos, const void *x, int32_t d_model, const void *wq,
                 const void *bq, const void *wk, const void *bk, const void *wv, const void *bv,
                 int32_t n_head, int32_t hd, const void *q_out, float freq_base,
                 float freq_scale, int32_t style)
{
    return kvc::check_qkv(geom(g5), layer, nt, seq_ids, pos, x, d_model, wq, bq, wk, bk, wv, bv,
                          n_head, hd, q_out, freq_base, freq_scale, style, g_msg);
}

// Prefill plan: meta[0..8] = GB, TQ, n_qtiles, n_hsub, KT, units_per_hgroup, max_seg,
// number of unit ints, contiguous positions (0/1); the unit table goes to units (at most
// cap ints).  Returns 0, or 1 if cap is too small.
int hc_plan_prefill(const int32_t *pos, int32_t nt, int32_t n_head, int32_t n_head_kv,
                    int32_t hd_kv, int32_t force_seg, int32_t *meta, int32_t *units, int32_t cap)
{
    const kvc::PrefillPlan pl = kvc::plan_prefill(pos, nt, n_head, n_head_kv, hd_kv, force_seg);
    const int32_t m[9] = {pl.GB, pl.TQ, pl.n_qtiles, pl.n_hsub, pl.KT, pl.units_per_hgroup,
                          pl.max_seg, (int32_t)pl.units.size(), pl.contiguous ? 1 : 0};
    std::memcpy(meta, m, sizeof(m));
    if ((int64_t)pl.units.size() > cap) return 1;
    std::copy(pl.units.begin(), pl.units.end(), units);
    return 0;
}

int64_t hc_max_part_bytes(void) { return kvc::kMaxPartBytes; }

// The constants of the RoPE table's exact evaluation: the digits of 2/pi (words) and
// pi/2, ln 2 as hi/lo pairs (dd = {pi/2 hi, lo, ln 2 hi, lo}).  Returns the word count.
int32_t hc_rope_consts(uint32_t *words, double *dd)
{
    static const uint32_t w[KVC_TWO_OVER_PI_NWORDS] = {KVC_TWO_OVER_PI_WORDS};
    std::copy(w, w + KVC_TWO_OVER_PI_NWORDS, words);
    const double d[4] = {KVC_PI_2_HI, KVC_PI_2_LO, KVC_LN2_HI, KVC_LN2_LO};
    std::copy(d, d + 4, dd);
    return KVC_TWO_OVER_PI_NWORDS;
}

int64_t hc_decode_chunk_rows(int64_t work, int32_t br, int32_t hpb, int64_t forced)
{
    return kvc::decode_chunk_rows(work, br, hpb, forced);
}

int64_t hc_decode_one_round_rows(const int64_t *len, int32_t m, int32_t n_head_kv, int32_t hpb,
                                 int64_t slots, int32_t br, int64_t rows, int32_t excess_pct)
{
    return kvc::decode_one_round_rows(len, m, n_head_kv, hpb, slots, br, rows, excess_pct);
}

int32_t hc_decode_one_round_excess(int32_t kv_fmt) { return kvc::decode_one_round_excess(kv_fmt); }

}  // extern "C"
