// Host-side argument checks (see validate.hpp).
#include "validate.hpp"

#include <algorithm>
#include <cmath>
#include <utility>
#include <vector>

namespace kvc {
namespace {

std::string s(long long x) { return std::to_string(x); }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// The query-head checks shared by every call that takes q.
kvc_status check_heads(const Geometry &g, int32_t n_head, int32_t hd, std::string &msg)
{
    if (n_head <= 0 || n_head % g.n_head_kv != 0) {
        msg = "n_head " + s(n_head) + " is not a positive multiple of n_head_kv " + s(g.n_head_kv);
        return KVC_E_ARG;
    }
    if (hd <= 0 || (hd & 1) || hd > KVC_MAX_HEAD_DIM) {
        msg = "query head dim " + s(hd) + " must be even and in [2, " + s(KVC_MAX_HEAD_DIM) + "]";
        return KVC_E_ARG;
    }
    if (hd < g.hd_kv) {
        msg = "query head dim " + s(hd) + " < kv head dim " + s(g.hd_kv) +
              ": a query head shorter than its key cannot be dotted against it";
        return KVC_E_GEOMETRY;
    }
    return KVC_OK;
}

kvc_status check_positions(const Geometry &g, int32_t n, const int32_t *pos, std::string &msg)
{
    for (int32_t t = 0; t < n; t++) {
        if (pos[t] < 0 || pos[t] >= g.capacity) {
            msg = "position " + s(pos[t]) + " (entry " + s(t) + ") outside [0, capacity " +
                  s(g.capacity) + ")";
            return KVC_E_RANGE;
        }
    }
    return KVC_OK;
}

kvc_status check_seq_ids(const Geometry &g, int32_t n, const int32_t *seq_ids, std::string &msg)
{
    for (int32_t t = 0; t < n; t++) {
        if (seq_ids[t] < 0 || seq_ids[t] >= g.n_seq) {
            msg = "sequence id " + s(seq_ids[t]) + " (entry " + s(t) + ") outside [0, " +
                  s(g.n_seq) + ")";
            return KVC_E_ARG;
        }
    }
    return KVC_OK;
}

}  // namespace

bool supported_kv_head_dim(int32_t hd_kv)
{
    switch (hd_kv) {
    case 16: case 32: case 64: case 80: case 96: case 112: case 128: case 160: case 192:
    case 256: return true;
    default: return false;
    }
}

kvc_status check_alloc(int32_t n_seq, int32_t n_layer, int32_t n_head_kv, int32_t hd_kv,
                       int32_t capacity, int32_t dtype, std::string &msg)
{
    if (n_seq <= 0 || n_layer <= 0 || n_head_kv <= 0) {
        msg = "n_seq, n_layer and n_head_kv must be >= 1";
        return KVC_E_ARG;
    }
    if (!supported_kv_head_dim(hd_kv)) {
        msg = "kv head dim " + s(hd_kv) +
              " unsupported (16, 32, 64, 80, 96, 112, 128, 160, 192 or 256)";
        return KVC_E_ARG;
    }
    if (capacity <= 0 || capacity > KVC_MAX_CAPACITY) {
        msg = "capacity " + s(capacity) + " outside [1, 2^24]";
        return KVC_E_ARG;
    }
    if (dtype != KVC_KV_F32 && dtype != KVC_KV_F16 && dtype != KVC_KV_Q8_0) {
        msg = "unknown region format " + s(dtype);
        return KVC_E_ARG;
    }
    // Q8_0 blocks of 32 run along a row; each must lie within one kv head.  This library's
    // Q8_0 kernels further take only the power-of-two head dims 32 .. 256.
    if (dtype == KVC_KV_Q8_0 && hd_kv % 32 != 0) {
        msg = "a Q8_0 cache needs hd_kv a multiple of 32, got " + s(hd_kv);
        return KVC_E_GEOMETRY;
    }
    if (dtype == KVC_KV_Q8_0 && (hd_kv & (hd_kv - 1)) != 0) {
        msg = "a Q8_0 cache here needs hd_kv of 32, 64, 128 or 256, got " + s(hd_kv);
        return KVC_E_GEOMETRY;
    }
    // Row width and region sizes must fit the 64-bit offsets the kernels use.
    const double bytes = 4.0 * n_seq * n_layer * (double)capacity * n_head_kv * hd_kv;
    if (bytes > 9.0e15) {
        msg = "cache of " + std::to_string(bytes) + " bytes is not addressable";
        return KVC_E_ARG;
    }
    return KVC_OK;
}

kvc_status check_append(const Geometry &g, int32_t layer, int32_t nt, const int32_t *seq_ids,
                        const int32_t *pos, const void *q, int32_t n_head, int32_t hd,
                        const void *k, const void *v, float freq_base, float freq_scale,
                        int32_t style, std::string &msg)
{
    if (layer < 0 || layer >= g.n_layer) {
        msg = "layer " + s(layer) + " outside [0, " + s(g.n_layer) + ")";
        return KVC_E_ARG;
    }
    if (nt < 0) {
        msg = "nt < 0";
        return KVC_E_ARG;
    }
    if (nt == 0) return KVC_OK;
    if (!seq_ids || !pos || !k || !v) {
        msg = "seq_ids, pos, k and v must be non-NULL";
        return KVC_E_ARG;
    }
    if (!aligned16(k) || !aligned16(v) || (q && !aligned16(q))) {
        msg = "device tensors must be 16-byte aligned";
        return KVC_E_ARG;
    }
    if (style != KVC_ROPE_NEOX && style != KVC_ROPE_INTERLEAVED && style != KVC_ROPE_NONE) {
        msg = "unknown rope style " + s(style);
        return KVC_E_ARG;
    }
    if (style != KVC_ROPE_NONE &&
        (!(freq_base > 0.0f) || !std::isfinite(freq_base) || !(freq_scale > 0.0f) ||
         !std::isfinite(freq_scale))) {
        msg = "freq_base and freq_scale must be finite and > 0";
        return KVC_E_ARG;
    }
    if (q) {
        kvc_status st = check_heads(g, n_head, hd, msg);
        if (st != KVC_OK) return st;
    }
    // One pass: ranges, and whether the (sequence, position) keys are strictly
    // increasing (a prompt's positions, a batch of distinct sequences), in which case no
    // key repeats; the error messages come from the per-array checks.
    bool in_range = true, increasing = true;
    int64_t prev = -1;
    for (int32_t t = 0; t < nt; t++) {
        in_range &= seq_ids[t] >= 0 && seq_ids[t] < g.n_seq && pos[t] >= 0 && pos[t] < g.capacity;
        const int64_t key = ((int64_t)seq_ids[t] << 32) | (int64_t)(uint32_t)pos[t];
        increasing &= key > prev;
        prev = key;
    }
    if (!in_range) {
        kvc_status st = check_seq_ids(g, nt, seq_ids, msg);
        if (st != KVC_OK) return st;
        st = check_positions(g, nt, pos, msg);
        if (st != KVC_OK) return st;
    }
    if (increasing) return KVC_OK;
    // Two rows aimed at one (sequence, position) would race on the device.
    auto key = [&](int32_t t) { return ((int64_t)seq_ids[t] << 32) | (int64_t)pos[t]; };
    std::vector<int64_t> keys((size_t)nt);
    for (int32_t t = 0; t < nt; t++) keys[t] = key(t);
    std::sort(keys.begin(), keys.end());
    for (size_t i = 1; i < keys.size(); i++) {
        if (keys[i] == keys[i - 1]) {
            msg = "sequence " + s(keys[i] >> 32) + " position " + s(keys[i] & 0xffffffff) +
                  " appears twice in one append";
            return KVC_E_DUP;
        }
    }
    return KVC_OK;
}

kvc_status check_prefill(const Geometry &g, int32_t seq, int32_t layer, int32_t nt,
                         const int32_t *pos, const void *q, int32_t n_head, int32_t hd,
                         float scale, const void *out, std::string &msg)
{
    if (seq < 0 || seq >= g.n_seq || layer < 0 || layer >= g.n_layer) {
        msg = "seq " + s(seq) + " / layer " + s(layer) + " out of range";
        return KVC_E_ARG;
    }
    if (nt < 0) {
        msg = "nt < 0";
        return KVC_E_ARG;
    }
    if (nt == 0) return KVC_OK;
    if (!pos || !q || !out || !std::isfinite(scale)) {
        msg = "pos, q and out must be non-NULL and scale finite";
        return KVC_E_ARG;
    }
    if (!aligned16(q) || !aligned16(out)) {
        msg = "device tensors must be 16-byte aligned";
        return KVC_E_ARG;
    }
    kvc_status st = check_heads(g, n_head, hd, msg);
    if (st != KVC_OK) return st;
    return check_positions(g, nt, pos, msg);
}

kvc_status check_decode(const Geometry &g, int32_t layer, int32_t n_seq, const int32_t *seq_ids,
                        const int32_t *pos, const void *q, int32_t n_head, int32_t hd,
                        float scale, const void *out, std::string &msg)
{
    if (layer < 0 || layer >= g.n_layer) {
        msg = "layer " + s(layer) + " outside [0, " + s(g.n_layer) + ")";
        return KVC_E_ARG;
    }
    if (n_seq < 0) {
        msg = "n_seq < 0";
        return KVC_E_ARG;
    }
    if (n_seq == 0) return KVC_OK;
    if (!seq_ids || !pos || !q || !out || !std::isfinite(scale)) {
        msg = "seq_ids, pos, q and out must be non-NULL and scale finite";
        return KVC_E_ARG;
    }
    if (!aligned16(q) || !aligned16(out)) {
        msg = "device tensors must be 16-byte aligned";
        return KVC_E_ARG;
    }
    kvc_status st = check_heads(g, n_head, hd, msg);
    if (st != KVC_OK) return st;
    st = check_seq_ids(g, n_seq, seq_ids, msg);
    if (st != KVC_OK) return st;
    return check_positions(g, n_seq, pos, msg);
}

kvc_status check_qkv(const Geometry &g, int32_t layer, int32_t nt, const int32_t *seq_ids,
                     const int32_t *pos, const void *x, int32_t d_model, const void *wq,
                     const void *bq, const void *wk, const void *bk, const void *wv,
                     const void *bv, int32_t n_head, int32_t hd, const void *q_out,
                     float freq_base, float freq_scale, int32_t style, std::string &msg)
{
    if (layer < 0 || layer >= g.n_layer || nt < 0) {
        msg = "layer out of range or nt < 0";
        return KVC_E_ARG;
    }
    if (nt == 0) return KVC_OK;
    if (!x || !wq || !wk || !wv || !q_out || d_model <= 0) {
        msg = "x, wq, wk, wv and q_out must be non-NULL and d_model >= 1";
        return KVC_E_ARG;
    }
    if (d_model % 4 != 0 || d_model > kMaxModelDim) {
        msg = "d_model " + s(d_model) + " must be a multiple of 4, at most " + s(kMaxModelDim);
        return KVC_E_ARG;
    }
    if (!aligned16(x) || !aligned16(wq) || !aligned16(wk) || !aligned16(wv) ||
        !aligned16(q_out) || !aligned4(bq) || !aligned4(bk) || !aligned4(bv)) {
        msg = "x, weights and q_out must be 16-byte aligned (biases 4-byte)";
        return KVC_E_ARG;
    }
    if (nt > kMaxFusedTokens) {
        msg = "the fused step takes at most " + s(kMaxFusedTokens) + " tokens, got " + s(nt);
        return KVC_E_ARG;
    }
    // Shapes the projections need (the append repeats these and adds hd >= hd_kv after
    // the style checks, in that order).
    if (n_head <= 0 || n_head % g.n_head_kv != 0 || hd <= 0 || (hd & 1) ||
        hd > KVC_MAX_HEAD_DIM) {
        msg = "n_head must be a positive multiple of n_head_kv and hd even, 2.." +
              s(KVC_MAX_HEAD_DIM);
        return KVC_E_ARG;
    }
    // Everything the append checks (the projected k and v stand in for its k and v).
    return check_append(g, layer, nt, seq_ids, pos, q_out, n_head, hd, q_out, q_out, freq_base,
                        freq_scale, style, msg);
}

kvc_status check_decode_runs(const Geometry &g, int32_t layer, int32_t n_seq,
                             const int32_t *seq_ids, const int32_t *run_off,
                             const int32_t *run_start, const int32_t *run_len, const void *q,
                             int32_t n_head, int32_t hd, float scale, const void *out,
                             std::string &msg)
{
    if (layer < 0 || layer >= g.n_layer) {
        msg = "layer " + s(layer) + " outside [0, " + s(g.n_layer) + ")";
        return KVC_E_ARG;
    }
    if (n_seq < 0) {
        msg = "n_seq < 0";
        return KVC_E_ARG;
    }
    if (n_seq == 0) return KVC_OK;
    if (!seq_ids || !run_off || !run_start || !run_len || !q || !out || !std::isfinite(scale)) {
        msg = "seq_ids, run_off, run_start, run_len, q and out must be non-NULL and scale finite";
        return KVC_E_ARG;
    }
    if (!aligned16(q) || !aligned16(out)) {
        msg = "device tensors must be 16-byte aligned";
        return KVC_E_ARG;
    }
    kvc_status st = check_heads(g, n_head, hd, msg);
    if (st != KVC_OK) return st;
    st = check_seq_ids(g, n_seq, seq_ids, msg);
    if (st != KVC_OK) return st;
    if (run_off[0] != 0) {
        msg = "run_off[0] must be 0";
        return KVC_E_ARG;
    }
    for (int32_t b = 0; b < n_seq; b++) {
        if (run_off[b + 1] <= run_off[b]) {
            msg = "entry " + s(b) + " has no run (run_off must increase)";
            return KVC_E_ARG;
        }
    }
    const int32_t nr = run_off[n_seq];
    for (int32_t r = 0; r < nr; r++) {
        if (run_len[r] <= 0) {
            msg = "run " + s(r) + " is empty";
            return KVC_E_ARG;
        }
    }
    for (int32_t r = 0; r < nr; r++) {
        if (run_start[r] < 0 || (int64_t)run_start[r] + run_len[r] > g.capacity) {
            msg = "run " + s(r) + " [" + s(run_start[r]) + ", +" + s(run_len[r]) +
                  ") outside the region's " + s(g.capacity) + " rows";
            return KVC_E_RANGE;
        }
    }
    std::vector<std::pair<int32_t, int32_t>> rs;
    for (int32_t b = 0; b < n_seq; b++) {
        rs.clear();
        for (int32_t r = run_off[b]; r < run_off[b + 1]; r++) rs.emplace_back(run_start[r], run_len[r]);
        std::sort(rs.begin(), rs.end());
        for (size_t i = 1; i < rs.size(); i++) {
            if ((int64_t)rs[i - 1].first + rs[i - 1].second > rs[i].first) {
                msg = "entry " + s(b) + ": runs overlap at row " + s(rs[i].first);
                return KVC_E_DUP;
            }
        }
    }
    return KVC_OK;
}

}  // namespace kvc
