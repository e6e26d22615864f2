// Launch planning shared by the library and the host test shim: how a prefill's query
// tiles are cut into workgroup units, and how long a decode chunk is.  Pure C++ (no HIP),
// so the CPU test suite checks these decisions directly.
#pragma once

#include <cstdint>
#include <vector>

namespace kvc {

// Keys per prefill tile for a kv head dim (the prefill kernel's tile height): K and V
// tiles of 64 keys up to head dim 128 (64 KB of LDS), of 32 keys beyond.
constexpr int prefill_key_tile(int hd_kv) { return hd_kv > 128 ? 32 : 64; }

// A prefill workgroup owns 64 query rows (GB heads of one kv group x TQ tokens: a "query
// tile") and scans key tiles of KT keys.  When there are too few query tiles to fill the
// chip, each query tile's key range is cut into segments of equal tile counts, one
// workgroup each; segments write (m, l, unnormalised O) partials and a merge pass
// combines them by log-sum-exp, as for decode.
constexpr int kUnitInts = 8;   // ints per work unit
struct PrefillPlan {
    int32_t GB = 1, TQ = 64, n_qtiles = 0, n_hsub = 1, KT = 64;
    int32_t units_per_hgroup = 0;  // workgroups per (kv head, head subset)
    int32_t max_seg = 1;           // most segments of any query tile (1: no split)
    bool contiguous = false;       // pos[t] == pos[0] + t for every token
    // Per unit, kUnitInts ints: {query tile, first key tile, key tiles, segment << 16 |
    // segments of the tile, largest and smallest position among the tile's tokens, 0, 0};
    // heavy (late) query tiles first.  Without a split each query tile is one unit that
    // scans key tiles [0, largest position / KT + 1).
    std::vector<int32_t> units;
};

// Most bytes of split-K partial records one prefill may use.
constexpr int64_t kMaxPartBytes = int64_t(256) << 20;

// pos: host [nt] positions of the prompt's tokens.  force_seg: 0 = choose, > 0 = force
// segments of that many key tiles (still grown to respect kMaxPartBytes), < 0 = never
// split.
PrefillPlan plan_prefill(const int32_t *pos, int32_t nt, int32_t n_head, int32_t n_head_kv,
                         int32_t hd_kv, int32_t force_seg);

// Rows per decode chunk (a multiple of br, at least br) for `work` = total window rows x
// kv heads of one call, with hpb kv heads per workgroup; forced > 0 overrides the choice
// (then rounded up to br).
int64_t decode_chunk_rows(int64_t work, int32_t br, int32_t hpb, int64_t forced);

// A chunk length for one launch whose workgroups all run at once: given the lengths of
// the m pieces a launch cuts into chunks (window or run lengths), n_head_kv kv heads in
// workgroups of hpb, `slots` workgroups resident at once on the device and the chunk
// length `rows` of decode_chunk_rows, returns the shortest multiple of br, at least rows,
// with (sum of chunks) x n_head_kv / hpb <= slots, if the work is above the small range
// of decode_chunk_rows (131,072 row-heads) and that length is at most excess_pct percent
// above a perfect balance (total rows x n_head_kv / hpb / slots per workgroup); otherwise
// rows.  decode_one_round_excess gives the limit measured best for a region format.
int64_t decode_one_round_rows(const int64_t *len, int32_t m, int32_t n_head_kv, int32_t hpb,
                              int64_t slots, int32_t br, int64_t rows, int32_t excess_pct);
// 20 for binary16 regions (one round gained up to 15-20% off balance), 15 for f32 and
// Q8_0 (f32 lost 3% at 18%; Q8_0 neither gained nor lost there).
inline int32_t decode_one_round_excess(int32_t kv_fmt) { return kv_fmt == 1 /* binary16 */ ? 20 : 15; }

}  // namespace kvc
