// Launch planning: prefill work units and decode chunk length (see plan.hpp).
#include "plan.hpp"

#include <algorithm>

namespace kvc {

PrefillPlan plan_prefill(const int32_t *pos, int32_t nt, int32_t n_head, int32_t n_head_kv,
                         int32_t hd_kv, int32_t force_seg)
{
    PrefillPlan pl;
    const int G = n_head / n_head_kv;
    // Heads per workgroup: the largest power of two <= min(G, 4); tokens fill the rest.
    while (pl.GB * 2 <= G && pl.GB * 2 <= 4) pl.GB *= 2;
    pl.TQ = 64 / pl.GB;
    pl.n_hsub = (G + pl.GB - 1) / pl.GB;
    pl.n_qtiles = (nt + pl.TQ - 1) / pl.TQ;
    pl.KT = prefill_key_tile(hd_kv);
    pl.units_per_hgroup = pl.n_qtiles;
    pl.contiguous = true;
    for (int t = 1; t < nt && pl.contiguous; t++) pl.contiguous = pos[t] == pos[0] + t;
    // Key tiles of each query tile, up to its largest position.
    std::vector<int32_t> tiles(pl.n_qtiles), qmax(pl.n_qtiles), qmin(pl.n_qtiles);
    int64_t total = 0;
    for (int q = 0; q < pl.n_qtiles; q++) {
        int32_t kmax = 0, kmin = 0x7fffffff;
        for (int t = q * pl.TQ; t < std::min(nt, (q + 1) * pl.TQ); t++) {
            kmax = std::max(kmax, pos[t]);
            kmin = std::min(kmin, pos[t]);
        }
        qmax[q] = kmax;
        qmin[q] = kmin;
        tiles[q] = kmax / pl.KT + 1;
        total += tiles[q];
    }
    auto push_unit = [&](int q, int32_t k0, int32_t nk, int32_t sg, int32_t nseg) {
        const int32_t u[kUnitInts] = {q, k0, nk, (sg << 16) | nseg, qmax[q], qmin[q], 0, 0};
        pl.units.insert(pl.units.end(), u, u + kUnitInts);
    };
    auto whole_tiles = [&]() {   // one unit per query tile, heavy (late) tiles first
        pl.units.clear();
        for (int q = pl.n_qtiles - 1; q >= 0; q--) push_unit(q, 0, tiles[q], 0, 1);
        pl.units_per_hgroup = pl.n_qtiles;
        return pl;
    };
    const int64_t hgroups = (int64_t)n_head_kv * pl.n_hsub;
    // Two resident workgroups per CU: 512 query tiles fill the chip without a split.
    constexpr int64_t kFill = 512;
    if (force_seg < 0 || (force_seg == 0 && hgroups * pl.n_qtiles >= kFill)) return whole_tiles();
    // Segment length: the tiles spread over about kFill units, but no fewer than 3 per
    // unit, so a unit's start-up (query load, first tile fetch, record write) is spread
    // over a few tiles.
    int64_t seg_tiles = force_seg > 0 ? force_seg
                      : std::max<int64_t>(3, (total * hgroups + kFill - 1) / kFill);
    // The partial records take max_seg x nt x n_head x (hd_kv + 4) floats.  A query tile
    // with far more key tiles than the rest (one late position among early ones) could
    // need hundreds of records per query row, so segments grow until they fit the cap.
    const int64_t rec_bytes = (int64_t)nt * n_head * (hd_kv + 4) * (int64_t)sizeof(float);
    const int64_t max_recs = std::max<int64_t>(1, kMaxPartBytes / rec_bytes);
    const int64_t tiles_max = *std::max_element(tiles.begin(), tiles.end());
    seg_tiles = std::max<int64_t>(seg_tiles, (tiles_max + max_recs - 1) / max_recs);
    int32_t max_seg = 1;
    for (int q = 0; q < pl.n_qtiles; q++)
        max_seg = std::max<int32_t>(max_seg, (int32_t)((tiles[q] + seg_tiles - 1) / seg_tiles));
    if (max_seg == 1) return whole_tiles();   // every query tile is one segment already
    pl.max_seg = max_seg;
    pl.units.clear();
    for (int q = pl.n_qtiles - 1; q >= 0; q--) {   // heavy (late) query tiles first
        const int32_t nseg = (int32_t)((tiles[q] + seg_tiles - 1) / seg_tiles);
        for (int32_t sg = 0; sg < nseg; sg++) {
            const int32_t k0 = (int32_t)(sg * seg_tiles);
            push_unit(q, k0, (int32_t)std::min<int64_t>(seg_tiles, tiles[q] - k0), sg, nseg);
        }
    }
    pl.units_per_hgroup = (int32_t)(pl.units.size() / kUnitInts);
    return pl;
}

namespace {
constexpr int64_t kDecodeLargeWork = 2048 * 512;   // ~2048 workgroups of >= 512 rows
constexpr int64_t kDecodeSmallWork = 131072;       // up to here: ~512 short chunks
}  // namespace

int64_t decode_chunk_rows(int64_t work, int32_t br, int32_t hpb, int64_t forced)
{
    // A workgroup streams its chunk in steps of br rows, each step a memory round trip,
    // so a chunk of many steps is latency-bound unless many workgroups run.  Large work:
    // ~2048 workgroups (8 per CU) and at least 512 rows per chunk, so the per-chunk
    // overheads (query load, merges, partial record, merge pass) stay small next to the
    // stream.  Small work (a few 100 K row-heads, e.g. one layer's decode at a few
    // hundred positions): chunks down to one step, aiming at ~512 workgroups, so the call
    // costs two short launches instead of one long chain of dependent loads.
    int64_t rows = forced;
    if (rows <= 0) {
        if (work > kDecodeLargeWork) rows = work / 2048;
        else if (work > kDecodeSmallWork) rows = 512;
        else rows = work / 512;
        // A workgroup of hpb kv heads gives each head 1/hpb of its waves: chunks 1/hpb as
        // long keep the rows per wave, and the workgroup count, of one head per workgroup.
        rows /= std::max<int32_t>(1, hpb);
    }
    return std::max<int64_t>(br, (rows + br - 1) / br * br);
}

int64_t decode_one_round_rows(const int64_t *len, int32_t m, int32_t n_head_kv, int32_t hpb,
                              int64_t slots, int32_t br, int64_t rows, int32_t excess_pct)
{
    // With the chunks of decode_chunk_rows (512 rows, or ~2048 workgroups), a launch of
    // more than small work runs in several rounds of resident workgroups, and the last
    // round leaves part of the device idle.  One round of chunks that fill the device and
    // are about equally long keeps every resident workgroup streaming to the end.
    int64_t total = 0, longest = 0;
    for (int32_t i = 0; i < m; i++) {
        total += len[i];
        longest = std::max(longest, len[i]);
    }
    if (m <= 0 || slots <= 0 || br <= 0 || total * n_head_kv <= kDecodeSmallWork) return rows;
    const int64_t blocks = n_head_kv / std::max<int32_t>(1, hpb);   // head blocks per chunk
    auto workgroups = [&](int64_t r) {
        int64_t c = 0;
        for (int32_t i = 0; i < m; i++) c += (len[i] + r - 1) / r;
        return c * blocks;
    };
    int64_t lo = (rows + br - 1) / br, hi = std::max(lo, (longest + br - 1) / br);
    if (workgroups(hi * br) > slots) return rows;   // no chunk length fits one round
    while (lo < hi) {   // workgroups(r) does not grow with r
        const int64_t mid = lo + (hi - lo) / 2;
        if (workgroups(mid * br) <= slots) hi = mid;
        else lo = mid + 1;
    }
    const int64_t r = lo * br;
    if (r * slots * 100 > total * blocks * (100 + excess_pct)) return rows;   // off balance
    return r;
}

}  // namespace kvc
