// Launch interface between the C ABI (kvc_api.cpp) and the gfx950 kernels.
// Each launcher checks nothing itself: kvc_api.cpp validates every argument first and
// hands over device pointers that the kernels' index arithmetic stays inside.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan.hpp"

namespace kvc {

// Cache layout: one region per (seq, layer), K and V alike, `region_bytes` apart, each
// holding rows = capacity rounded up to a multiple of kRegionRowAlign rows of
// nkt = n_head_kv * hd_kv values:
//   kFmtF32, kFmtF16: [rows][nkt] f32 or binary16 values;
//   kFmtQ8:           [rows][nkt] int8 codes, then at byte `scale_off` (= rows * nkt)
//                     [n_head_kv][rows / 4][hd_kv / 32][4] binary16 block scales (Q8_0:
//                     32 values per block, value = scale * code).  Head-major and
//                     interleaved by row quads, so the scales of one block of one kv
//                     head for 4 consecutive rows (4p .. 4p+3) are 8 contiguous bytes.
// Rows at or past the capacity stay zero and are never inside a window; they let the
// prefill kernel load whole key tiles unconditionally.
constexpr int kRegionRowAlign = 64;
enum KvFmt : int32_t { kFmtF32 = 0, kFmtF16 = 1, kFmtQ8 = 2 };
constexpr int kQ8Block = 32;

// Index (in binary16 units from the scales' start) of the scale of value j of row `row`
// of a Q8_0 region with `rows` rows (a multiple of 4).
__host__ __device__ inline int64_t q8_scale_index(int64_t row, int32_t j, int32_t hd_kv,
                                                  int64_t rows)
{
    const int32_t h = j / hd_kv;
    const int32_t blk = (j - h * hd_kv) / kQ8Block;
    return (((int64_t)h * (rows >> 2) + (row >> 2)) * (hd_kv / kQ8Block) + blk) * 4 + (row & 3);
}

// ---- RoPE cos/sin table: tab[p][i] = (cos, sin) of f32(p) * speed_i, p < rows ---------
// Every entry is the correctly rounded f32; exact = true skips the certified f64 fast
// path and evaluates every entry in double-double (tests of that path).
hipError_t launch_rope_table(float2 *tab, int32_t rows, int32_t hd, float freq_base,
                             float freq_scale, bool exact, hipStream_t s);

// Kernel arguments cost host time at every launch: on MI355X a launch with 16 bytes of
// arguments took 2.6 us of host time, one with 816 bytes 3.8 us.  The arrays a call passes
// in the arguments therefore come in two capacities, and a call with up to kSmallInline
// tokens or entries launches kernels whose arguments hold only that many.
constexpr int kSmallInline = 8;

// ---- K1: RoPE(q, k) + in-place K/V row store ------------------------------------------
// Up to kInlineTokens positions / sequence ids ride in the kernel arguments (no upload);
// longer appends pass them through device memory (pos/seq non-null).
constexpr int kInlineTokens = 64;
struct AppendArgs {
    float *q;               // [nt][n_head][hd] or nullptr
    const float *k, *v;     // [nt][n_head_kv][hd_kv]
    void *kc, *vc;          // cache bases
    const int32_t *pos;     // device [nt], or nullptr: use ipos
    const int32_t *seq;     // device [nt], or nullptr: use iseq
    const float2 *tab_q;    // [capacity][hd/2] (nullptr if q is nullptr or style NONE)
    const float2 *tab_k;    // [capacity][hd_kv/2] (nullptr for style NONE)
    int64_t region_bytes, scale_off;
    int32_t nt, n_head, hd, n_head_kv, hd_kv, n_layer, layer, style;
    int32_t kv_fmt;         // KvFmt: the store rounds to binary16 or quantizes to Q8_0
};
template <int E>
struct AppendParamsT : AppendArgs {
    int32_t ipos[E], iseq[E];
};
using AppendParams = AppendParamsT<kInlineTokens>;
hipError_t launch_append(const AppendParams &p, hipStream_t s);

// ---- Fused decode step: q/k/v projections + biases + RoPE + K/V store -------------------
// Up to kInlineTokens tokens per call (positions and sequence ids in the arguments).
struct QkvParams {
    const float *x;          // [nt][d]
    const float *w[3];       // q, k, v weights: [rows][d], row j produces output j
    const float *b[3];       // biases [rows] or nullptr
    float *q_out;            // [nt][n_head][hd], rotated
    void *kc, *vc;           // cache bases
    const float2 *tab_q, *tab_k;  // RoPE tables (nullptr for style NONE)
    int64_t region_bytes, scale_off;
    int32_t d, nt, n_head, hd, n_head_kv, hd_kv, n_layer, layer, style, kv_fmt;
    int32_t units_q, units_kv;     // workgroup units of the q and of the k (= v) projection
    int32_t ipos[kInlineTokens], iseq[kInlineTokens];
};
// Rotation pairs per workgroup unit (units per head = ceil((head dim / 2) / this)).
int32_t qkv_pairs_per_unit(int32_t kv_fmt);
hipError_t launch_qkv(const QkvParams &p, hipStream_t s);

// ---- K2 + K3: split-K decode and log-sum-exp combine -----------------------------------
// One launch covers up to kInlineEntries batch entries, whose positions, sequence ids
// and chunk offsets ride in the kernel arguments.
constexpr int kInlineEntries = 64;
struct DecodeArgs {
    const float *q;          // [n][n_head][hd] (this launch's entries)
    float *out;              // [n][n_head][hd_kv]
    float *part;             // [total_chunks][n_head][hd_kv + 4]: m, l, -, -, acc[hd_kv]
    const void *kc, *vc;     // cache bases
    // Explicit windows: chunk c reads rows [pieces[2c], pieces[2c] + pieces[2c+1]) of its
    // entry's region (device-visible memory).  nullptr: entry b's window is rows
    // [0, pos[b]], cut into chunks of rows_per_chunk rows.
    const int32_t *pieces;
    int64_t region_bytes, scale_off;
    int32_t n, n_head, hd, n_head_kv, hd_kv, n_layer, layer, kv_fmt;
    int32_t rows_per_chunk, total_chunks;
    int32_t hpb;             // kv heads per split-K workgroup (decode_heads_per_block)
    float qscale;            // scale * log2(e): scores are kept in base-2 units
};
template <int E>
struct DecodeParamsT : DecodeArgs {
    int32_t pos[E];
    int32_t seq[E];
    int32_t cbase[E + 1];    // first chunk of entry b; cbase[n] = total_chunks
};
using DecodeParams = DecodeParamsT<kInlineEntries>;
// The allocation-free decode keeps its split-K records in a fixed device array of this
// many floats (16 MiB per GPU).  static_scratch_addr returns the device address of the
// array's copy on `device`; the first lookup for a device must run with that device
// current, later ones only read the kept address.
constexpr size_t kStaticScratchFloats = size_t(4) << 20;
hipError_t static_scratch_addr(int device, float **addr);

// kv heads per split-K workgroup for a region format and query-head group G: 2 for
// binary16 regions, and for Q8_0 regions at G = 2, with an even n_head_kv; else 1.
int32_t decode_heads_per_block(int32_t kv_fmt, int32_t n_head_kv, int32_t G);
// Workgroups of the split kernel that a call launches first (for this kv head dim,
// query-head group G, format, heads per workgroup and n entries in the launch) that
// `device` holds resident at once: resident workgroups per CU (HIP's occupancy query,
// looked up once per kernel) x CUs.  0 if a lookup fails.
int32_t decode_resident_blocks(int32_t device, int32_t hd_kv, int32_t G, int32_t kv_fmt,
                               int32_t hpb, int32_t n);
// Rows per step of the split-K kernel that a call with query-head group G (n_head /
// n_head_kv) launches first, for a kv head dim, region format and heads per workgroup
// (chunks should be a multiple of it).
int32_t decode_block_rows(int32_t hd_kv, int32_t G, int32_t kv_fmt, int32_t hpb);
hipError_t launch_decode(const DecodeParams &p, hipStream_t s);

// ---- K4: causal prefill with fp32 MFMA -------------------------------------------------
// Unit tables of up to kInlineUnits units ride in the kernel arguments.
constexpr int kInlineUnits = 64;
struct PrefillParams {
    const float *q;          // [nt][n_head][hd]
    float *out;              // [nt][n_head][hd_kv]
    const void *kc, *vc;     // this (seq, layer)'s K and V regions
    int64_t scale_off;       // Q8_0: byte offset of the scales in a region
    const int32_t *pos;      // device-visible [nt], or nullptr: pos[t] = pos0 + t
    int32_t pos0;
    const int32_t *units;    // device-visible plan.units, or nullptr: iunits holds them
    float *part;             // split only: [max_seg][nt][n_head][hd_kv + 4]: O, m, l, nseg
    float *dq;               // binary16 / Q8_0: f32 copies of rows [0, dq_rows) of K, then V
    int32_t dq_rows;         // a multiple of 64 covering every position of the call
    int32_t nt, n_head, hd, n_head_kv, hd_kv, capacity, kv_fmt;
    int32_t GB, TQ, n_qtiles, n_hsub, units_per_hgroup;
    int32_t max_seg;         // split only: records per (token, head) in `part`
    float qscale;            // scale * log2(e)
    int32_t iunits[kInlineUnits * kUnitInts];
};
hipError_t launch_prefill(const PrefillParams &p, hipStream_t s);

}  // namespace kvc
