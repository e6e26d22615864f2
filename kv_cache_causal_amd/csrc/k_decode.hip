// K2 + K3: decode attention over long KV windows, split along the KV axis, then merged.
//
// "11 · Attention, vec ops, and the KV cache":
//   §2.1   out = sum_s softmax_s(q . k_s * scale) v_s over the window s in [0, pos].
//   §2.4   query head h reads kv head h / (n_head / n_head_kv).
//   §3.2.4 the window of a query at position p is rows [0, p]: a length, not a mask.
//   §2.5   on a GPU the softmax runs online (running max and sum, block by block) and the
//          KV axis is split across workgroups, then reduced.
//
// Decode is a pure stream over K and V: every cached byte of the window is read once and
// used G = n_head / n_head_kv times, so it is bound by HBM bandwidth (G/2 flop per byte).
// Design for gfx950:
//   * Workgroup = one (batch entry, chunk of rows, block of HPB kv heads); 4 wave64s, of
//     which 4 / HPB share each kv head's rows.  Chunks are sized on the host so the grid
//     fills the chip several times over; the workgroups of one chunk's head blocks are
//     adjacent in dispatch order.  binary16 regions take 2 heads per workgroup (HPB = 2):
//     each workgroup then reads 2 adjacent 256-byte slices of every row of its chunk,
//     which streamed 6% faster in the batch decode than one slice per row.  f32 slices
//     (512 bytes) stream best one head per workgroup (2 or 4 heads: 6-8% slower), and
//     Q8_0 gained nothing from 2 or 4 (its decode is bound by its per-value arithmetic as
//     much as by its 128-byte slices).
//   * A row slice (hd_kv values of one kv head) is read by a group of LPR lanes: each
//     lane holds 8 values (4 for larger head groups, to save registers) -- two float4
//     loads of an f32 cache, or one 16-byte load of packed halves of a binary16 cache
//     (widened to f32 as they are used); one load instruction across the wave covers
//     64/LPR rows, whole 128-byte lines.  A Q8_0 cache gives each lane 8 codes (one
//     8-byte load, all in one 32-value block) plus that block's binary16 scale; the
//     codes are converted as they are used and the scale is applied once per lane and
//     row: to the lane's partial dot product for K, to the softmax weight for V (each
//     dequantized value is scale * code exactly, so only the rounding order differs
//     from dequantize-then-multiply).  Two register sets of 4 rows per lane group
//     alternate, so one set's loads are in flight while the other is reduced.
//   * The query vectors of every head of the kv group (up to 8 per pass) stay in
//     registers, so each K/V element loaded from HBM is used for all of them in-register:
//     the group's sharing costs no LDS traffic.
//   * Dot products reduce over the LPR lanes of a row with DPP row operations (no LDS);
//     each lane group keeps its own running max / sum / accumulator (online softmax,
//     base-2 exponent), and the lane groups of a wave and the 4 waves of the block are
//     merged once at the end (shuffles, then LDS).
//   * A window that fits one chunk is finished in place.  Otherwise each chunk writes its
//     (m, l, acc) partial and K3 merges them by log-sum-exp:
//     out = sum_c 2^(m_c-M) acc_c / sum_c 2^(m_c-M) l_c.  The merge is a separate kernel
//     on purpose: a device-scope fence inside K2 (to let the last chunk merge) compiles
//     on gfx950 to a full write-back and invalidate of the XCD's L2, which measured far
//     slower than one extra launch.
//   * The batch's positions, sequence ids and chunk offsets travel in the kernel
//     arguments (up to 64 entries per launch), so a decode needs no host-to-device copy.
//   * Explicit windows ("13 · The decode loop and graph reuse" §2.2: a query's cells are
//     an input, a list of runs): the host cuts every run into chunks of at most
//     rows_per_chunk rows and passes the (first row, rows) table; the kernel and the
//     merge are otherwise the same -- a chunk is a contiguous row range either way.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kWaves = 4;

// Dims of a row slice each lane holds.  f32: 8 (two float4) for kv groups of up to 2
// query heads, 4 (one float4) for larger groups, whose per-head registers would otherwise
// crowd out the load buffers.  binary16: 8 dims (16 bytes per lane) for groups of up to
// 4, 4 beyond.  Q8_0: 8 codes (8 bytes) for groups of up to 4, 4 beyond.
template <int GP, typename KVT>
constexpr int dims_per_lane()
{
    if constexpr (sizeof(KVT) == 1) return GP <= 4 ? 8 : 4;
    if constexpr (sizeof(KVT) == 2) return GP <= 4 ? 8 : 4;
    return GP <= 2 ? 8 : 4;
}

// Rows per lane group per step (two steps in flight).
template <int GP, typename KVT>
constexpr int rows_per_step()
{
    return 4;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over aligned groups of W lanes; every lane of a group gets the same bits (each step
// adds a pair in both orders, which IEEE addition makes identical).
template <int W>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (W >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (W >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (W >= 8) x += dpp<0x141>(x);  // row_half_mirror: i <-> 7 - i
    if constexpr (W >= 16) x += dpp<0x140>(x); // row_mirror: i <-> 15 - i
    if constexpr (W >= 32) x = add_xor16(x);
    if constexpr (W >= 64) x = add_xor32(x);
    return x;
}

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef int32_t intx2 __attribute__((ext_vector_type(2)));
typedef int32_t intx4 __attribute__((ext_vector_type(4)));

// Where one kv head's slices live in a region: row r's values start at element
// r * nkt + hk * hd; a Q8_0 region's scales start at `scales` (q8_scale_index: head-major,
// `rows` rows per head, interleaved by row quads).  hd is the kv head dim; the lane layout
// may be laid out for a wider power of two (padded lanes load nothing and hold zeros).
struct Slice {
    const char *region, *scales;
    int64_t rows;
    int32_t nkt, hk, hd;
};

// How a lane group reads its DPL dims of a row slice (LPR lanes per row).  Raw is what
// one row occupies in registers until it is used (binary16 and codes stay packed);
// get(r, i) is the lane's i-th value (a code for Q8_0); dim(li, i) is the head dim of the
// lane's i-th value, so q is loaded in the same order.  Per-row factors that turn codes
// into values come per quad of rows: with kQuads, a lane group's rows of a step are
// 4 consecutive rows 4p .. 4p+3, load_quad(s, p, li) fetches their factors for the
// lane's dims in one load and scale(quad, u) is row 4p+u's; the float formats have none
// (scale 1).
//   f32, 8 dims: two float4 at li*4 and 4*LPR + li*4 (each load instruction covers whole
//                lines of several rows);  f32, 4 dims: one float4 at li*4;
//   f16, 8 dims: one 16-byte load at li*8;  f16, 4 dims: 4 halves at li*4 (16 halves
//                per lane, as two loads, measured slower: more registers, fewer waves);
//   Q8_0, DPL dims: DPL codes at li*DPL (16, 8 or 4 bytes) and the scale of their block.
template <typename KVT, int DPL, int LPR>
struct RowIO;

struct NoRowScale {
    static constexpr bool kQuads = false;
    struct Quad {};
    static __device__ __forceinline__ Quad load_quad(const Slice &, int64_t, int) { return {}; }
    static __device__ __forceinline__ float scale(const Quad &, int) { return 1.0f; }
};

// Every K/V byte of a decode window is read exactly once, so row loads are nontemporal:
// they stream past the caches instead of displacing lines other work will reuse
// (measured: the batch decode 9% faster, the long-context one 6%).
template <typename T>
__device__ __forceinline__ T stream_load(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
}

template <typename KVT>
__device__ __forceinline__ const KVT *slice_row(const Slice &s, int64_t row)
{
    return reinterpret_cast<const KVT *>(s.region) + row * s.nkt + (int64_t)s.hk * s.hd;
}

// PAD: the head dim is below the lane layout's; a lane loads only the pieces that start
// inside the head (head dims are multiples of 16, so a piece is wholly in or out).
template <bool PAD, typename T>
__device__ __forceinline__ T load_if(const void *p, bool inside)
{
    if (!PAD || inside) return stream_load<T>(p);
    return T{};
}

template <int LPR>
struct RowIO<float, 8, LPR> : NoRowScale {
    struct Raw { floatx4 a, b; };
    template <bool PAD>
    static __device__ __forceinline__ Raw load(const Slice &s, int64_t row, int li)
    {
        const float *p = slice_row<float>(s, row);
        Raw r;
        r.a = load_if<PAD, floatx4>(p + li * 4, li * 4 < s.hd);
        r.b = load_if<PAD, floatx4>(p + 4 * LPR + li * 4, 4 * LPR + li * 4 < s.hd);
        return r;
    }
    static __device__ __forceinline__ float get(const Raw &r, int i) { return i < 4 ? r.a[i] : r.b[i - 4]; }
    static __device__ __forceinline__ int dim(int li, int i) { return (i / 4) * 4 * LPR + li * 4 + (i % 4); }
};
template <int LPR>
struct RowIO<float, 4, LPR> : NoRowScale {
    typedef floatx4 Raw;
    template <bool PAD>
    static __device__ __forceinline__ Raw load(const Slice &s, int64_t row, int li)
    {
        return load_if<PAD, floatx4>(slice_row<float>(s, row) + li * 4, li * 4 < s.hd);
    }
    static __device__ __forceinline__ float get(const Raw &r, int i) { return r[i]; }
    static __device__ __forceinline__ int dim(int li, int i) { return li * 4 + i; }
};
template <int LPR>
struct RowIO<_Float16, 8, LPR> : NoRowScale {
    typedef half8_t Raw;
    template <bool PAD>
    static __device__ __forceinline__ Raw load(const Slice &s, int64_t row, int li)
    {
        return load_if<PAD, half8_t>(slice_row<_Float16>(s, row) + li * 8, li * 8 < s.hd);
    }
    static __device__ __forceinline__ float get(const Raw &r, int i) { return (float)r[i]; }
    static __device__ __forceinline__ int dim(int li, int i) { return li * 8 + i; }
};
template <int LPR>
struct RowIO<_Float16, 4, LPR> : NoRowScale {
    typedef half4_t Raw;
    template <bool PAD>
    static __device__ __forceinline__ Raw load(const Slice &s, int64_t row, int li)
    {
        return load_if<PAD, half4_t>(slice_row<_Float16>(s, row) + li * 4, li * 4 < s.hd);
    }
    static __device__ __forceinline__ float get(const Raw &r, int i) { return (float)r[i]; }
    static __device__ __forceinline__ int dim(int li, int i) { return li * 4 + i; }
};

// Signed byte k of w as f32: one v_cvt_f32_i32 with an SDWA sign-extending byte select.
// (Written out because the compiler, given byte vectors that pass through the
// double-buffered register sets, unpacks every byte into its own register first.)
__device__ __forceinline__ float code_to_f32(int32_t w, int k)
{
    float f;
    switch (k) {
    case 0: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(f) : "v"(w)); break;
    case 1: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(f) : "v"(w)); break;
    case 2: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(f) : "v"(w)); break;
    default: asm("v_cvt_f32_i32_sdwa %0, sext(%1) dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(f) : "v"(w)); break;
    }
    return f;
}

template <int DPL>
struct CodeVec;
template <> struct CodeVec<16> { typedef intx4 T; };
template <> struct CodeVec<8> { typedef intx2 T; };
template <> struct CodeVec<4> { typedef int32_t T; };

template <int DPL, int LPR>
struct RowIO<int8_t, DPL, LPR> {
    static constexpr int HD = DPL * LPR;
    typedef typename CodeVec<DPL>::T Codes;
    struct Raw { Codes c; };
    static constexpr bool kQuads = true;
    typedef half4_t Quad;   // the scales of the lane's block for 4 consecutive rows
    template <bool PAD>
    static __device__ __forceinline__ Raw load(const Slice &s, int64_t row, int li)
    {
        static_assert(!PAD, "Q8_0 head dims fill the lane layout");
        const int64_t v0 = row * s.nkt + (int64_t)s.hk * HD + li * DPL;   // first value
        return Raw{stream_load<Codes>(s.region + v0)};
    }
    static __device__ __forceinline__ Quad load_quad(const Slice &s, int64_t quad, int li)
    {
        const int64_t si = (((int64_t)s.hk * (s.rows >> 2) + quad) * (HD / kQ8Block) + li * DPL / kQ8Block) * 4;
        return stream_load<Quad>(s.scales + 2 * si);
    }
    // Codes stay packed four to a register until used; a signed byte of a register
    // converts in one instruction (sign-extending byte select on the operand).
    static __device__ __forceinline__ float get(const Raw &r, int i)
    {
        int32_t w;
        if constexpr (DPL == 4) w = r.c;
        else w = r.c[i / 4];
        return code_to_f32(w, i % 4);
    }
    static __device__ __forceinline__ float scale(const Quad &q, int u) { return (float)q[u]; }
    static __device__ __forceinline__ int dim(int li, int i) { return li * DPL + i; }
};

// Merge (m2, l2) into (m, l) in base-2 units; returns the scale factors for acc.
__device__ __forceinline__ void lse_merge(float &m, float &l, float m2, float l2, float &a,
                                          float &b)
{
    const float mn = fmaxf(m, m2);
    const float ref = (mn == -INFINITY) ? 0.0f : mn;  // both empty: keep zeros, no NaN
    a = fast_exp2(m - ref);
    b = fast_exp2(m2 - ref);
    l = l * a + l2 * b;
    m = mn;
}

// HD is the lane layout's head dim; PAD: the kv head dim p.hd_kv is below it (a multiple
// of 16), and the lanes past it load nothing.
template <int HD, int GP, typename KVT, int HPB, int E, bool PAD>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeParamsT<E> p, int32_t g0)
{
    constexpr int kDimsPerLane = dims_per_lane<GP, KVT>();
    constexpr int kUnroll = rows_per_step<GP, KVT>();
    constexpr int LPR = HD / kDimsPerLane;   // lanes per row
    constexpr int RPW = 64 / LPR;            // rows per wave per unrolled step
    constexpr int WPH = kWaves / HPB;        // waves per kv head
    using IO = RowIO<KVT, kDimsPerLane, LPR>;
    using Raw = typename IO::Raw;
    static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "head dim");
    static_assert(kWaves % HPB == 0, "heads per workgroup");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane % LPR;
    const int rg = lane / LPR;
    // Linear grid, head block fastest: the workgroups of one chunk are dispatched together
    // and read the slices of the same rows at about the same time.  Waves wh * WPH ..
    // wh * WPH + WPH - 1 take kv head hb * HPB + wh; wr numbers them within the head.
    const int nhb = p.n_head_kv / HPB;
    const int wh = wave / WPH;
    const int wr = wave - wh * WPH;
    const int hk = (blockIdx.x % nhb) * HPB + wh;
    const int cg = blockIdx.x / nhb;
    const int G = p.n_head / p.n_head_kv;

    // Batch entry owning this chunk: cbase[b] <= cg < cbase[b + 1] (kernel arguments).
    int lo = 0, hi = p.n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cbase[mid] <= cg) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int nchunks = p.cbase[b + 1] - p.cbase[b];
    int r0, r1;   // this chunk's rows [r0, r1), never empty
    if (p.pieces) {
        r0 = p.pieces[2 * cg];
        r1 = r0 + p.pieces[2 * cg + 1];
    } else {
        r0 = (cg - p.cbase[b]) * p.rows_per_chunk;
        r1 = min(r0 + p.rows_per_chunk, p.pos[b] + 1);
    }
    const int seq = p.seq[b];
    const int hdr = PAD ? p.hd_kv : HD;   // the kv head dim
    const int nkt = p.n_head_kv * hdr;
    const int64_t reg = ((int64_t)seq * p.n_layer + p.layer) * p.region_bytes;
    const int64_t qrows = p.scale_off / nkt;   // region rows (Q8_0 only)
    const char *kreg = static_cast<const char *>(p.kc) + reg;
    const char *vreg = static_cast<const char *>(p.vc) + reg;
    const Slice K{kreg, kreg + p.scale_off, qrows, nkt, hk, hdr};
    const Slice V{vreg, vreg + p.scale_off, qrows, nkt, hk, hdr};

    // The lane's query values in the order its row values arrive (IO::dim).  Loaded here,
    // scaled only after the first step's row loads are issued (below), so that the query
    // and the first rows are in flight together.
    float qf[GP][kDimsPerLane];
#pragma unroll
    for (int g = 0; g < GP; g++) {
        const bool ok = g0 + g < G;
        const float *qrow = p.q + ((int64_t)b * p.n_head + (hk * G + (ok ? g0 + g : 0))) * p.hd;
#pragma unroll
        for (int i = 0; i < kDimsPerLane; i++)
            qf[g][i] = (!PAD || IO::dim(li, i) < hdr) ? qrow[IO::dim(li, i)] : 0.0f;
    }

    float m[GP], l[GP], acc[GP][kDimsPerLane];
#pragma unroll
    for (int g = 0; g < GP; g++) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < kDimsPerLane; d++) acc[g][d] = 0.0f;
    }

    // Rows are consumed in steps of BR per kv head; two register sets alternate so the
    // loads of step i+1 are in flight while step i is reduced.  Row of unrolled row u of
    // a step starting at rb: instruction u of the wave reads RPW rows, RPW apart with row
    // quads (the lane group's rows are the quad rb + 4 (wr RPW + rg) + 0..3, so steps
    // start at r0 rounded down to a quad; rows before r0 are read and masked), adjacent
    // otherwise.
    constexpr int BR = WPH * RPW * kUnroll;
    constexpr bool kQuads = IO::kQuads;
    static_assert(!kQuads || kUnroll == 4, "row quads need 4 rows per lane group per step");
    const int rbase = kQuads ? (r0 & ~3) : r0;
    const int nsteps = (r1 - rbase + BR - 1) / BR;
    auto row_of = [&](int rb, int u) {
        return kQuads ? rb + (wr * RPW + rg) * 4 + u : rb + (u * WPH + wr) * RPW + rg;
    };
    using Quad = typename IO::Quad;
    Raw kA[kUnroll], vA[kUnroll], kB[kUnroll], vB[kUnroll];
    Quad kqA, vqA, kqB, vqB;

    auto load = [&](Raw (&kf)[kUnroll], Raw (&vf)[kUnroll], Quad &kq, Quad &vq, int step) {
        const int rb = rbase + step * BR;
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            int row = row_of(rb, u);
            row = row < r1 ? row : r0;  // rows past the chunk re-read row r0 and are masked
            kf[u] = IO::template load<PAD>(K, row, li);
            vf[u] = IO::template load<PAD>(V, row, li);
        }
        if constexpr (kQuads) {
            // A quad wholly past the chunk re-reads r0's quad (inside the region).
            const int q4 = row_of(rb, 0);
            const int quad = (q4 < r1 ? q4 : r0) >> 2;
            kq = IO::load_quad(K, quad, li);
            vq = IO::load_quad(V, quad, li);
        }
    };
    auto consume = [&](const Raw (&kf)[kUnroll], Raw (&vf)[kUnroll], const Quad &kq,
                       const Quad &vq, int step) {
        const int rb = rbase + step * BR;
        if constexpr (!kQuads) {
            // The chunk's last step: its rows past r1 hold row r0's values (see load).
            // Their weight is 0, but 0 * inf is NaN, so a non-finite V value of row r0
            // would leak into the result through them: their V registers become 0.
            // (Q8_0 codes are finite, and a masked row's V factor is 0 instead.)
            if (rb + BR > r1) {
#pragma unroll
                for (int u = 0; u < kUnroll; u++)
                    if (row_of(rb, u) >= r1) vf[u] = Raw{};
            }
        }
        float sc[kUnroll][GP], pv[kUnroll][GP], vs[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int row = row_of(rb, u);
            const bool valid = row < r1 && (!kQuads || row >= r0);
            // A masked row's weight is 0; its own V factor (a row outside the window,
            // possibly holding an infinite scale) must not turn that into NaN.
            vs[u] = (kQuads && !valid) ? 0.0f : IO::scale(vq, u);
#pragma unroll
            for (int g = 0; g < GP; g++) {
                float s = 0.0f;
#pragma unroll
                for (int i = 0; i < kDimsPerLane; i++) s += qf[g][i] * IO::get(kf[u], i);
                s = group_sum<LPR>(s * IO::scale(kq, u));
                sc[u][g] = valid ? s : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < GP; g++) {
            float mt = sc[0][g];
#pragma unroll
            for (int u = 1; u < kUnroll; u++) mt = fmaxf(mt, sc[u][g]);
            // Rescale only when the running max grows (alpha = 0 on the first valid rows);
            // after the first steps it rarely does, and an unchanged max would multiply by
            // exactly 1.
            const float mn = fmaxf(m[g], mt);
            if (mn > m[g]) {
                const float alpha = fast_exp2(m[g] - mn);
                l[g] *= alpha;
#pragma unroll
                for (int d = 0; d < kDimsPerLane; d++) acc[g][d] *= alpha;
                m[g] = mn;
            }
            const float ref = (m[g] == -INFINITY) ? 0.0f : m[g];
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                const float pu = fast_exp2(sc[u][g] - ref);
                l[g] += pu;
                pv[u][g] = pu * vs[u];
            }
        }
        // Each V value is widened once and feeds every head of the group.
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
#pragma unroll
            for (int i = 0; i < kDimsPerLane; i++) {
                const float x = IO::get(vf[u], i);
#pragma unroll
                for (int g = 0; g < GP; g++) acc[g][i] += pv[u][g] * x;
            }
        }
    };

    __builtin_amdgcn_sched_barrier(0);
    load(kA, vA, kqA, vqA, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < GP; g++) {
        const bool ok = g0 + g < G;
#pragma unroll
        for (int i = 0; i < kDimsPerLane; i++) qf[g][i] = ok ? qf[g][i] * p.qscale : 0.0f;
    }
    // The loads inside the loop are unconditional: with a load that a branch may skip, the
    // compiler's wait counts must hold on the path without it, and consuming one set then
    // also waits for the other set's loads, so the two sets never overlap.
    int st = 0;
    for (; st + 2 < nsteps; st += 2) {
        load(kB, vB, kqB, vqB, st + 1);
        consume(kA, vA, kqA, vqA, st);
        load(kA, vA, kqA, vqA, st + 2);
        consume(kB, vB, kqB, vqB, st + 1);
    }
    if (st + 1 < nsteps) {
        load(kB, vB, kqB, vqB, st + 1);
        consume(kA, vA, kqA, vqA, st);
        consume(kB, vB, kqB, vqB, st + 1);
    } else if (st < nsteps) {
        consume(kA, vA, kqA, vqA, st);
    }

    // Merge the row groups of the wave (lanes that share li).
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < GP; g++) {
            const float mo = __shfl_xor(m[g], off);
            const float lo2 = __shfl_xor(l[g], off);
            float a, bsc;
            lse_merge(m[g], l[g], mo, lo2, a, bsc);
#pragma unroll
            for (int d = 0; d < kDimsPerLane; d++) {
                const float ao = __shfl_xor(acc[g][d], off);
                acc[g][d] = acc[g][d] * a + ao * bsc;
            }
        }
    }

    // Merge the waves through LDS.
    __shared__ float sm[kWaves][GP][HD + 2];
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < GP; g++) {
            if (li == 0) {
                sm[wave][g][0] = m[g];
                sm[wave][g][1] = l[g];
            }
#pragma unroll
            for (int i = 0; i < kDimsPerLane; i++) sm[wave][g][2 + IO::dim(li, i)] = acc[g][i];
        }
    }
    __syncthreads();

    const int ngp = min(GP, G - g0);   // heads of this pass that exist
    float *out_b = p.out + (int64_t)b * p.n_head * hdr;
    for (int idx = threadIdx.x; idx < HPB * ngp * hdr; idx += blockDim.x) {
        const int bh = idx / (ngp * hdr);   // kv head of the block
        const int g = (idx - bh * ngp * hdr) / hdr;
        const int d = idx - (bh * ngp + g) * hdr;
        const int w0 = bh * WPH;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WPH; w++) M = fmaxf(M, sm[w0 + w][g][0]);
        const float ref = (M == -INFINITY) ? 0.0f : M;
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < WPH; w++) {
            const float f = fast_exp2(sm[w0 + w][g][0] - ref);
            L += f * sm[w0 + w][g][1];
            A += f * sm[w0 + w][g][2 + d];
        }
        const int h = (hk - wh + bh) * G + g0 + g;
        if (nchunks == 1) {
            out_b[(int64_t)h * hdr + d] = A / L;
        } else {
            float *rec = p.part + ((int64_t)cg * p.n_head + h) * (hdr + 4);
            if (d == 0) {
                rec[0] = M;
                rec[1] = L;
            }
            rec[4 + d] = A;
        }
    }
}

// K3: one workgroup per (batch entry, query head) with more than one chunk.  Each thread
// owns 4 consecutive output dims (one 16-byte load per record) and a slice of the chunks
// (256 / (HD/4) slices: 8 for head dim 128), and folds its chunks' records (m, l,
// acc[d..d+3]) into a running (M, L, A) by log-sum-exp, eight chunks per trip (their
// loads are independent, so they are in flight together); the slices are then merged
// the same way through LDS.  A window of up to 8 x slices chunks (64 for head dim 128)
// is merged in one trip of loads.
template <int HD, int E>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeParamsT<E> p)
{
    constexpr int QPR = HD / 4;                          // dim quads per record
    constexpr int SLICES = 256 / QPR;                    // chunk slices
    constexpr int NT = QPR * SLICES;                     // threads with a (quad, slice)
    __shared__ float sM[NT], sL[NT];
    __shared__ floatx4 sA[NT];
    const int b = blockIdx.x;
    const int h = blockIdx.y;
    const int c0 = p.cbase[b], c1 = p.cbase[b + 1];
    if (c1 - c0 <= 1) return;  // finished in place by the split kernel
    const int tid = threadIdx.x;
    const float *base = p.part + (int64_t)h * (HD + 4);
    const int64_t cstride = (int64_t)p.n_head * (HD + 4);
    const int quad = tid % QPR;
    const int slice = tid / QPR;

    float M = -INFINITY, L = 0.0f;
    floatx4 A = {0.0f, 0.0f, 0.0f, 0.0f};
    if (tid < NT) {
        int c = c0 + slice;
        for (; c + 7 * SLICES < c1; c += 8 * SLICES) {
            float mm[8], ll[8];
            floatx4 aa[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float *rec = base + (int64_t)(c + j * SLICES) * cstride;
                mm[j] = rec[0];
                ll[j] = rec[1];
                aa[j] = *reinterpret_cast<const floatx4 *>(rec + 4 + 4 * quad);
            }
            float mn = M;
#pragma unroll
            for (int j = 0; j < 8; j++) mn = fmaxf(mn, mm[j]);   // finite: chunks hold rows
            const float r = fast_exp2(M - mn);                   // 0 while M is -inf
            L *= r;
            A *= r;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const float w = fast_exp2(mm[j] - mn);
                L += w * ll[j];
                A += w * aa[j];
            }
            M = mn;
        }
        for (; c < c1; c += SLICES) {
            const float *rec = base + (int64_t)c * cstride;
            const float mc = rec[0];
            const float mn = fmaxf(M, mc);
            const float r = fast_exp2(M - mn), w = fast_exp2(mc - mn);
            L = L * r + w * rec[1];
            A = A * r + w * *reinterpret_cast<const floatx4 *>(rec + 4 + 4 * quad);
            M = mn;
        }
        sM[tid] = M;
        sL[tid] = L;
        sA[tid] = A;
    }
    __syncthreads();
    if (tid < QPR) {
        float Mt = -INFINITY;
#pragma unroll
        for (int sl = 0; sl < SLICES; sl++) Mt = fmaxf(Mt, sM[sl * QPR + tid]);
        float Lt = 0.0f;
        floatx4 At = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sl = 0; sl < SLICES; sl++) {
            // A slice with no chunk has M = -inf and contributes exp2(-inf) * 0 = 0.
            const float w = fast_exp2(sM[sl * QPR + tid] - Mt);
            Lt += w * sL[sl * QPR + tid];
            At += w * sA[sl * QPR + tid];
        }
        *reinterpret_cast<floatx4 *>(p.out + ((int64_t)b * p.n_head + h) * HD + 4 * tid) = At / Lt;
    }
}

template <int HD, typename KVT, int HPB, int E, bool PAD>
void launch_split_hpb(const DecodeParamsT<E> &p, hipStream_t s)
{
    const int G = p.n_head / p.n_head_kv;
    const dim3 grid((unsigned)p.total_chunks * (unsigned)(p.n_head_kv / HPB)), block(256);
    for (int g0 = 0; g0 < G; g0 += 8) {
        const int left = G - g0;
        if (left >= 5) decode_split_kernel<HD, 8, KVT, HPB, E, PAD><<<grid, block, 0, s>>>(p, g0);
        else if (left >= 3) decode_split_kernel<HD, 4, KVT, HPB, E, PAD><<<grid, block, 0, s>>>(p, g0);
        else if (left == 2) decode_split_kernel<HD, 2, KVT, HPB, E, PAD><<<grid, block, 0, s>>>(p, g0);
        else decode_split_kernel<HD, 1, KVT, HPB, E, PAD><<<grid, block, 0, s>>>(p, g0);
    }
}

template <int HD, typename KVT, int E, bool PAD>
void launch_split(const DecodeParamsT<E> &p, hipStream_t s)
{
    if constexpr (sizeof(KVT) <= 2) {
        if (p.hpb == 2) return launch_split_hpb<HD, KVT, 2, E, PAD>(p, s);
    }
    launch_split_hpb<HD, KVT, 1, E, PAD>(p, s);
}

// The split kernel that launch_split launches first (the pass of the first 8 heads).
template <int HD, typename KVT, int HPB, int E, bool PAD>
const void *first_split_kernel(int32_t G)
{
    if (G >= 5) return reinterpret_cast<const void *>(decode_split_kernel<HD, 8, KVT, HPB, E, PAD>);
    if (G >= 3) return reinterpret_cast<const void *>(decode_split_kernel<HD, 4, KVT, HPB, E, PAD>);
    if (G == 2) return reinterpret_cast<const void *>(decode_split_kernel<HD, 2, KVT, HPB, E, PAD>);
    return reinterpret_cast<const void *>(decode_split_kernel<HD, 1, KVT, HPB, E, PAD>);
}
template <int HD, typename KVT, int E, bool PAD>
const void *first_split_kernel_hpb(int32_t G, int32_t hpb)
{
    if constexpr (sizeof(KVT) <= 2) {
        if (hpb == 2) return first_split_kernel<HD, KVT, 2, E, PAD>(G);
    }
    return first_split_kernel<HD, KVT, 1, E, PAD>(G);
}

// HDL: the lane layout's head dim (a power of two); HDR: the kv head dim (HDR <= HDL).
template <int HDL, int HDR, int E>
hipError_t launch_hd(const DecodeParamsT<E> &p, hipStream_t s)
{
    constexpr bool PAD = HDR != HDL;
    if constexpr (!PAD && HDL % kQ8Block == 0) {
        if (p.kv_fmt == kFmtQ8) launch_split<HDL, int8_t, E, false>(p, s);
    }
    if (p.kv_fmt == kFmtF16) launch_split<HDL, _Float16, E, PAD>(p, s);
    else if (p.kv_fmt == kFmtF32) launch_split<HDL, float, E, PAD>(p, s);
    if (p.total_chunks > p.n) {  // some entry spans several chunks
        const dim3 cgrid((unsigned)p.n, (unsigned)p.n_head);
        decode_combine_kernel<HDR, E><<<cgrid, 256, 0, s>>>(p);
    }
    return hipGetLastError();
}

template <int HDL, int HDR, int E>
const void *first_split_kernel_hd(int32_t G, int32_t kv_fmt, int32_t hpb)
{
    constexpr bool PAD = HDR != HDL;
    if constexpr (!PAD && HDL % kQ8Block == 0) {
        if (kv_fmt == kFmtQ8) return first_split_kernel_hpb<HDL, int8_t, E, false>(G, hpb);
    }
    if (kv_fmt == kFmtF16) return first_split_kernel_hpb<HDL, _Float16, E, PAD>(G, hpb);
    if (kv_fmt == kFmtF32) return first_split_kernel_hpb<HDL, float, E, PAD>(G, hpb);
    return nullptr;
}

// Index of a supported kv head dim (0 .. kNumHd - 1), and the kernel of launch_hd's first
// launch for it.
constexpr int kNumHd = 10;
int hd_index(int32_t hd_kv)
{
    switch (hd_kv) {
    case 16: return 0;
    case 32: return 1;
    case 64: return 2;
    case 80: return 3;
    case 96: return 4;
    case 112: return 5;
    case 128: return 6;
    case 160: return 7;
    case 192: return 8;
    case 256: return 9;
    default: return -1;
    }
}
template <int E>
const void *first_split_kernel_any(int32_t hd_kv, int32_t G, int32_t kv_fmt, int32_t hpb)
{
    switch (hd_kv) {
    case 16: return first_split_kernel_hd<16, 16, E>(G, kv_fmt, hpb);
    case 32: return first_split_kernel_hd<32, 32, E>(G, kv_fmt, hpb);
    case 64: return first_split_kernel_hd<64, 64, E>(G, kv_fmt, hpb);
    case 80: return first_split_kernel_hd<128, 80, E>(G, kv_fmt, hpb);
    case 96: return first_split_kernel_hd<128, 96, E>(G, kv_fmt, hpb);
    case 112: return first_split_kernel_hd<128, 112, E>(G, kv_fmt, hpb);
    case 128: return first_split_kernel_hd<128, 128, E>(G, kv_fmt, hpb);
    case 160: return first_split_kernel_hd<256, 160, E>(G, kv_fmt, hpb);
    case 192: return first_split_kernel_hd<256, 192, E>(G, kv_fmt, hpb);
    case 256: return first_split_kernel_hd<256, 256, E>(G, kv_fmt, hpb);
    default: return nullptr;
    }
}

template <int E>
hipError_t launch_by_hd(const DecodeParamsT<E> &p, hipStream_t s)
{
    switch (p.hd_kv) {
    case 16: return launch_hd<16, 16, E>(p, s);
    case 32: return launch_hd<32, 32, E>(p, s);
    case 64: return launch_hd<64, 64, E>(p, s);
    case 80: return launch_hd<128, 80, E>(p, s);
    case 96: return launch_hd<128, 96, E>(p, s);
    case 112: return launch_hd<128, 112, E>(p, s);
    case 128: return launch_hd<128, 128, E>(p, s);
    case 160: return launch_hd<256, 160, E>(p, s);
    case 192: return launch_hd<256, 192, E>(p, s);
    case 256: return launch_hd<256, 256, E>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {
// The decode lane layout's head dim for a kv head dim: the next power of two from 16.
constexpr int32_t decode_lane_dim(int32_t hd_kv)
{
    return hd_kv <= 16 ? 16 : hd_kv <= 32 ? 32 : hd_kv <= 64 ? 64 : hd_kv <= 128 ? 128 : 256;
}

// Rows per step of the split kernel for a query-head group of GP with hpb kv heads per
// workgroup: each of a head's 4 / hpb waves covers 64 * dims / hd_kv rows per unrolled row.
template <int GP, typename KVT>
int32_t step_rows(int32_t hd_kv, int32_t hpb)
{
    const int32_t hdl = decode_lane_dim(hd_kv);
    return kWaves / hpb * (64 * dims_per_lane<GP, KVT>() / hdl) * rows_per_step<GP, KVT>();
}
template <typename KVT>
int32_t step_rows_fmt(int32_t hd_kv, int32_t G, int32_t hpb)
{
    // The group of the first pass (launch_split): 8 heads from 5 up, then 4, 2, 1.
    if (G >= 5) return step_rows<8, KVT>(hd_kv, hpb);
    if (G >= 3) return step_rows<4, KVT>(hd_kv, hpb);
    if (G == 2) return step_rows<2, KVT>(hd_kv, hpb);
    return step_rows<1, KVT>(hd_kv, hpb);
}
}  // namespace

// ---- Fixed scratch for the allocation-free decode (gqa_attn_decode_noalloc) ----------
// The split-K records of that entry point live in this array instead of in handle-owned
// memory that grows on demand.  Each GPU the library runs on holds its own copy, at its
// own address, for the life of the process.  On the host the name `scratch` stands for
// the variable, not for device memory: kernels get the address hipGetSymbolAddress
// returns for the device, kept per device below.
static __device__ __align__(256) float scratch[kStaticScratchFloats];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch_addr(int device, float **addr)
{
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    float *a = g_scratch_addr[device].load(std::memory_order_acquire);
    if (!a) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        a = g_scratch_addr[device].load(std::memory_order_relaxed);
        if (!a) {
            // The address of the device's copy is looked up with that device current.
            int cur = -1;
            hipError_t e = hipGetDevice(&cur);
            if (e != hipSuccess) return e;
            if (cur != device) return hipErrorInvalidDevice;
            void *p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            a = static_cast<float *>(p);
            g_scratch_addr[device].store(a, std::memory_order_release);
        }
    }
    *addr = a;
    return hipSuccess;
}

int32_t decode_heads_per_block(int32_t kv_fmt, int32_t n_head_kv, int32_t G)
{
    if (n_head_kv % 2 != 0) return 1;
    if (kv_fmt == kFmtF16) return 2;
    return kv_fmt == kFmtQ8 && G == 2 ? 2 : 1;
}

namespace {
// Resident workgroups per CU of each first-pass split kernel (0: not looked up yet), by
// kv head dim, query-head group class, format, heads per workgroup and argument block.
// The library holds gfx950 code only, so the count is the same on every device it runs on.
std::atomic<int32_t> g_blocks_per_cu[kNumHd][4][3][2][2];
std::atomic<int32_t> g_cus[kMaxDevices];
}  // namespace

int32_t decode_resident_blocks(int32_t device, int32_t hd_kv, int32_t G, int32_t kv_fmt,
                               int32_t hpb, int32_t n)
{
    const int hi = hd_index(hd_kv);
    if (hi < 0 || kv_fmt < 0 || kv_fmt > 2 || hpb < 1 || hpb > 2 || device < 0 ||
        device >= kMaxDevices)
        return 0;
    const int gc = G >= 5 ? 3 : G >= 3 ? 2 : G == 2 ? 1 : 0;
    const bool small = n <= kSmallInline;
    std::atomic<int32_t> &slot = g_blocks_per_cu[hi][gc][kv_fmt][hpb - 1][small ? 1 : 0];
    int32_t per_cu = slot.load(std::memory_order_relaxed);
    if (per_cu == 0) {
        const void *k = small ? first_split_kernel_any<kSmallInline>(hd_kv, G, kv_fmt, hpb)
                              : first_split_kernel_any<kInlineEntries>(hd_kv, G, kv_fmt, hpb);
        int nb = 0;
        if (!k || hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, 256, 0) != hipSuccess ||
            nb <= 0)
            return 0;
        per_cu = nb;
        slot.store(per_cu, std::memory_order_relaxed);
    }
    int32_t cus = g_cus[device].load(std::memory_order_relaxed);
    if (cus == 0) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, device) !=
                hipSuccess ||
            c <= 0)
            return 0;
        cus = c;
        g_cus[device].store(cus, std::memory_order_relaxed);
    }
    return per_cu * cus;
}

int32_t decode_block_rows(int32_t hd_kv, int32_t G, int32_t kv_fmt, int32_t hpb)
{
    if (kv_fmt == kFmtQ8) return step_rows_fmt<int8_t>(hd_kv, G, hpb);
    if (kv_fmt == kFmtF16) return step_rows_fmt<_Float16>(hd_kv, G, hpb);
    return step_rows_fmt<float>(hd_kv, G, hpb);
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t s)
{
    if (p.n <= kSmallInline) {
        // Few entries: the same launches with an argument block sized for them.
        DecodeParamsT<kSmallInline> sp;
        static_cast<DecodeArgs &>(sp) = p;
        for (int i = 0; i < kSmallInline; i++) {
            sp.pos[i] = i < p.n ? p.pos[i] : 0;
            sp.seq[i] = i < p.n ? p.seq[i] : 0;
        }
        for (int i = 0; i <= kSmallInline; i++) sp.cbase[i] = p.cbase[i < p.n ? i : p.n];
        return launch_by_hd(sp, s);
    }
    return launch_by_hd(p, s);
}

}  // namespace kvc
