// K2 + K3: decode attention over long KV windows, split along the KV axis.
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
//   * Workgroup = one (batch entry, kv head, chunk of rows); 4 wave64s.  Chunks are sized
//     on the host so the grid holds ~4 workgroups per CU.
//   * A row slice (hd_kv floats of one kv head) is read by a group of LPR = hd_kv/8 lanes,
//     each lane holding 8 dims as two float4 loads; one load instruction across the wave
//     covers 64/LPR rows, whole 128-byte lines.
//   * The query vectors of every head of the kv group (up to 8 per pass) stay in
//     registers, so each K/V element loaded from HBM is used for all of them in-register:
//     the group's sharing costs no LDS traffic.
//   * Dot products reduce over the LPR lanes of a row with xor shuffles; each lane group
//     keeps its own running max / sum / accumulator (online softmax, base-2 exponent),
//     and the 64/LPR groups of a wave and the 4 waves of the block are merged once at the
//     end (shuffles, then LDS).  The merged (m, l, acc) of the chunk goes to a partial.
//   * K3 merges the partials of each (entry, head) by log-sum-exp: out = sum_c 2^(m_c-M)
//     acc_c / sum_c 2^(m_c-M) l_c.
#include <hip/hip_runtime.h>

#include <cmath>

#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kWaves = 4;
constexpr int kDimsPerLane = 8;   // two float4 per lane per row
constexpr int kUnroll = 4;        // rows per lane group per iteration (loads in flight)

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

template <int HD, int GP>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeParams p, int32_t g0)
{
    constexpr int LPR = HD / kDimsPerLane;   // lanes per row
    constexpr int RPW = 64 / LPR;            // rows per wave per unrolled step
    constexpr int NF4 = kDimsPerLane / 4;
    static_assert(LPR >= 1 && LPR <= 64 && (64 % LPR) == 0, "head dim");

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane % LPR;
    const int rg = lane / LPR;
    const int hk = blockIdx.y;
    const int cg = blockIdx.x;
    const int G = p.n_head / p.n_head_kv;

    // Batch entry owning this chunk: cbase[b] <= cg < cbase[b + 1].
    int lo = 0, hi = p.n;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cbase[mid] <= cg) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int vl = p.pos[b] + 1;
    const int r0 = (cg - p.cbase[b]) * p.rows_per_chunk;
    const int r1 = min(r0 + p.rows_per_chunk, vl);
    const int seq = p.seq[b];
    const int nkt = p.n_head_kv * HD;
    const int64_t region = ((int64_t)seq * p.n_layer + p.layer) * p.region;
    const float *K = p.kc + region + hk * HD;
    const float *V = p.vc + region + hk * HD;

    // Lane dims: d(c, e) = c * 4 * LPR + li * 4 + e, so one float4 load across the LPR
    // lanes of a row covers 16 * LPR contiguous bytes.
    float qf[GP][kDimsPerLane];
#pragma unroll
    for (int g = 0; g < GP; g++) {
        const bool ok = g0 + g < G;
        const float *qrow = p.q + ((int64_t)b * p.n_head + (hk * G + (ok ? g0 + g : 0))) * p.hd;
#pragma unroll
        for (int c = 0; c < NF4; c++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                qf[g][c * 4 + e] = ok ? qrow[c * 4 * LPR + li * 4 + e] * p.qscale : 0.0f;
    }

    float m[GP], l[GP], acc[GP][kDimsPerLane];
#pragma unroll
    for (int g = 0; g < GP; g++) {
        m[g] = -INFINITY;
        l[g] = 0.0f;
#pragma unroll
        for (int d = 0; d < kDimsPerLane; d++) acc[g][d] = 0.0f;
    }

    constexpr int BR = kWaves * RPW * kUnroll;
    for (int rb = r0; rb < r1; rb += BR) {
        float4 kf[kUnroll][NF4], vf[kUnroll][NF4];
        bool valid[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int row = rb + (u * kWaves + wave) * RPW + rg;
            valid[u] = row < r1;
            const float *kr = K + (int64_t)(valid[u] ? row : r0) * nkt + li * 4;
            const float *vr = V + (int64_t)(valid[u] ? row : r0) * nkt + li * 4;
#pragma unroll
            for (int c = 0; c < NF4; c++) {
                kf[u][c] = *reinterpret_cast<const float4 *>(kr + c * 4 * LPR);
                vf[u][c] = *reinterpret_cast<const float4 *>(vr + c * 4 * LPR);
            }
        }
        float sc[kUnroll][GP];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
#pragma unroll
            for (int g = 0; g < GP; g++) {
                float s = 0.0f;
#pragma unroll
                for (int c = 0; c < NF4; c++) {
                    s += qf[g][c * 4 + 0] * kf[u][c].x;
                    s += qf[g][c * 4 + 1] * kf[u][c].y;
                    s += qf[g][c * 4 + 2] * kf[u][c].z;
                    s += qf[g][c * 4 + 3] * kf[u][c].w;
                }
#pragma unroll
                for (int off = 1; off < LPR; off <<= 1) s += __shfl_xor(s, off);
                sc[u][g] = valid[u] ? s : -INFINITY;
            }
        }
#pragma unroll
        for (int g = 0; g < GP; g++) {
            float mt = sc[0][g];
#pragma unroll
            for (int u = 1; u < kUnroll; u++) mt = fmaxf(mt, sc[u][g]);
            const float mn = fmaxf(m[g], mt);
            const float ref = (mn == -INFINITY) ? 0.0f : mn;
            const float alpha = fast_exp2(m[g] - ref);
            l[g] *= alpha;
#pragma unroll
            for (int d = 0; d < kDimsPerLane; d++) acc[g][d] *= alpha;
#pragma unroll
            for (int u = 0; u < kUnroll; u++) {
                const float pu = fast_exp2(sc[u][g] - ref);
                l[g] += pu;
#pragma unroll
                for (int c = 0; c < NF4; c++) {
                    acc[g][c * 4 + 0] += pu * vf[u][c].x;
                    acc[g][c * 4 + 1] += pu * vf[u][c].y;
                    acc[g][c * 4 + 2] += pu * vf[u][c].z;
                    acc[g][c * 4 + 3] += pu * vf[u][c].w;
                }
            }
            m[g] = mn;
        }
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

    // Merge the waves through LDS and write the chunk's partial.
    __shared__ float sm[kWaves][GP][HD + 2];
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < GP; g++) {
            if (li == 0) {
                sm[wave][g][0] = m[g];
                sm[wave][g][1] = l[g];
            }
#pragma unroll
            for (int c = 0; c < NF4; c++)
#pragma unroll
                for (int e = 0; e < 4; e++) sm[wave][g][2 + c * 4 * LPR + li * 4 + e] = acc[g][c * 4 + e];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < GP * HD; idx += blockDim.x) {
        const int g = idx / HD;
        const int d = idx - g * HD;
        if (g0 + g >= G) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, sm[w][g][0]);
        const float ref = (M == -INFINITY) ? 0.0f : M;
        float L = 0.0f, A = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            const float f = fast_exp2(sm[w][g][0] - ref);
            L += f * sm[w][g][1];
            A += f * sm[w][g][2 + d];
        }
        const int h = hk * G + g0 + g;
        float *rec = p.part + ((int64_t)cg * p.n_head + h) * (HD + 4);
        if (d == 0) {
            rec[0] = M;
            rec[1] = L;
        }
        rec[4 + d] = A;
    }
}

// One workgroup per (batch entry, query head); thread d owns output dim d.
template <int HD>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeParams p)
{
    const int b = blockIdx.x;
    const int h = blockIdx.y;
    const int c0 = p.cbase[b], c1 = p.cbase[b + 1];
    for (int d = threadIdx.x; d < HD; d += blockDim.x) {
        float M = -INFINITY;
        for (int c = c0; c < c1; c++) M = fmaxf(M, p.part[((int64_t)c * p.n_head + h) * (HD + 4)]);
        float L = 0.0f, A = 0.0f;
        for (int c = c0; c < c1; c++) {
            const float *rec = p.part + ((int64_t)c * p.n_head + h) * (HD + 4);
            const float f = fast_exp2(rec[0] - M);
            L += f * rec[1];
            A += f * rec[4 + d];
        }
        p.out[((int64_t)b * p.n_head + h) * HD + d] = A / L;
    }
}

template <int HD>
hipError_t launch_hd(const DecodeParams &p, hipStream_t s)
{
    const int G = p.n_head / p.n_head_kv;
    const dim3 grid((unsigned)p.total_chunks, (unsigned)p.n_head_kv), block(256);
    for (int g0 = 0; g0 < G; g0 += 8) {
        const int left = G - g0;
        if (left >= 5) decode_split_kernel<HD, 8><<<grid, block, 0, s>>>(p, g0);
        else if (left >= 3) decode_split_kernel<HD, 4><<<grid, block, 0, s>>>(p, g0);
        else if (left == 2) decode_split_kernel<HD, 2><<<grid, block, 0, s>>>(p, g0);
        else decode_split_kernel<HD, 1><<<grid, block, 0, s>>>(p, g0);
    }
    const dim3 cgrid((unsigned)p.n, (unsigned)p.n_head), cblock(HD < 64 ? 64 : HD);
    decode_combine_kernel<HD><<<cgrid, cblock, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

int32_t decode_block_rows(int32_t hd_kv)
{
    const int lpr = hd_kv / kDimsPerLane;
    return kWaves * (64 / lpr) * kUnroll;
}

hipError_t launch_decode(const DecodeParams &p, hipStream_t s)
{
    switch (p.hd_kv) {
    case 16: return launch_hd<16>(p, s);
    case 32: return launch_hd<32>(p, s);
    case 64: return launch_hd<64>(p, s);
    case 128: return launch_hd<128>(p, s);
    case 256: return launch_hd<256>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kvc
