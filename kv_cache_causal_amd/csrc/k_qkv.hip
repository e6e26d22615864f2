// Fused decode step: q/k/v projections, their biases, RoPE on q and k, and the K/V
// store, in one kernel.
//
// "13 · The decode loop and graph reuse" §2.3: on a GPU build a one-token step merges
// three matmuls, three biases, two RoPEs and two KV stores into a single operation;
// §3.4 item 5: the fused and the unfused paths must agree bit for bit.  Here "unfused"
// is the projection followed by kv_append_rope, and the kernel reproduces it exactly:
//   * each projection output is the f32 nearest to the exact dot product x . w_j: every
//     f32 x f32 product is exact in f64; a plain f64 sum with a rigorous error bound
//     settles the rounding whenever the bound's whole interval rounds to one f32 (all
//     but a vanishing fraction of rows), and otherwise a wave recomputes the sum as an
//     unevaluated pair of f64 values (hi + lo, hi accumulated with the error-free TwoSum
//     and the errors in lo), merges lane partials the same way and rounds the pair to
//     f32 once, through round-to-odd at f64 precision (53 >= 24 + 2 bits makes that one
//     correct rounding); the bias is then added in f32;
//   * the rotation, the binary16 rounding and the Q8_0 quantization are the append
//     kernel's own functions (kvc_device.hpp).
// The pages' reading of the matmul's precision is only that fused and unfused agree;
// the exact-then-round definition makes the result independent of summation order, so
// it can be checked against any exact evaluation.
//
// Work split: a workgroup owns one "unit" -- up to 8 rotation pairs (32 for a Q8_0
// cache, so that a unit holds whole 32-value blocks) of one head of q, k or v -- for all
// the call's tokens.  NEOX pairs (i, i + D/2) and interleaved pairs (2i, 2i+1) of a unit
// are computed together, so the rotation happens in LDS without another launch.
//   * Up to 4 tokens (qkv_one_kernel, one workgroup per unit and token): rows are
//     reduced by 16 lanes each (four rows per wave at a time), every lane streaming
//     16-byte pieces of its row.
//   * Several tokens (qkv_mfma_kernel, one workgroup per unit and tile of 16 tokens):
//     the unit's rows times the tokens' x as f64 matrix products
//     (v_mfma_f64_16x16x4f64), so each operand a lane holds feeds 16 products.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kNeox = 0, kInterleaved = 1, kNone = 2;
constexpr int kMaxRows = 64;   // rows of a unit (32 pairs)
constexpr int kLanesPerRow = 16;
constexpr int kOneTokenMax = 4;   // up to this many tokens: a workgroup per (unit, token)
typedef double doublex4 __attribute__((ext_vector_type(4)));

// Error-free sum: s + e == a + b exactly (s = fl(a + b)).
__device__ __forceinline__ void two_sum(double a, double b, double &s, double &e)
{
#pragma clang fp contract(off)
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

// (hi, lo) += p, p exact.
__device__ __forceinline__ void dd_add(double &hi, double &lo, double p)
{
#pragma clang fp contract(off)
    double s, e;
    two_sum(hi, p, s, e);
    hi = s;
    lo += e;
}

// (hi, lo) += (bhi, blo).
__device__ __forceinline__ void dd_merge(double &hi, double &lo, double bhi, double blo)
{
#pragma clang fp contract(off)
    double s, e;
    two_sum(hi, bhi, s, e);
    hi = s;
    lo += e + blo;
}

// The f32 nearest to hi + lo: normalise, round to odd at f64 precision, round to f32.
__device__ __forceinline__ float dd_to_f32(double hi, double lo)
{
    double h, l;
    two_sum(hi, lo, h, l);
    if (l != 0.0 && h != 0.0) {
        unsigned long long bits = (unsigned long long)__double_as_longlong(h);
        if (!(bits & 1ull)) {
            // The neighbour of h on l's side is odd: step the magnitude up when l has h's
            // sign, down otherwise.
            bits = ((l > 0.0) == (h > 0.0)) ? bits + 1ull : bits - 1ull;
            h = __longlong_as_double((long long)bits);
        }
    }
    return (float)h;
}

// What a workgroup computes: rows [0, R) of projection `proj` (0 q, 1 k, 2 v) of head
// `head` (head dim D), the R = 2 np rows of rotation pairs [i_begin, i_begin + np).
struct Unit {
    int proj, D, half, head, i_begin, np, R;
    bool rot, neox;
    // Local row lr -> index within the head.  NEOX: first the np first-half rows, then
    // their partners; otherwise the unit's rows in order.
    __device__ int head_row(int lr) const
    {
        if (neox) return lr < np ? i_begin + lr : half + i_begin + (lr - np);
        return 2 * i_begin + lr;
    }
};

template <int STYLE>
__device__ __forceinline__ Unit unit_of(const QkvParams &p, int unit, int pairs_per_unit)
{
    Unit u;
    u.proj = 0;
    if (unit >= p.units_q) {
        unit -= p.units_q;
        u.proj = 1;
        if (unit >= p.units_kv) {
            unit -= p.units_kv;
            u.proj = 2;
        }
    }
    u.D = u.proj == 0 ? p.hd : p.hd_kv;
    u.half = u.D >> 1;
    const int upr = (u.half + pairs_per_unit - 1) / pairs_per_unit;   // units per head
    u.head = unit / upr;
    u.i_begin = (unit - u.head * upr) * pairs_per_unit;
    u.np = min(pairs_per_unit, u.half - u.i_begin);
    u.R = 2 * u.np;
    u.rot = u.proj < 2 && STYLE != kNone;
    u.neox = u.rot && STYLE == kNeox;
    return u;
}

// The certified rounding of a plain f64 sum S: |S - exact| <= gamma_m * A for a bound A
// on the sum of the products' magnitudes and m roundings on the longest chain;
// err = 4 m u A + 2 u |S| (u = 2^-53) covers that, the rounding of A, and the rounding
// of S -/+ err themselves.  Rounding to f32 is monotonic, so when both ends of
// [S - err, S + err] round to the same f32 (bit for bit: a straddled zero has two signs),
// that f32 is the one nearest the exact sum.  Otherwise (a value within err of an f32
// rounding boundary, or a non-finite sum) the caller recomputes it exactly.
__device__ __forceinline__ bool certify(double S, double A, int m, float &y)
{
    const double err = 4.0 * (double)m * 0x1p-53 * A + 0x1p-52 * fabs(S);
    const float lo32 = (float)(S - err), hi32 = (float)(S + err);
    y = lo32;
    return __builtin_isfinite(S) && __builtin_isfinite(err) &&
           __float_as_uint(lo32) == __float_as_uint(hi32);
}

// The exact f32 projection of x-row xr on weight row wr by 64 lanes (an unevaluated f64
// pair per lane, TwoSum-merged across the wave, rounded once).
__device__ float exact_row_wave(const float *xr, const float *wr, int d, int lane)
{
    double hi = 0.0, lo = 0.0;
    for (int i = lane * 4; i < d; i += 4 * 64) {
        const float4 wb = *reinterpret_cast<const float4 *>(wr + i);
        const float4 xb = *reinterpret_cast<const float4 *>(xr + i);
        dd_add(hi, lo, (double)xb.x * (double)wb.x);
        dd_add(hi, lo, (double)xb.y * (double)wb.y);
        dd_add(hi, lo, (double)xb.z * (double)wb.z);
        dd_add(hi, lo, (double)xb.w * (double)wb.w);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const double oh = __shfl_xor(hi, off);
        const double ol = __shfl_xor(lo, off);
        dd_merge(hi, lo, oh, ol);
    }
    return dd_to_f32(hi, lo);
}

// RoPE in LDS (q and k) with the append kernel's rotate_pair and table rows, then the
// stores: q to q_out, k/v rows to the cache with the append's own binary16 / Q8_0
// functions.  ys[t][lr] holds the projection (bias added) of local row lr, token t0 + t.
// Every thread of the block calls it after a barrier that made ys complete.
template <int STYLE, typename KVT>
__device__ void finish_unit(const QkvParams &p, const Unit &u, float (*ys)[kMaxRows], int t0,
                            int ntk)
{
    if (u.rot) {
        const float2 *tab = u.proj == 0 ? p.tab_q : p.tab_k;
        for (int idx = threadIdx.x; idx < ntk * u.np; idx += blockDim.x) {
            const int t = idx / u.np;
            const int il = idx - t * u.np;
            const int lr0 = u.neox ? il : 2 * il;
            const int lr1 = u.neox ? u.np + il : 2 * il + 1;
            const float2 cs = tab[(int64_t)p.ipos[t0 + t] * u.half + u.i_begin + il];
            float y0, y1;
            rotate_pair(ys[t][lr0], ys[t][lr1], cs, y0, y1);
            ys[t][lr0] = y0;
            ys[t][lr1] = y1;
        }
        __syncthreads();
    }

    if (u.proj == 0) {
        for (int idx = threadIdx.x; idx < ntk * u.R; idx += blockDim.x) {
            const int t = idx / u.R;
            const int lr = idx - t * u.R;
            p.q_out[((int64_t)(t0 + t) * p.n_head + u.head) * p.hd + u.head_row(lr)] = ys[t][lr];
        }
        return;
    }

    // K or V rows: 4 consecutive local rows are 4 consecutive head dims (np is a
    // multiple of 4 for every supported hd_kv); for Q8_0 the R/4 quads of a token are a
    // multiple of 8, so the 8 lanes of a 32-value block are aligned and active together.
    const int nkt = p.n_head_kv * p.hd_kv;
    char *cache = static_cast<char *>(u.proj == 1 ? p.kc : p.vc);
    const int nq = u.R / 4;
    for (int idx = threadIdx.x; idx < ntk * nq; idx += blockDim.x) {
        const int t = idx / nq;
        const int qd = idx - t * nq;
        const int lr = 4 * qd;
        const float4 y = make_float4(ys[t][lr], ys[t][lr + 1], ys[t][lr + 2], ys[t][lr + 3]);
        const int j = u.head * p.hd_kv + u.head_row(lr);   // value index in the row
        const int64_t reg = ((int64_t)p.iseq[t0 + t] * p.n_layer + p.layer) * p.region_bytes;
        const int64_t row = p.ipos[t0 + t];
        if constexpr (std::is_same<KVT, int8_t>::value) {
            int8_t *codes = reinterpret_cast<int8_t *>(cache + reg) + row * nkt + j;
            _Float16 *scale = reinterpret_cast<_Float16 *>(cache + reg + p.scale_off) +
                              q8_scale_index(row, j, p.hd_kv, p.scale_off / nkt);
            q8_store4(y, codes, scale, idx);
        } else {
            store4(reinterpret_cast<KVT *>(cache + reg) + row * nkt + j, y);
        }
    }
}

// One token per workgroup (token blockIdx.y): the step streams the weights.  Row lr is
// reduced by 16 lanes; lane li takes elements 4 li + 64 k, first issuing the loads of up
// to kBatch pieces of its row (and of x), then doing their arithmetic: the plain f64 sum
// S of the exact products and A, the sum of their magnitudes.
template <int STYLE, typename KVT>
__global__ void __launch_bounds__(256) qkv_one_kernel(QkvParams p, int32_t pairs_per_unit)
{
    __shared__ float ys[1][kMaxRows];
    const Unit u = unit_of<STYLE>(p, blockIdx.x, pairs_per_unit);
    const float *W = p.w[u.proj] + (int64_t)u.head * u.D * p.d;
    const float *B = p.b[u.proj] ? p.b[u.proj] + u.head * u.D : nullptr;
    const int t0 = blockIdx.y;
    const float *xr = p.x + (int64_t)t0 * p.d;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane % kLanesPerRow;
    // Longest rounding chain: a lane's ceil(d / 64) * 4 products plus 4 merge levels.
    const int m = p.d / 16 + 8;
    for (int base = 0; base < u.R; base += 16) {
        const int lr = base + wave * 4 + lane / kLanesPerRow;
        const bool row_ok = lr < u.R;
        const float *wr = W + (int64_t)u.head_row(row_ok ? lr : 0) * p.d;
        constexpr int kBatch = 16;
        double S = 0.0, A = 0.0;
        for (int i0 = li * 4; i0 < p.d; i0 += kBatch * 4 * kLanesPerRow) {
            float4 wb[kBatch], xb[kBatch];
#pragma unroll
            for (int k = 0; k < kBatch; k++) {
                const int i = i0 + k * 4 * kLanesPerRow;
                if (i < p.d) {
                    wb[k] = *reinterpret_cast<const float4 *>(wr + i);
                    xb[k] = *reinterpret_cast<const float4 *>(xr + i);
                }
            }
#pragma unroll
            for (int k = 0; k < kBatch; k++) {
                if (i0 + k * 4 * kLanesPerRow < p.d) {
                    const double xv[4] = {xb[k].x, xb[k].y, xb[k].z, xb[k].w};
                    const double wv[4] = {wb[k].x, wb[k].y, wb[k].z, wb[k].w};
#pragma unroll
                    for (int c = 0; c < 4; c++) {
                        S = fma(xv[c], wv[c], S);
                        A = fma(fabs(xv[c]), fabs(wv[c]), A);
                    }
                }
            }
        }
#pragma unroll
        for (int off = kLanesPerRow / 2; off >= 1; off >>= 1) {
            S += __shfl_xor(S, off);
            A += __shfl_xor(A, off);
        }
        float y;
        const bool certain = certify(S, A, m, y);
        if (row_ok && li == 0) ys[0][lr] = B ? y + B[u.head_row(lr)] : y;
        // Exact sum when some row of the wave is unsettled (rare: a value within the
        // bound of an f32 rounding boundary), 16 lanes per row; x and w come from global
        // memory (no barrier: the choice is per wave), and the exact value replaces the
        // stored one (they agree where both exist).
        if (__any(!certain)) {
            double hi = 0.0, lo = 0.0;
            for (int i = li * 4; i < p.d; i += 4 * kLanesPerRow) {
                const float4 wb = *reinterpret_cast<const float4 *>(wr + i);
                const float4 xb = *reinterpret_cast<const float4 *>(xr + i);
                dd_add(hi, lo, (double)xb.x * (double)wb.x);
                dd_add(hi, lo, (double)xb.y * (double)wb.y);
                dd_add(hi, lo, (double)xb.z * (double)wb.z);
                dd_add(hi, lo, (double)xb.w * (double)wb.w);
            }
#pragma unroll
            for (int off = kLanesPerRow / 2; off >= 1; off >>= 1) {
                const double oh = __shfl_xor(hi, off);
                const double ol = __shfl_xor(lo, off);
                dd_merge(hi, lo, oh, ol);
            }
            const float ye = dd_to_f32(hi, lo);
            if (row_ok && li == 0) ys[0][lr] = B ? ye + B[u.head_row(lr)] : ye;
        }
    }
    __syncthreads();
    finish_unit<STYLE, KVT>(p, u, ys, t0, 1);
}

// Several tokens (2 .. kInlineTokens): a workgroup takes one unit and one tile of up
// to 16 tokens (blockIdx.y).  The unit's R rows form nrt tiles of 16 (rows past R repeat
// row 0 and are dropped; x of absent tokens is 0); each wave takes one row tile and one
// of ks = 4 / nrt parts of the reduction dimension, and accumulates D[row][token] with
// v_mfma_f64_16x16x4f64 (A = 16 rows x 4 weight values, B = 4 x values x 16 tokens;
// A[i][k] and B[k][j] come from lane i + 16 k, resp. j + 16 k, and D[i][j] lands in
// register i / 4 of lane j + 16 (i % 4) -- checked on the hardware).  Within a group of
// 16 reduction indices, step c of the 4 takes index 4 k + c in slot k, so a lane's 4
// values of a group are one float4 of its weight row and one of its token's x row.
// Products of f32 values are exact in f64; per output, a wave's chain has at most kper
// additions (4 per step, however the matrix core orders them) and the ks partials add
// ks - 1 more.  The error bound takes A = |x|_2 |w|_2 (1 + 2^-30) (Cauchy-Schwarz),
// from f64 sums of squares, each within a relative gamma_d of its exact value, far
// inside the margin; a bound that is less tight only sends more values to the exact path.
template <int STYLE, typename KVT>
__global__ void __launch_bounds__(256) qkv_mfma_kernel(QkvParams p, int32_t pairs_per_unit)
{
    constexpr int TM = 16;   // tokens per workgroup
    __shared__ float ys[TM][kMaxRows];
    __shared__ double sp[4][16 * TM];      // per wave: D[i][t] at i * TM + t
    __shared__ double swq[4][16];          // per wave: sum of w^2 of its tile's rows
    __shared__ double sxq[4][TM];          // per wave: sum of x^2 of each token
    __shared__ unsigned long long s_unsure[TM];   // per token: rows to recompute exactly

    const Unit u = unit_of<STYLE>(p, blockIdx.x, pairs_per_unit);
    const float *W = p.w[u.proj] + (int64_t)u.head * u.D * p.d;
    const float *B = p.b[u.proj] ? p.b[u.proj] + u.head * u.D : nullptr;
    const int t0 = blockIdx.y * TM;
    const int ntk = min(TM, p.nt - t0);
    const int nrt = (u.R + 15) >> 4;
    const int ks = 4 / nrt;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, kk = lane >> 4;
    const int rt = wave % nrt, kp = wave / nrt;
    const bool active = kp < ks;
    const int kper = (p.d + 16 * ks - 1) / (16 * ks) * 16;   // reduction indices per part
    const int kb = kp * kper, ke = min(p.d, kb + kper);
    if (threadIdx.x < TM) s_unsure[threadIdx.x] = 0ull;

    doublex4 acc = doublex4{0.0, 0.0, 0.0, 0.0};
    double wsq = 0.0, xsq = 0.0;
    if (active) {
        const int lr = rt * 16 + l16;
        const float *wr = W + (int64_t)u.head_row(lr < u.R ? lr : 0) * p.d;
        const float *xr = l16 < ntk ? p.x + (int64_t)(t0 + l16) * p.d : nullptr;
        // Groups of 16 reduction indices, kG at a time, in two register sets: the loads
        // of the next batch are in flight while this one's products run.
        constexpr int kG = 4;
        float4 wA[kG], xA[kG], wB[kG], xB[kG];
        auto load = [&](float4 (&wv)[kG], float4 (&xv)[kG], int g0) {
#pragma unroll
            for (int g = 0; g < kG; g++) {
                const int e = g0 + 16 * g + 4 * kk;   // e < ke implies e + 3 < ke
                const bool in = e < ke;
                wv[g] = in ? *reinterpret_cast<const float4 *>(wr + e) : make_float4(0.f, 0.f, 0.f, 0.f);
                xv[g] = (in && xr) ? *reinterpret_cast<const float4 *>(xr + e) : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        };
        auto products = [&](const float4 (&wv)[kG], const float4 (&xv)[kG]) {
#pragma unroll
            for (int g = 0; g < kG; g++) {
                const double w4[4] = {wv[g].x, wv[g].y, wv[g].z, wv[g].w};
                const double x4[4] = {xv[g].x, xv[g].y, xv[g].z, xv[g].w};
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    wsq = fma(w4[c], w4[c], wsq);
                    xsq = fma(x4[c], x4[c], xsq);
                    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(w4[c], x4[c], acc, 0, 0, 0);
                }
            }
        };
        const int nb = (ke - kb + 16 * kG - 1) / (16 * kG);   // batches (0 if kb >= ke)
        if (nb > 0) load(wA, xA, kb);
        for (int b = 0; b < nb; b += 2) {
            if (b + 1 < nb) load(wB, xB, kb + (b + 1) * 16 * kG);
            products(wA, xA);
            if (b + 1 >= nb) break;
            if (b + 2 < nb) load(wA, xA, kb + (b + 2) * 16 * kG);
            products(wB, xB);
        }
        // Lane (l16, kk) holds its slot's share of row l16's and token l16's squares.
#pragma unroll
        for (int off = 16; off <= 32; off <<= 1) {
            wsq += __shfl_xor(wsq, off);
            xsq += __shfl_xor(xsq, off);
        }
        if (kk == 0) {
            swq[wave][l16] = wsq;
            sxq[wave][l16] = xsq;
        }
#pragma unroll
        for (int r = 0; r < 4; r++) sp[wave][(4 * r + kk) * TM + l16] = acc[r];
    }
    __syncthreads();

    // Sum the parts (in part order), certify, and mark what needs the exact path.
    const int m = kper + ks + 8;
    for (int idx = threadIdx.x; idx < u.R * ntk; idx += blockDim.x) {
        const int lr = idx / ntk;
        const int t = idx - lr * ntk;
        const int trt = lr >> 4, i = lr & 15;
        double S = 0.0, w2 = 0.0, x2 = 0.0;
        for (int q = 0; q < ks; q++) {
            const int w = trt + q * nrt;
            S += sp[w][i * TM + t];
            w2 += swq[w][i];
            x2 += sxq[q * nrt][t];
        }
        const double A = sqrt(x2) * sqrt(w2) * (1.0 + 0x1p-30);
        float y;
        if (!certify(S, A, m, y)) atomicOr(&s_unsure[t], 1ull << lr);
        ys[t][lr] = B ? y + B[u.head_row(lr)] : y;
    }
    __syncthreads();

    // Exact path for the marked (row, token) pairs: wave w takes tokens w, w + 4, ...
    for (int t = wave; t < ntk; t += 4) {
        unsigned long long rows = s_unsure[t];
        while (rows) {
            const int lr = __builtin_ctzll(rows);
            rows &= rows - 1;
            const float ye = exact_row_wave(p.x + (int64_t)(t0 + t) * p.d,
                                            W + (int64_t)u.head_row(lr) * p.d, p.d, lane);
            if (lane == 0) ys[t][lr] = B ? ye + B[u.head_row(lr)] : ye;
        }
    }
    __syncthreads();
    finish_unit<STYLE, KVT>(p, u, ys, t0, ntk);
}

template <int STYLE, typename KVT>
void launch_style_fmt(const QkvParams &p, int32_t ppu, hipStream_t s)
{
    const int units = p.units_q + 2 * p.units_kv;
    if (p.nt <= kOneTokenMax) qkv_one_kernel<STYLE, KVT><<<dim3(units, p.nt), 256, 0, s>>>(p, ppu);
    else qkv_mfma_kernel<STYLE, KVT><<<dim3(units, (p.nt + 15) / 16), 256, 0, s>>>(p, ppu);
}

template <typename KVT>
void launch_fmt(const QkvParams &p, int32_t ppu, hipStream_t s)
{
    switch (p.style) {
    case kNeox: launch_style_fmt<kNeox, KVT>(p, ppu, s); break;
    case kInterleaved: launch_style_fmt<kInterleaved, KVT>(p, ppu, s); break;
    default: launch_style_fmt<kNone, KVT>(p, ppu, s); break;
    }
}

}  // namespace

int32_t qkv_pairs_per_unit(int32_t kv_fmt) { return kv_fmt == kFmtQ8 ? 32 : 8; }

hipError_t launch_qkv(const QkvParams &p, hipStream_t s)
{
    if (p.nt <= 0) return hipSuccess;
    const int32_t ppu = qkv_pairs_per_unit(p.kv_fmt);
    if (p.kv_fmt == kFmtQ8) launch_fmt<int8_t>(p, ppu, s);
    else if (p.kv_fmt == kFmtF16) launch_fmt<_Float16>(p, ppu, s);
    else launch_fmt<float>(p, ppu, s);
    return hipGetLastError();
}

}  // namespace kvc
