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
//     but a vanishing fraction of rows), and otherwise the wave recomputes the sum as an
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
// cache, so that a unit holds whole 32-value blocks) of one head of q, k or v -- for a
// group of up to 8 tokens.  NEOX pairs (i, i + D/2) and interleaved pairs (2i, 2i+1) of
// a unit are computed together, so the rotation happens in LDS without another launch.
// Rows are reduced by 16 lanes each (four rows per wave at a time), every lane streaming
// 16-byte pieces of its row; the weight rows are read once per token group.
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
constexpr int kXChunk = 512;   // x values per token staged in LDS at a time

// LDS slot (in doubles) of the value pair (e + 2 half, e + 2 half + 1) of a staged x
// chunk, e = 4 li + 64 k the first value of lane li's k-th piece: the pairs of one
// (k, half) are contiguous over li, so the 16 lanes of a row read 256 consecutive bytes
// (no bank conflicts; the other rows of the wave read the same bytes).
__device__ __forceinline__ int xs_slot(int e, int half)
{
    const int k = e >> 6, li = (e >> 2) & 15;
    return ((k * 2 + half) * 16 + li) * 2;
}

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

template <int STYLE, typename KVT, int TT>
__global__ void __launch_bounds__(256) qkv_kernel(QkvParams p, int32_t pairs_per_unit)
{
    __shared__ float ys[TT][kMaxRows];   // [token][local row]
    __shared__ double xs[TT > 1 ? TT : 1][TT > 1 ? kXChunk : 1];   // x chunk, several tokens

    // Unit -> (projection, head, pair range).
    int unit = blockIdx.x;
    int proj = 0;
    if (unit >= p.units_q) {
        unit -= p.units_q;
        proj = 1;
        if (unit >= p.units_kv) {
            unit -= p.units_kv;
            proj = 2;
        }
    }
    const int D = proj == 0 ? p.hd : p.hd_kv;
    const int half = D >> 1;
    const int upr = (half + pairs_per_unit - 1) / pairs_per_unit;   // units per head
    const int head = unit / upr;
    const int i_begin = (unit - head * upr) * pairs_per_unit;
    const int np = min(pairs_per_unit, half - i_begin);
    const int R = 2 * np;
    const bool rot = proj < 2 && STYLE != kNone;
    const bool neox = rot && STYLE == kNeox;
    // Local row lr -> index within the head.  NEOX: first the np first-half rows, then
    // their partners; otherwise the unit's rows in order.
    auto head_row = [&](int lr) {
        if (neox) return lr < np ? i_begin + lr : half + i_begin + (lr - np);
        return 2 * i_begin + lr;
    };
    const float *W = p.w[proj] + (int64_t)head * D * p.d;
    const float *B = p.b[proj] ? p.b[proj] + head * D : nullptr;
    const int t0 = blockIdx.y * TT;
    const int ntk = min(TT, p.nt - t0);

    // Projections.  Row lr is reduced by 16 lanes; lane li takes elements 4 li + 64 k.
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int li = lane % kLanesPerRow;
    for (int base = 0; base < R; base += 16) {
        const int lr = base + wave * 4 + lane / kLanesPerRow;
        const bool row_ok = lr < R;
        const float *wr = W + (int64_t)head_row(row_ok ? lr : 0) * p.d;
        // Feed op(t, x, w) every (x, w) element pair of this lane's share of the row, as
        // f64 (each f32 x f32 product is then exact): a lane takes elements 4 li + 64 k.
        auto accumulate = [&](auto &&op) {
            if constexpr (TT == 1) {
                // One token: the step streams the weights, so each lane first issues the
                // loads of up to kBatch pieces of its row (and of x), then does their
                // arithmetic.
                constexpr int kBatch = 16;
                const float *xr = p.x + (int64_t)t0 * p.d;
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
                            op(0, (double)xb[k].x, (double)wb[k].x);
                            op(0, (double)xb[k].y, (double)wb[k].y);
                            op(0, (double)xb[k].z, (double)wb[k].z);
                            op(0, (double)xb[k].w, (double)wb[k].w);
                        }
                    }
                }
            } else {
                // Several tokens: each weight piece serves all of them.  The group's x
                // rows pass through LDS as f64 in chunks of kXChunk values (one batch of
                // loads per thread; rows past the group's tokens read as zeros), and each
                // lane loads its kPieces weight pieces of the chunk together, before the
                // staging, so a chunk costs about one memory round trip.  The arithmetic runs over all TT tokens
                // without branches, token-minor, so consecutive operations feed
                // independent sums.  Every thread of the block reaches the barriers: the
                // row loop is uniform across the block.  (Loading the next chunk during
                // the current one's arithmetic needs ~250 registers and ran slower.)
                constexpr int kPieces = kXChunk / (4 * kLanesPerRow);
                for (int c0 = 0; c0 < p.d; c0 += kXChunk) {
                    const int cn = min(kXChunk, p.d - c0);
                    // This chunk's weight pieces are requested first: their round trip
                    // overlaps the x staging and its barriers.
                    float4 wb[kPieces];
#pragma unroll
                    for (int k = 0; k < kPieces; k++) {
                        const int e = li * 4 + k * 4 * kLanesPerRow;
                        if (e < cn) wb[k] = *reinterpret_cast<const float4 *>(wr + c0 + e);
                    }
                    __syncthreads();   // the previous chunk's readers are done
                    for (int idx = threadIdx.x; idx < TT * (kXChunk / 4); idx += blockDim.x) {
                        const int t = idx / (kXChunk / 4);
                        const int e = (idx - t * (kXChunk / 4)) * 4;
                        float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                        if (t < ntk && e < cn)
                            v = *reinterpret_cast<const float4 *>(p.x + (int64_t)(t0 + t) * p.d + c0 + e);
                        *reinterpret_cast<double2 *>(&xs[t][xs_slot(e, 0)]) = make_double2(v.x, v.y);
                        *reinterpret_cast<double2 *>(&xs[t][xs_slot(e, 1)]) = make_double2(v.z, v.w);
                    }
                    __syncthreads();
#pragma unroll
                    for (int k = 0; k < kPieces; k++) {
                        const int e = li * 4 + k * 4 * kLanesPerRow;
                        if (e < cn) {
                            const double wv[4] = {wb[k].x, wb[k].y, wb[k].z, wb[k].w};
                            double xv[TT][4];
#pragma unroll
                            for (int t = 0; t < TT; t++) {
                                const double2 a = *reinterpret_cast<const double2 *>(&xs[t][xs_slot(e, 0)]);
                                const double2 b = *reinterpret_cast<const double2 *>(&xs[t][xs_slot(e, 1)]);
                                xv[t][0] = a.x; xv[t][1] = a.y; xv[t][2] = b.x; xv[t][3] = b.y;
                            }
#pragma unroll
                            for (int c = 0; c < 4; c++)
#pragma unroll
                                for (int t = 0; t < TT; t++) op(t, xv[t][c], wv[c]);
                        }
                    }
                }
            }
        };

        // Fast path: the plain f64 sum S of the products and the sum A of their
        // magnitudes.  Each product is exact and every partial sum is far from the f64
        // range limits, so |S - exact| <= gamma_m * sum|products| with m <= d/16 + 8
        // roundings on any path; err = 4 m u A + 2 u |S| (u = 2^-53) covers that bound,
        // the rounding of A, and the rounding of S -/+ err themselves.  Rounding to f32
        // is monotonic, so when both ends of [S - err, S + err] round to the same f32
        // (bit for bit: a straddled zero has two signs), that f32 is the one nearest the
        // exact sum.  Otherwise (a value within err of an f32 rounding boundary, or a
        // non-finite sum) that row and token is recomputed exactly below.
        double S[TT], A[TT];
#pragma unroll
        for (int t = 0; t < TT; t++) S[t] = A[t] = 0.0;
        accumulate([&](int t, double xv, double wv) {
            S[t] = fma(xv, wv, S[t]);
            A[t] = fma(fabs(xv), fabs(wv), A[t]);
        });
#pragma unroll
        for (int t = 0; t < TT; t++) {
#pragma unroll
            for (int off = kLanesPerRow / 2; off >= 1; off >>= 1) {
                S[t] += __shfl_xor(S[t], off);
                A[t] += __shfl_xor(A[t], off);
            }
        }
        // Longest rounding chain: a lane's ceil(d / 64) * 4 products plus 4 merge levels.
        const double kErr = 4.0 * (double)(p.d / 16 + 8) * 0x1p-53;
        uint32_t unsure = 0;   // tokens some row of this lane's wave could not settle
#pragma unroll
        for (int t = 0; t < TT; t++) {
            const double err = kErr * A[t] + 0x1p-52 * fabs(S[t]);
            const float lo32 = (float)(S[t] - err), hi32 = (float)(S[t] + err);
            const bool certain = t >= ntk || (__builtin_isfinite(S[t]) && __builtin_isfinite(err) &&
                                              __float_as_uint(lo32) == __float_as_uint(hi32));
            if (__any(!certain)) unsure |= 1u << t;
            if (row_ok && li == 0 && t < ntk) ys[t][lr] = B ? lo32 + B[head_row(lr)] : lo32;
        }
        // Exact sum for an unsettled token of this wave's rows (rare: a value within the
        // bound of an f32 rounding boundary): an unevaluated pair of f64 values (hi + lo,
        // hi accumulated with the error-free TwoSum and the errors in lo), lane partials
        // merged the same way, the pair rounded to f32 once.  x and w come from global
        // memory (no barrier: the choice is per wave); every row of the wave recomputes,
        // and the exact value replaces the stored one (they agree where both exist).
        while (unsure) {
            const int t = __builtin_ctz(unsure);
            unsure &= unsure - 1;
            const float *xr = p.x + (int64_t)(t0 + t) * p.d;
            double hi = 0.0, lo = 0.0;
            for (int i0 = li * 4; i0 < p.d; i0 += 4 * 4 * kLanesPerRow) {
                float4 wb[4], xb[4];
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    const int i = i0 + k * 4 * kLanesPerRow;
                    if (i < p.d) {
                        wb[k] = *reinterpret_cast<const float4 *>(wr + i);
                        xb[k] = *reinterpret_cast<const float4 *>(xr + i);
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    if (i0 + k * 4 * kLanesPerRow < p.d) {
                        dd_add(hi, lo, (double)xb[k].x * (double)wb[k].x);
                        dd_add(hi, lo, (double)xb[k].y * (double)wb[k].y);
                        dd_add(hi, lo, (double)xb[k].z * (double)wb[k].z);
                        dd_add(hi, lo, (double)xb[k].w * (double)wb[k].w);
                    }
                }
            }
#pragma unroll
            for (int off = kLanesPerRow / 2; off >= 1; off >>= 1) {
                const double oh = __shfl_xor(hi, off);
                const double ol = __shfl_xor(lo, off);
                dd_merge(hi, lo, oh, ol);
            }
            const float ye = dd_to_f32(hi, lo);
            if (row_ok && li == 0) ys[t][lr] = B ? ye + B[head_row(lr)] : ye;
        }
    }
    __syncthreads();

    // RoPE in LDS (q and k), with the append kernel's rotate_pair and table rows.
    if (rot) {
        const float2 *tab = proj == 0 ? p.tab_q : p.tab_k;
        for (int idx = threadIdx.x; idx < ntk * np; idx += blockDim.x) {
            const int t = idx / np;
            const int il = idx - t * np;
            const int lr0 = neox ? il : 2 * il;
            const int lr1 = neox ? np + il : 2 * il + 1;
            const float2 cs = tab[(int64_t)p.ipos[t0 + t] * half + i_begin + il];
            float y0, y1;
            rotate_pair(ys[t][lr0], ys[t][lr1], cs, y0, y1);
            ys[t][lr0] = y0;
            ys[t][lr1] = y1;
        }
        __syncthreads();
    }

    if (proj == 0) {
        for (int idx = threadIdx.x; idx < ntk * R; idx += blockDim.x) {
            const int t = idx / R;
            const int lr = idx - t * R;
            p.q_out[((int64_t)(t0 + t) * p.n_head + head) * p.hd + head_row(lr)] = ys[t][lr];
        }
        return;
    }

    // K or V rows: 4 consecutive local rows are 4 consecutive head dims (np is a
    // multiple of 4 for every supported hd_kv); for Q8_0 the R/4 quads of a token are a
    // multiple of 8, so the 8 lanes of a 32-value block are aligned and active together.
    const int nkt = p.n_head_kv * p.hd_kv;
    char *cache = static_cast<char *>(proj == 1 ? p.kc : p.vc);
    const int nq = R / 4;
    for (int idx = threadIdx.x; idx < ntk * nq; idx += blockDim.x) {
        const int t = idx / nq;
        const int qd = idx - t * nq;
        const int lr = 4 * qd;
        const float4 y = make_float4(ys[t][lr], ys[t][lr + 1], ys[t][lr + 2], ys[t][lr + 3]);
        const int j = head * p.hd_kv + head_row(lr);   // value index in the row
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

template <int STYLE, typename KVT>
void launch_style_fmt(const QkvParams &p, int32_t ppu, hipStream_t s)
{
    const int units = p.units_q + 2 * p.units_kv;
    if (p.nt == 1) {
        qkv_kernel<STYLE, KVT, 1><<<dim3(units, 1), 256, 0, s>>>(p, ppu);
    } else {
        qkv_kernel<STYLE, KVT, 8><<<dim3(units, (p.nt + 7) / 8), 256, 0, s>>>(p, ppu);
    }
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
