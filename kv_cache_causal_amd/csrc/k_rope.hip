// RoPE cos/sin table and K1: rotate q and k at positions given as data, store K/V rows.
//
// "11 · Attention, vec ops, and the KV cache":
//   §2.3  RoPE: subspace i turns at speed freq_scale / base^(2i/hd); the angle is
//         position x speed; each pair rotates as a 2-D vector.
//   §3.2.2 the pair layouts: NEOX (i, i + hd/2) and interleaved (2i, 2i + 1).
//   §3.2.3 the store: row t of this step goes to offset pos[t] x row width of its layer's
//         region, a plain copy of the (rotated) k row and the v row.
// "IV.2: Zero-copy KV cache": the append writes one row in place, no reallocation and no
// copy of the rows already there.
// Region formats ("11 · ..." §2.5 "Storage"): f32, binary16 (rounded to nearest even),
// or Q8_0 blocks of 32 values (scale max|x| / 127 stored as binary16, codes rounded
// half away from zero with the f32 reciprocal of the f32 scale: the GGML block).
//
// Reproducibility: the table holds, for every position p < capacity and pair i, the f32
// nearest to cos/sin of the f32 angle f32(p) * speed_i, with speed_i the f32 nearest to
// the exact expression -- each one certified correctly rounded.  The values are first
// evaluated in f64 (pow, cos, sin) with a stated bound on their error; an f64 value is
// rounded to f32 only when no f32 rounding boundary (midpoint of two neighbouring f32)
// lies within that bound of it, which makes the rounding the same as that of the exact
// value.  The rest (near-ties: about one value in 10^7, and none on the workloads' grids)
// is evaluated again in double-double arithmetic: the angle reduced modulo pi/2 exactly
// (Payne-Hanek: the f32 angle times a window of the binary digits of 2/pi, in integer
// arithmetic), cos and sin of the reduced angle by their Taylor series, the speed as
// freq_scale * exp(-(2i/hd) ln base) with exp by its series and ln by a Newton step --
// about 100 correct bits -- and rounded once.  The rotation (rotate_pair,
// kvc_device.hpp) is compiled with FMA contraction off, so each product and each sum is
// rounded on its own and the result is the same bits as any correctly rounded IEEE
// evaluation of the same formula.
#include <hip/hip_runtime.h>

#include "kvc.h"
#include "kvc_device.hpp"
#include "kvc_internal.hpp"
#include "rope_consts.hpp"

namespace kvc {
namespace {

constexpr int kNeox = 0, kInterleaved = 1, kNone = 2;

// ---- Double-double arithmetic (about 106 significant bits): a value is hi + lo with
// |lo| <= half an ulp of hi.  The error-free transformations need every operation
// rounded as written, so contraction into fused multiply-adds is off in them.
struct DD {
    double hi, lo;
};

__device__ __forceinline__ DD dd_two_sum(double a, double b)
{
#pragma clang fp contract(off)
    const double s = a + b;
    const double bb = s - a;
    return DD{s, (a - (s - bb)) + (b - bb)};
}

__device__ __forceinline__ DD dd_fast_two_sum(double a, double b)   // |a| >= |b|
{
#pragma clang fp contract(off)
    const double s = a + b;
    return DD{s, b - (s - a)};
}

__device__ __forceinline__ DD dd_two_prod(double a, double b)
{
#pragma clang fp contract(off)
    const double p = a * b;
    return DD{p, fma(a, b, -p)};
}

__device__ __forceinline__ DD dd_neg(DD a) { return DD{-a.hi, -a.lo}; }

__device__ DD dd_add(DD a, DD b)
{
#pragma clang fp contract(off)
    DD s = dd_two_sum(a.hi, b.hi);
    const DD t = dd_two_sum(a.lo, b.lo);
    s.lo += t.hi;
    s = dd_fast_two_sum(s.hi, s.lo);
    s.lo += t.lo;
    return dd_fast_two_sum(s.hi, s.lo);
}

__device__ DD dd_mul(DD a, DD b)
{
#pragma clang fp contract(off)
    DD p = dd_two_prod(a.hi, b.hi);
    p.lo += a.hi * b.lo + a.lo * b.hi;
    return dd_fast_two_sum(p.hi, p.lo);
}

__device__ DD dd_mul_d(DD a, double b)
{
#pragma clang fp contract(off)
    DD p = dd_two_prod(a.hi, b);
    p.lo += a.lo * b;
    return dd_fast_two_sum(p.hi, p.lo);
}

// a / b for a double b, by three quotient digits.
__device__ DD dd_div_d(DD a, double b)
{
    const double q1 = a.hi / b;
    DD r = dd_add(a, dd_neg(dd_two_prod(q1, b)));
    const double q2 = r.hi / b;
    r = dd_add(r, dd_neg(dd_two_prod(q2, b)));
    const double q3 = r.hi / b;
    return dd_add(dd_fast_two_sum(q1, q2), DD{q3, 0.0});
}

// exp(a): a = k ln 2 + t with |t| <= ln(2)/2, then the Taylor series of exp(t) to 27
// terms (the first omitted is below 2^-110 of the sum), then the factor 2^k.
__device__ DD dd_exp(DD a)
{
    const DD ln2{KVC_LN2_HI, KVC_LN2_LO};
    const double k = rint(a.hi / KVC_LN2_HI);
    const DD t = dd_add(a, dd_neg(dd_mul_d(ln2, k)));
    DD sum{1.0, 0.0}, term{1.0, 0.0};
    for (int n = 1; n <= 27; n++) {
        term = dd_div_d(dd_mul(term, t), (double)n);
        sum = dd_add(sum, term);
    }
    return DD{ldexp(sum.hi, (int)k), ldexp(sum.lo, (int)k)};
}

// ln b for a positive finite double: one Newton step y0 - 1 + b exp(-y0) from the f64
// logarithm y0 doubles its correct bits.
__device__ DD dd_log(double b)
{
    const double y0 = log(b);
    const DD t = dd_mul_d(dd_exp(DD{-y0, 0.0}), b);
    return dd_add(DD{y0, 0.0}, dd_add(t, DD{-1.0, 0.0}));
}

// The f32 nearest to hi + lo.  Rounding hi alone gives it unless hi lies exactly on a
// midpoint of two neighbouring f32 (hi + lo cannot cross one otherwise: |lo| is at most
// half an f64 ulp of hi, and f32 midpoints are f64 values), where lo's sign decides.
__device__ float dd_to_f32(DD v)
{
    float f = (float)v.hi;
    if (v.lo != 0.0 && __builtin_isfinite(f)) {
        const float below = nextafterf(f, -INFINITY), above = nextafterf(f, INFINITY);
        if (v.hi == 0.5 * ((double)f + (double)below) && v.lo < 0.0) f = below;
        else if (v.hi == 0.5 * ((double)f + (double)above) && v.lo > 0.0) f = above;
    }
    return f;
}

// Round y, an f64 value within `err` of an exact value x, to f32.  True (with *out the
// f32) when that is certainly the f32 nearest to x: no f32 rounding boundary lies within
// err of y, so x and y round alike.
__device__ __forceinline__ bool certified_f32(double y, double err, float *out)
{
    const float f = (float)y;
    if (!__builtin_isfinite(f)) return false;
    const double mb = 0.5 * ((double)f + (double)nextafterf(f, -INFINITY));
    const double ma = 0.5 * ((double)f + (double)nextafterf(f, INFINITY));
    *out = f;
    return y - mb > err && ma - y > err;
}

// An f64 ulp of y (of the smallest subnormal at 0).
__device__ __forceinline__ double ulp64(double y)
{
    return y == 0.0 ? 0x1p-1074 : ldexp(1.0, ilogb(y) - 52);
}

// Speed of pair i: the f32 nearest to freq_scale / freq_base^(2i/hd).
__constant__ uint32_t c_two_over_pi[KVC_TWO_OVER_PI_NWORDS] = {KVC_TWO_OVER_PI_WORDS};

__device__ float rope_speed(int32_t i, int32_t hd, float freq_base, float freq_scale, bool exact)
{
    if (i == 0) return freq_scale;   // base^0 = 1 exactly
    if (!exact) {
        // f64: the exponent 2i/hd rounded once (relative 2^-53, times |ln base| in the
        // power), pow within 2 ulps, the division within half an ulp; bounded with room.
        const double e = (double)(2 * i) / (double)hd;
        const double y = (double)freq_scale / pow((double)freq_base, e);
        const double err = (2.0 * fabs(e * log((double)freq_base)) + 8.0) * 0x1p-53 * fabs(y);
        float f;
        if (certified_f32(y, err, &f)) return f;
    }
    const DD ex = dd_div_d(DD{(double)(2 * i), 0.0}, (double)hd);
    const DD z = dd_exp(dd_neg(dd_mul(ex, dd_log((double)freq_base))));
    return dd_to_f32(dd_mul_d(z, (double)freq_scale));
}

// cos and sin of a finite f32 angle theta >= 2^-12 in double-double.  Payne-Hanek
// reduction: theta = m 2^e (m a 24-bit integer) times the 160 bits of 2/pi from the
// first one whose product with m 2^e is not a multiple of 4, an exact integer product
// whose bits are the quadrant (the two above the binary point) and the fraction; the
// fraction, moved to [-1/2, 1/2), times pi/2 is the reduced angle r, |r| <= pi/4, good to
// about 2^-99 of its size; then the Taylor series of cos r and sin r (the first omitted
// terms are below 2^-100).
__device__ void dd_sincos(float theta, DD *c, DD *s)
{
    const uint32_t bits = __float_as_uint(theta);
    const int ex = (int)(bits >> 23) & 0xff;
    const uint32_t m = ex ? ((bits & 0x7fffffu) | 0x800000u) : (bits & 0x7fffffu);
    const int e = ex ? ex - 150 : -149;
    const int n0 = max(1, e - 1);   // first digit taken: weight 2^-n0 (e <= 104: n0 <= 103)
    const int w = (n0 - 1) >> 5, sh = (n0 - 1) & 31;
    uint32_t x[5];                  // the 160 digits, most significant word first
#pragma unroll
    for (int j = 0; j < 5; j++) {
        const uint32_t a = c_two_over_pi[w + j], b = c_two_over_pi[w + j + 1];
        x[j] = sh ? (a << sh) | (b >> (32 - sh)) : a;
    }
    // P = m * x, 184 bits, least significant 64-bit word first (two zero words above).
    uint32_t pw[6];
    uint64_t carry = 0;
#pragma unroll
    for (int j = 0; j < 5; j++) {
        const uint64_t t = (uint64_t)x[4 - j] * m + carry;
        pw[j] = (uint32_t)t;
        carry = t >> 32;
    }
    pw[5] = (uint32_t)carry;
    const uint64_t p64[5] = {pw[0] | (uint64_t)pw[1] << 32, pw[2] | (uint64_t)pw[3] << 32,
                             pw[4] | (uint64_t)pw[5] << 32, 0, 0};
    // Bit b of P weighs 2^(b + e - n0 - 159): the units bit is b0 = n0 + 159 - e, in
    // [158, 195] for theta >= 2^-12.
    const int b0 = n0 + 159 - e;
    auto window = [&](int lo) -> uint64_t {   // bits [lo, lo + 64) of P, 0 <= lo <= 195
        const int i = lo >> 6, r = lo & 63;
        return r ? (p64[i] >> r) | (p64[i + 1] << (64 - r)) : p64[i];
    };
    uint64_t fhi = window(b0 - 64), flo = window(b0 - 128);   // fraction * 2^128
    int q = (int)(window(b0) & 3);
    const bool neg = (fhi >> 63) != 0;   // fraction >= 1/2: take fraction - 1, next quadrant
    if (neg) {
        flo = ~flo + 1;
        fhi = ~fhi + (flo == 0 ? 1 : 0);
        q = (q + 1) & 3;
    }
    // |fraction| * 2^128 < 2^127 as three exact doubles of at most 53 bits each.
    const double c2 = (double)(fhi >> 42);
    const double c1 = (double)(((fhi & ((1ull << 42) - 1)) << 11) | (flo >> 53));
    const double c0 = (double)(flo & ((1ull << 53) - 1));
    DD f = dd_add(dd_add(DD{ldexp(c2, -22), 0.0}, DD{ldexp(c1, -75), 0.0}), DD{ldexp(c0, -128), 0.0});
    if (neg) f = dd_neg(f);
    const DD r = dd_mul(f, DD{KVC_PI_2_HI, KVC_PI_2_LO});
    const DD r2 = dd_mul(r, r);
    DD sn = r, cs{1.0, 0.0}, term = r;
    for (int n = 2; n <= 26; n += 2) {   // term = (-1)^k r^(2k+1) / (2k+1)!, n = 2k
        term = dd_div_d(dd_mul(term, r2), -(double)(n * (n + 1)));
        sn = dd_add(sn, term);
    }
    term = DD{1.0, 0.0};
    for (int n = 1; n <= 27; n += 2) {   // term = (-1)^k r^(2k) / (2k)!, n = 2k - 1
        term = dd_div_d(dd_mul(term, r2), -(double)(n * (n + 1)));
        cs = dd_add(cs, term);
    }
    // theta = q pi/2 + r.
    switch (q) {
    case 0: *c = cs; *s = sn; break;
    case 1: *c = dd_neg(sn); *s = cs; break;
    case 2: *c = dd_neg(cs); *s = dd_neg(sn); break;
    default: *c = sn; *s = dd_neg(cs); break;
    }
}

// (cos, sin) of the f32 angle theta >= 0, each the f32 nearest to the exact value.
__device__ float2 rope_cos_sin(float theta, bool exact)
{
    if (!__builtin_isfinite(theta))   // an overflowed angle: NaN, as the f64 functions give
        return make_float2((float)cos((double)theta), (float)sin((double)theta));
    // Below 2^-12, cos theta = 1 - theta^2/2 + ... and sin theta = theta (1 - theta^2/6 +
    // ...) are within half an f32 ulp of 1 and of theta.
    if (theta < 0x1p-12f) return make_float2(1.0f, theta);
    if (!exact) {
        // f64 cos and sin: within a few ulps; bounded by 16 ulps plus 2^-90.
        const double yc = cos((double)theta), ys = sin((double)theta);
        float fc, fs;
        if (certified_f32(yc, 16.0 * ulp64(yc) + 0x1p-90, &fc) &&
            certified_f32(ys, 16.0 * ulp64(ys) + 0x1p-90, &fs))
            return make_float2(fc, fs);
    }
    DD c, s;
    dd_sincos(theta, &c, &s);
    return make_float2(dd_to_f32(c), dd_to_f32(s));
}

// One thread per (p, i), grid-stride; each workgroup first derives the hd/2 speeds into
// LDS.  exact != 0 evaluates every entry in double-double (a test switch: the same
// results, slower).
__global__ void __launch_bounds__(256) rope_table_kernel(float2 *tab, int32_t rows, int32_t hd,
                                                         float freq_base, float freq_scale,
                                                         int32_t exact)
{
    __shared__ float s_speed[KVC_MAX_HEAD_DIM / 2];
    const int32_t half = hd >> 1;
    for (int32_t i = threadIdx.x; i < half; i += blockDim.x)
        s_speed[i] = rope_speed(i, hd, freq_base, freq_scale, exact != 0);
    __syncthreads();
    const int64_t n = (int64_t)rows * half;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int32_t p = (int32_t)(idx / half);
        const int32_t i = (int32_t)(idx - (int64_t)p * half);
        tab[idx] = rope_cos_sin(__fmul_rn((float)p, s_speed[i]), exact != 0);
    }
}

// Rotate nh heads of width w (even) from src into dst (dst may equal src), using the
// table row `tab` (w/2 entries).  Threads of the block stride over the nh * w/2 pairs,
// so consecutive threads touch consecutive elements of a head.
template <int STYLE>
__device__ __forceinline__ void rotate_heads(const float *src, float *dst, int32_t nh, int32_t w,
                                             const float2 *tab)
{
    const int32_t half = w >> 1;
    const int32_t npairs = nh * half;
    for (int32_t idx = threadIdx.x; idx < npairs; idx += blockDim.x) {
        const int32_t h = idx / half;
        const int32_t i = idx - h * half;
        const int32_t i0 = STYLE == kNeox ? i : 2 * i;
        const int32_t i1 = STYLE == kNeox ? i + half : 2 * i + 1;
        const float *x = src + (int64_t)h * w;
        float *y = dst + (int64_t)h * w;
        float y0, y1;
        rotate_pair(x[i0], x[i1], tab[i], y0, y1);
        y[i0] = y0;
        y[i1] = y1;
    }
}

// Vector form of rotate_heads for widths where every access is a whole, aligned float4:
// a NEOX thread rotates 4 consecutive pairs (i..i+3 with i+half..i+half+3), an
// interleaved thread 2 consecutive pairs (4 consecutive elements).  Same arithmetic.
template <int STYLE, typename DT>
__device__ __forceinline__ void rotate_heads_vec(const float *src, DT *dst, int32_t nh,
                                                 int32_t w, const float2 *tab)
{
    const int32_t half = w >> 1;
    const int32_t per_head = w >> 2;  // float4 units per head
    const int32_t nq = nh * (STYLE == kNeox ? per_head / 2 : per_head);
    for (int32_t idx = threadIdx.x; idx < nq; idx += blockDim.x) {
        if constexpr (STYLE == kNeox) {
            const int32_t h = idx / (per_head / 2);
            const int32_t i = (idx - h * (per_head / 2)) * 4;
            const float *x = src + (int64_t)h * w;
            DT *y = dst + (int64_t)h * w;
            const float4 a = *reinterpret_cast<const float4 *>(x + i);
            const float4 b = *reinterpret_cast<const float4 *>(x + half + i);
            const float4 t0 = *reinterpret_cast<const float4 *>(tab + i);
            const float4 t1 = *reinterpret_cast<const float4 *>(tab + i + 2);
            float4 ya, yb;
            rotate_pair(a.x, b.x, make_float2(t0.x, t0.y), ya.x, yb.x);
            rotate_pair(a.y, b.y, make_float2(t0.z, t0.w), ya.y, yb.y);
            rotate_pair(a.z, b.z, make_float2(t1.x, t1.y), ya.z, yb.z);
            rotate_pair(a.w, b.w, make_float2(t1.z, t1.w), ya.w, yb.w);
            store4(y + i, ya);
            store4(y + half + i, yb);
        } else {
            const int32_t h = idx / per_head;
            const int32_t e = (idx - h * per_head) * 4;
            const float *x = src + (int64_t)h * w;
            DT *y = dst + (int64_t)h * w;
            const float4 a = *reinterpret_cast<const float4 *>(x + e);
            const float4 t = *reinterpret_cast<const float4 *>(tab + e / 2);
            float4 ya;
            rotate_pair(a.x, a.y, make_float2(t.x, t.y), ya.x, ya.y);
            rotate_pair(a.z, a.w, make_float2(t.z, t.w), ya.z, ya.w);
            store4(y + e, ya);
        }
    }
}

// One workgroup per token.  Reads: q row (if any), k row, v row, one table row per head
// dim.  Writes: q row in place, one K row and one V row of the cache (elements of type
// KVT: f32, or binary16 rounded from the f32 result).  QVEC selects the float4 form for q
// (hd a multiple of 8 for NEOX, of 4 for interleaved); k always qualifies (hd_kv is a
// multiple of 16).
// Rotate q of token t in place (f32, whatever the region format).
template <int STYLE, bool QVEC>
__device__ __forceinline__ void rotate_q(const AppendArgs &p, int32_t t, int32_t pos)
{
    if (STYLE != kNone && p.q) {
        float *qt = p.q + (int64_t)t * p.n_head * p.hd;
        const float2 *tq = p.tab_q + (int64_t)pos * (p.hd >> 1);
        if constexpr (QVEC) rotate_heads_vec<STYLE>(qt, qt, p.n_head, p.hd, tq);
        else rotate_heads<STYLE>(qt, qt, p.n_head, p.hd, tq);
    }
}

template <int STYLE, bool QVEC, typename KVT, int E>
__global__ void __launch_bounds__(256) append_kernel(AppendParamsT<E> p)
{
    const int32_t t = blockIdx.x;
    const int32_t pos = p.pos ? p.pos[t] : p.ipos[t];
    const int32_t seq = p.seq ? p.seq[t] : p.iseq[t];
    const int32_t nkt = p.n_head_kv * p.hd_kv;
    const int64_t reg = ((int64_t)seq * p.n_layer + p.layer) * p.region_bytes;
    const float *ksrc = p.k + (int64_t)t * nkt;
    const float *vsrc = p.v + (int64_t)t * nkt;
    KVT *kdst = reinterpret_cast<KVT *>(static_cast<char *>(p.kc) + reg) + (int64_t)pos * nkt;
    KVT *vdst = reinterpret_cast<KVT *>(static_cast<char *>(p.vc) + reg) + (int64_t)pos * nkt;

    rotate_q<STYLE, QVEC>(p, t, pos);
    if (STYLE != kNone) {
        rotate_heads_vec<STYLE>(ksrc, kdst, p.n_head_kv, p.hd_kv,
                                p.tab_k + (int64_t)pos * (p.hd_kv >> 1));
    } else {
        const float4 *ks4 = reinterpret_cast<const float4 *>(ksrc);
        for (int32_t i = threadIdx.x; i < (nkt >> 2); i += blockDim.x) store4(kdst + 4 * i, ks4[i]);
    }
    // hd_kv is a multiple of 16, so rows are whole float4s (half4s) and aligned.
    const float4 *vs4 = reinterpret_cast<const float4 *>(vsrc);
    for (int32_t i = threadIdx.x; i < (nkt >> 2); i += blockDim.x) store4(vdst + 4 * i, vs4[i]);
}

// Values e..e+3 (e a multiple of 4) of one head of width w after rotation, computed
// with rotate_pair exactly as rotate_heads_vec computes them.  NEOX: all four lie in
// one half (w / 2 is a multiple of 4), each the first or second output of its pair.
template <int STYLE>
__device__ __forceinline__ float4 rotated4(const float *x, int32_t e, int32_t w,
                                           const float2 *tab)
{
    float4 y;
    if constexpr (STYLE == kNeox) {
        const int32_t half = w >> 1;
        const bool lo = e < half;
        const int32_t i = lo ? e : e - half;
        const float4 a = *reinterpret_cast<const float4 *>(x + i);
        const float4 b = *reinterpret_cast<const float4 *>(x + i + half);
        const float4 t0 = *reinterpret_cast<const float4 *>(tab + i);
        const float4 t1 = *reinterpret_cast<const float4 *>(tab + i + 2);
        float4 y0, y1;
        rotate_pair(a.x, b.x, make_float2(t0.x, t0.y), y0.x, y1.x);
        rotate_pair(a.y, b.y, make_float2(t0.z, t0.w), y0.y, y1.y);
        rotate_pair(a.z, b.z, make_float2(t1.x, t1.y), y0.z, y1.z);
        rotate_pair(a.w, b.w, make_float2(t1.z, t1.w), y0.w, y1.w);
        y = lo ? y0 : y1;
    } else if constexpr (STYLE == kInterleaved) {
        const float4 a = *reinterpret_cast<const float4 *>(x + e);
        const float4 t = *reinterpret_cast<const float4 *>(tab + e / 2);
        rotate_pair(a.x, a.y, make_float2(t.x, t.y), y.x, y.y);
        rotate_pair(a.z, a.w, make_float2(t.z, t.w), y.z, y.w);
    } else {
        y = *reinterpret_cast<const float4 *>(x + e);
    }
    return y;
}

// Q8_0 variant of append_kernel: the same rotation, then each row is quantized block by
// block as it is stored.  Thread idx handles values 4 idx .. 4 idx + 3 of the row;
// nkt / 4 is a multiple of 8 and so is the block size, so the 8 lanes of a block are
// always active together.
template <int STYLE, bool QVEC, int E>
__global__ void __launch_bounds__(256) append_q8_kernel(AppendParamsT<E> p)
{
    const int32_t t = blockIdx.x;
    const int32_t pos = p.pos ? p.pos[t] : p.ipos[t];
    const int32_t seq = p.seq ? p.seq[t] : p.iseq[t];
    const int32_t nkt = p.n_head_kv * p.hd_kv;
    const int64_t reg = ((int64_t)seq * p.n_layer + p.layer) * p.region_bytes;
    const float *ksrc = p.k + (int64_t)t * nkt;
    const float *vsrc = p.v + (int64_t)t * nkt;
    char *kr = static_cast<char *>(p.kc) + reg;
    char *vr = static_cast<char *>(p.vc) + reg;
    int8_t *kcodes = reinterpret_cast<int8_t *>(kr) + (int64_t)pos * nkt;
    int8_t *vcodes = reinterpret_cast<int8_t *>(vr) + (int64_t)pos * nkt;
    _Float16 *kscales = reinterpret_cast<_Float16 *>(kr + p.scale_off);
    _Float16 *vscales = reinterpret_cast<_Float16 *>(vr + p.scale_off);
    const int64_t rows = p.scale_off / nkt;
    const float2 *tk = STYLE == kNone ? nullptr : p.tab_k + (int64_t)pos * (p.hd_kv >> 1);

    rotate_q<STYLE, QVEC>(p, t, pos);
    for (int32_t idx = threadIdx.x; idx < (nkt >> 2); idx += blockDim.x) {
        const int32_t j = idx * 4;
        const int32_t h = j / p.hd_kv;
        const int32_t e = j - h * p.hd_kv;
        const float4 y = rotated4<STYLE>(ksrc + (int64_t)h * p.hd_kv, e, p.hd_kv, tk);
        const int64_t si = q8_scale_index(pos, j, p.hd_kv, rows);
        q8_store4(y, kcodes + j, kscales + si, idx);
        q8_store4(*reinterpret_cast<const float4 *>(vsrc + j), vcodes + j, vscales + si, idx);
    }
}

}  // namespace

hipError_t launch_rope_table(float2 *tab, int32_t rows, int32_t hd, float freq_base,
                             float freq_scale, bool exact, hipStream_t s)
{
    const int64_t n = (int64_t)rows * (hd >> 1);
    const int64_t want = (n + 255) / 256;
    const unsigned grid = (unsigned)(want < 65536 ? (want > 0 ? want : 1) : 65536);
    rope_table_kernel<<<grid, 256, 0, s>>>(tab, rows, hd, freq_base, freq_scale, exact ? 1 : 0);
    return hipGetLastError();
}

template <typename KVT, int E>
void launch_append_t(const AppendParamsT<E> &p, hipStream_t s)
{
    const dim3 grid((unsigned)p.nt), block(256);
    switch (p.style) {
    case kNeox:
        if (p.hd % 8 == 0) append_kernel<kNeox, true, KVT, E><<<grid, block, 0, s>>>(p);
        else append_kernel<kNeox, false, KVT, E><<<grid, block, 0, s>>>(p);
        break;
    case kInterleaved:
        if (p.hd % 4 == 0) append_kernel<kInterleaved, true, KVT, E><<<grid, block, 0, s>>>(p);
        else append_kernel<kInterleaved, false, KVT, E><<<grid, block, 0, s>>>(p);
        break;
    default: append_kernel<kNone, false, KVT, E><<<grid, block, 0, s>>>(p); break;
    }
}

template <int E>
void launch_append_q8(const AppendParamsT<E> &p, hipStream_t s)
{
    const dim3 grid((unsigned)p.nt), block(256);
    switch (p.style) {
    case kNeox:
        if (p.hd % 8 == 0) append_q8_kernel<kNeox, true, E><<<grid, block, 0, s>>>(p);
        else append_q8_kernel<kNeox, false, E><<<grid, block, 0, s>>>(p);
        break;
    case kInterleaved:
        if (p.hd % 4 == 0) append_q8_kernel<kInterleaved, true, E><<<grid, block, 0, s>>>(p);
        else append_q8_kernel<kInterleaved, false, E><<<grid, block, 0, s>>>(p);
        break;
    default: append_q8_kernel<kNone, false, E><<<grid, block, 0, s>>>(p); break;
    }
}

template <int E>
void launch_append_fmt(const AppendParamsT<E> &p, hipStream_t s)
{
    if (p.kv_fmt == kFmtQ8) launch_append_q8<E>(p, s);
    else if (p.kv_fmt == kFmtF16) launch_append_t<_Float16, E>(p, s);
    else launch_append_t<float, E>(p, s);
}

hipError_t launch_append(const AppendParams &p, hipStream_t s)
{
    if (p.nt <= 0) return hipSuccess;
    if (!p.pos && !p.seq && p.nt <= kSmallInline) {
        // Few inline tokens: the same launch with an argument block sized for them.
        AppendParamsT<kSmallInline> sp;
        static_cast<AppendArgs &>(sp) = p;
        for (int i = 0; i < kSmallInline; i++) {
            sp.ipos[i] = i < p.nt ? p.ipos[i] : 0;
            sp.iseq[i] = i < p.nt ? p.iseq[i] : 0;
        }
        launch_append_fmt(sp, s);
    } else {
        launch_append_fmt(p, s);
    }
    return hipGetLastError();
}

}  // namespace kvc
