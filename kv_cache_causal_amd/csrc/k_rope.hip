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
// the exact expression.  Both are evaluated in f64 and rounded once to f32 (an f64
// result sits within an f64 ulp or so of the exact value, far inside an f32 half-ulp
// except at near-ties).  The rotation (rotate_pair, kvc_device.hpp) is compiled with FMA
// contraction off, so each product and each sum is rounded on its own and the result is
// the same bits as any correctly rounded IEEE evaluation of the same formula.
#include <hip/hip_runtime.h>

#include "kvc_device.hpp"
#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr int kNeox = 0, kInterleaved = 1, kNone = 2;

__global__ void __launch_bounds__(256) rope_table_kernel(float2 *tab, int32_t rows, int32_t hd,
                                                         float freq_base, float freq_scale)
{
    const int32_t half = hd >> 1;
    const int64_t n = (int64_t)rows * half;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int32_t p = (int32_t)(idx / half);
        const int32_t i = (int32_t)(idx - (int64_t)p * half);
        const double expo = (double)(2 * i) / (double)hd;
        const float speed = (float)((double)freq_scale / pow((double)freq_base, expo));
        const float theta = __fmul_rn((float)p, speed);
        tab[idx] = make_float2((float)cos((double)theta), (float)sin((double)theta));
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
__device__ __forceinline__ void rotate_q(const AppendParams &p, int32_t t, int32_t pos)
{
    if (STYLE != kNone && p.q) {
        float *qt = p.q + (int64_t)t * p.n_head * p.hd;
        const float2 *tq = p.tab_q + (int64_t)pos * (p.hd >> 1);
        if constexpr (QVEC) rotate_heads_vec<STYLE>(qt, qt, p.n_head, p.hd, tq);
        else rotate_heads<STYLE>(qt, qt, p.n_head, p.hd, tq);
    }
}

template <int STYLE, bool QVEC, typename KVT>
__global__ void __launch_bounds__(256) append_kernel(AppendParams p)
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
template <int STYLE, bool QVEC>
__global__ void __launch_bounds__(256) append_q8_kernel(AppendParams p)
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
                             float freq_scale, hipStream_t s)
{
    const int64_t n = (int64_t)rows * (hd >> 1);
    const int64_t want = (n + 255) / 256;
    const unsigned grid = (unsigned)(want < 65536 ? (want > 0 ? want : 1) : 65536);
    rope_table_kernel<<<grid, 256, 0, s>>>(tab, rows, hd, freq_base, freq_scale);
    return hipGetLastError();
}

template <typename KVT>
void launch_append_t(const AppendParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)p.nt), block(256);
    switch (p.style) {
    case kNeox:
        if (p.hd % 8 == 0) append_kernel<kNeox, true, KVT><<<grid, block, 0, s>>>(p);
        else append_kernel<kNeox, false, KVT><<<grid, block, 0, s>>>(p);
        break;
    case kInterleaved:
        if (p.hd % 4 == 0) append_kernel<kInterleaved, true, KVT><<<grid, block, 0, s>>>(p);
        else append_kernel<kInterleaved, false, KVT><<<grid, block, 0, s>>>(p);
        break;
    default: append_kernel<kNone, false, KVT><<<grid, block, 0, s>>>(p); break;
    }
}

void launch_append_q8(const AppendParams &p, hipStream_t s)
{
    const dim3 grid((unsigned)p.nt), block(256);
    switch (p.style) {
    case kNeox:
        if (p.hd % 8 == 0) append_q8_kernel<kNeox, true><<<grid, block, 0, s>>>(p);
        else append_q8_kernel<kNeox, false><<<grid, block, 0, s>>>(p);
        break;
    case kInterleaved:
        if (p.hd % 4 == 0) append_q8_kernel<kInterleaved, true><<<grid, block, 0, s>>>(p);
        else append_q8_kernel<kInterleaved, false><<<grid, block, 0, s>>>(p);
        break;
    default: append_q8_kernel<kNone, false><<<grid, block, 0, s>>>(p); break;
    }
}

hipError_t launch_append(const AppendParams &p, hipStream_t s)
{
    if (p.nt <= 0) return hipSuccess;
    if (p.kv_fmt == kFmtQ8) launch_append_q8(p, s);
    else if (p.kv_fmt == kFmtF16) launch_append_t<_Float16>(p, s);
    else launch_append_t<float>(p, s);
    return hipGetLastError();
}

}  // namespace kvc
