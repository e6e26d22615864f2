/*
 * oracle.c -- plain, slow CPU statement of causal grouped-query attention over a
 * per-layer KV cache.
 *
 * THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT PATH.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg load it.  It shares no code,
 * header, table or constant with the HIP library: every step below is written out
 * from the pages it cites.
 *
 * Sources (titles of the pages; sections named inline):
 *   [MINFER-11] "11 · Attention, vec ops, and the KV cache"
 *   [ZEROCOPY]  "IV.2: Zero-copy KV cache"
 *   [MINFER-13] "13 · The decode loop and graph reuse"
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fopenmp -fPIC -shared -lm.
 * No FMA contraction anywhere: every product and sum below is rounded to f32 on its
 * own, as the scalar code on the pages does.
 *
 * Precision follows the pages where they fix it: scores, exponentials, normalisation
 * and the weighted V sum are f32; the softmax denominator is summed in f64
 * ([MINFER-11] §3.2.5, the softmax routine's f64 accumulator).  RoPE frequencies and
 * cos/sin are the correctly rounded f32 values of the exact expressions (evaluated in
 * long double and rounded once), because the pages' f32 powf/sin_cos depend on the libm
 * that runs them.
 *
 * Regions hold f32, or IEEE binary16 for the half-precision cache ([MINFER-11] §2.5):
 * the store rounds each f32 value to binary16 (nearest, ties to even) and attention
 * widens it back to f32 exactly before the same f32 arithmetic.  A third format packs
 * each row as Q8_0 blocks ([MINFER-11] §2.5 "Storage" and the FAQ on cache formats:
 * 34 bytes per 32 values, quantized by the store, dequantized by attention).  The pages
 * give the block size but not its arithmetic; the reading taken here is the published
 * Q8_0 block of the GGML family: scale d = max|x| / 127 in f32, stored as binary16;
 * codes round(x * (1/d)) to nearest, halves away from zero, with 1/d the f32 reciprocal
 * of the f32 scale (0 for an all-zero block); value = f32(binary16 d) * code, which is
 * exact in f32.
 *
 * Pins: every function here is checked by tests against closed forms, the pages'
 * worked examples, arbitrary-precision values, numpy's binary16 conversion and an f64
 * brute force; no function is "parity unpinned".
 */
#include <float.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Status values.  They use the same numbers as the library's public status enum so a
 * test can compare error behaviour call by call (a format that must agree). */
enum {
    ORC_OK = 0,
    ORC_E_ARG = 1,
    ORC_E_GEOMETRY = 2,
    ORC_E_RANGE = 3,
    ORC_E_DUP = 4,
    ORC_E_NOMEM = 5
};

/* RoPE pair layouts ([MINFER-11] §3.2.2, the two layout styles). */
enum { ORC_ROPE_NEOX = 0, ORC_ROPE_INTERLEAVED = 1, ORC_ROPE_NONE = 2 };

#define ORC_MAX_HEAD_DIM 256        /* the pages' fixed 128-entry frequency table */
#define ORC_MAX_POSITION (1 << 24)  /* positions travel as exact integers in f32 */

/* ------------------------------------------------------------------------------ */
/* RoPE ([MINFER-11] §2.3 "RoPE: position without position embeddings",            */
/*       §3.2.2 "RoPE -- the node arm and cpu_rope")                                */
/* ------------------------------------------------------------------------------ */

/* Angular speed of subspace i: freq_scale / base^(2i/hd), rounded once to f32. */
int orc_rope_inv_freq(int32_t hd, float freq_base, float freq_scale, float *inv)
{
    if (hd <= 0 || (hd & 1) || hd > ORC_MAX_HEAD_DIM || !inv) return ORC_E_ARG;
    for (int32_t i = 0; i < hd / 2; i++) {
        long double expo = (long double)(2 * i) / (long double)hd;
        long double speed = (long double)freq_scale / powl((long double)freq_base, expo);
        inv[i] = (float)speed;
    }
    return ORC_OK;
}

/* cos and sin of the angle position x speed.  The angle itself is an f32 product, as
 * on the page; its cos and sin are correctly rounded to f32. */
int orc_rope_cos_sin(int32_t hd, float freq_base, float freq_scale, int32_t p,
                     float *cs, float *sn)
{
    float inv[ORC_MAX_HEAD_DIM / 2];
    int st = orc_rope_inv_freq(hd, freq_base, freq_scale, inv);
    if (st != ORC_OK) return st;
    if (p < 0) return ORC_E_RANGE;
    for (int32_t i = 0; i < hd / 2; i++) {
        float theta = (float)p * inv[i];
        cs[i] = (float)cosl((long double)theta);
        sn[i] = (float)sinl((long double)theta);
    }
    return ORC_OK;
}

/* Rotate one head vector x[0..hd) in place at position p.
 * NEOX pairs are (i, i + hd/2); interleaved pairs are (2i, 2i+1).  The rotation is
 *   x0' = x0*cos - x1*sin,  x1' = x0*sin + x1*cos,
 * each product and each sum rounded to f32 separately. */
static void rotate_head(float *x, int32_t hd, const float *cs, const float *sn, int32_t style)
{
    int32_t half = hd / 2;
    for (int32_t i = 0; i < half; i++) {
        int32_t i0, i1;
        if (style == ORC_ROPE_NEOX) { i0 = i; i1 = i + half; }
        else { i0 = 2 * i; i1 = 2 * i + 1; }
        float x0 = x[i0], x1 = x[i1];
        float a = x0 * cs[i];
        float b = x1 * sn[i];
        float c = x0 * sn[i];
        float d = x1 * cs[i];
        x[i0] = a - b;
        x[i1] = c + d;
    }
}

/* Apply RoPE in place to x laid out [nt][nh][hd], token t at position pos[t]. */
int orc_rope(float *x, int32_t nt, int32_t nh, int32_t hd, const int32_t *pos,
             float freq_base, float freq_scale, int32_t style)
{
    if (style == ORC_ROPE_NONE) return ORC_OK;
    if (style != ORC_ROPE_NEOX && style != ORC_ROPE_INTERLEAVED) return ORC_E_ARG;
    if (nt < 0 || nh <= 0 || (nt > 0 && (!x || !pos))) return ORC_E_ARG;
    float cs[ORC_MAX_HEAD_DIM / 2], sn[ORC_MAX_HEAD_DIM / 2];
    for (int32_t t = 0; t < nt; t++) {
        int st = orc_rope_cos_sin(hd, freq_base, freq_scale, pos[t], cs, sn);
        if (st != ORC_OK) return st;
        for (int32_t h = 0; h < nh; h++)
            rotate_head(x + ((size_t)t * nh + h) * hd, hd, cs, sn, style);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* The KV cache: persistent per-layer K and V regions, row p at offset p * row     */
/* width ([MINFER-11] §2.2 "Why the KV cache exists", §3.2.3 "The KV store / load  */
/* pair"; [ZEROCOPY] "The cache appends in place").  Regions are sized once and    */
/* start zeroed, so rows never written read as zeros.                              */
/* ------------------------------------------------------------------------------ */

/* Storage formats of the regions.  F16 is the half-precision cache of [MINFER-11] §2.5
 * ("Storage") and §3.3: the store rounds each value to IEEE binary16, attention widens
 * it back to f32 and computes in f32. */
enum { ORC_KV_F32 = 0, ORC_KV_F16 = 1, ORC_KV_Q8_0 = 2 };

/* IEEE-754 binary32 -> binary16, round to nearest, ties to even; overflow gives inf,
 * tiny values become subnormals or signed zero; NaN stays a (quiet) NaN. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t x;
    memcpy(&x, &f, sizeof x);
    const uint32_t sign = (x >> 16) & 0x8000u;
    const uint32_t exp = (x >> 23) & 0xffu;
    uint32_t man = x & 0x7fffffu;
    if (exp == 0xffu) return (uint16_t)(sign | (man ? 0x7e00u : 0x7c00u));
    const int32_t e = (int32_t)exp - 127 + 15;        /* binary16 biased exponent */
    if (e >= 31) return (uint16_t)(sign | 0x7c00u);     /* beyond the largest finite */
    if (e <= 0) {                                       /* subnormal or zero result */
        if (e < -10) return (uint16_t)sign;             /* below half the smallest subnormal */
        man |= 0x800000u;                               /* make the leading 1 explicit */
        const int32_t shift = 14 - e;                   /* value = man * 2^-24 after shift */
        uint32_t h = man >> shift;
        const uint32_t rem = man & ((1u << shift) - 1u);
        const uint32_t half = 1u << (shift - 1);
        if (rem > half || (rem == half && (h & 1u))) h++;
        return (uint16_t)(sign | h);                    /* a carry lands on the smallest normal */
    }
    uint32_t h = sign | ((uint32_t)e << 10) | (man >> 13);
    const uint32_t rem = man & 0x1fffu;
    if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h++; /* a carry may reach inf: correct */
    return (uint16_t)h;
}

/* IEEE-754 binary16 -> binary32 (exact). */
float orc_f16_to_f32(uint16_t h)
{
    const uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t exp = ((uint32_t)h >> 10) & 0x1fu;
    uint32_t man = (uint32_t)h & 0x3ffu;
    uint32_t x;
    if (exp == 0) {
        if (man == 0) {
            x = sign;
        } else {                                        /* subnormal: normalise */
            int32_t shifts = 0;
            while (!(man & 0x400u)) { man <<= 1; shifts++; }
            man &= 0x3ffu;
            x = sign | ((uint32_t)(127 - 14 - shifts) << 23) | (man << 13);
        }
    } else if (exp == 31) {
        x = sign | 0x7f800000u | (man << 13);
    } else {
        x = sign | ((exp - 15 + 127) << 23) | (man << 13);
    }
    float f;
    memcpy(&f, &x, sizeof f);
    return f;
}

/* ------------------------------------------------------------------------------ */
/* Q8_0 blocks (reading stated in the header).                                       */
/* ------------------------------------------------------------------------------ */

#define ORC_Q8_BLOCK 32

/* One block: the binary16 scale, then the 32 signed 8-bit codes (34 bytes). */
typedef struct {
    uint16_t d;
    int8_t qs[ORC_Q8_BLOCK];
} orc_q8_block;

_Static_assert(sizeof(orc_q8_block) == 34, "a Q8_0 block is 34 bytes");

/* Quantize n values (n a multiple of 32) into n / 32 blocks.  Inputs must be finite:
 * a non-finite value makes its block's codes unspecified (here 0). */
int orc_q8_quantize_row(const float *x, int32_t n, void *out)
{
    if (!x || !out || n < 0 || n % ORC_Q8_BLOCK) return ORC_E_ARG;
    orc_q8_block *b = (orc_q8_block *)out;
    for (int32_t blk = 0; blk < n / ORC_Q8_BLOCK; blk++) {
        const float *xb = x + (size_t)blk * ORC_Q8_BLOCK;
        float amax = 0.0f;
        for (int32_t i = 0; i < ORC_Q8_BLOCK; i++) {
            const float a = fabsf(xb[i]);
            if (a > amax) amax = a;
        }
        const float d = amax / 127.0f;
        const float id = d != 0.0f ? 1.0f / d : 0.0f;
        b[blk].d = orc_f32_to_f16(d);
        for (int32_t i = 0; i < ORC_Q8_BLOCK; i++) {
            const float r = roundf(xb[i] * id);   /* halves away from zero */
            b[blk].qs[i] = (r >= -127.0f && r <= 127.0f) ? (int8_t)r : 0;
        }
    }
    return ORC_OK;
}

/* Dequantize n / 32 blocks into n values. */
int orc_q8_dequantize_row(const void *in, int32_t n, float *out)
{
    if (!in || !out || n < 0 || n % ORC_Q8_BLOCK) return ORC_E_ARG;
    const orc_q8_block *b = (const orc_q8_block *)in;
    for (int32_t blk = 0; blk < n / ORC_Q8_BLOCK; blk++) {
        const float d = orc_f16_to_f32(b[blk].d);
        for (int32_t i = 0; i < ORC_Q8_BLOCK; i++)
            out[(size_t)blk * ORC_Q8_BLOCK + i] = d * (float)b[blk].qs[i];
    }
    return ORC_OK;
}

typedef struct orc_cache {
    int32_t n_seq, n_layer, n_head_kv, hd_kv, capacity, dtype;
    size_t region;      /* values per (seq, layer) region: capacity * n_head_kv * hd_kv */
    size_t region_bytes;
    void *k, *v;        /* [n_seq][n_layer][capacity][row]: a row is n_head_kv * hd_kv f32
                           values, binary16 bit patterns, or Q8_0 blocks */
    int32_t *hw;        /* high-water mark per (seq, layer): max written position + 1 */
} orc_cache;

orc_cache *orc_cache_new_typed(int32_t n_seq, int32_t n_layer, int32_t n_head_kv,
                               int32_t hd_kv, int32_t capacity, int32_t dtype)
{
    if (n_seq <= 0 || n_layer <= 0 || n_head_kv <= 0 || hd_kv <= 0 || (hd_kv & 1) ||
        hd_kv > ORC_MAX_HEAD_DIM || capacity <= 0 || capacity > ORC_MAX_POSITION ||
        (dtype != ORC_KV_F32 && dtype != ORC_KV_F16 && dtype != ORC_KV_Q8_0))
        return NULL;
    /* Q8_0 blocks run along the row; with hd_kv a multiple of 32 each block lies in one
     * kv head, so a head's slice is whole blocks. */
    if (dtype == ORC_KV_Q8_0 && hd_kv % ORC_Q8_BLOCK) return NULL;
    orc_cache *c = (orc_cache *)calloc(1, sizeof(orc_cache));
    if (!c) return NULL;
    c->n_seq = n_seq; c->n_layer = n_layer; c->n_head_kv = n_head_kv;
    c->hd_kv = hd_kv; c->capacity = capacity; c->dtype = dtype;
    c->region = (size_t)capacity * (size_t)n_head_kv * (size_t)hd_kv;
    if (dtype == ORC_KV_Q8_0)
        c->region_bytes = c->region / ORC_Q8_BLOCK * sizeof(orc_q8_block);
    else
        c->region_bytes = c->region * (dtype == ORC_KV_F16 ? sizeof(uint16_t) : sizeof(float));
    const size_t total = (size_t)n_seq * (size_t)n_layer * c->region_bytes;
    c->k = calloc(total, 1);   /* all-zero bytes are +0.0 in every format */
    c->v = calloc(total, 1);
    c->hw = (int32_t *)calloc((size_t)n_seq * n_layer, sizeof(int32_t));
    if (!c->k || !c->v || !c->hw) {
        free(c->k); free(c->v); free(c->hw); free(c);
        return NULL;
    }
    return c;
}

orc_cache *orc_cache_new(int32_t n_seq, int32_t n_layer, int32_t n_head_kv, int32_t hd_kv,
                         int32_t capacity)
{
    return orc_cache_new_typed(n_seq, n_layer, n_head_kv, hd_kv, capacity, ORC_KV_F32);
}

void orc_cache_free(orc_cache *c)
{
    if (!c) return;
    free(c->k); free(c->v); free(c->hw); free(c);
}

/* which = 0 for K, 1 for V.  Returns the [capacity][row] region (f32 values, binary16
 * bit patterns, or n_head_kv * hd_kv / 32 Q8_0 blocks per row). */
void *orc_cache_region(orc_cache *c, int32_t which, int32_t seq, int32_t layer)
{
    if (!c || seq < 0 || seq >= c->n_seq || layer < 0 || layer >= c->n_layer) return NULL;
    char *base = (char *)(which ? c->v : c->k);
    return base + ((size_t)seq * c->n_layer + layer) * c->region_bytes;
}

/* Write n f32 values into a region at value offset off (a row start), in the cache's
 * format. */
static void store_values(orc_cache *c, void *region, size_t off, const float *src, int32_t n)
{
    if (c->dtype == ORC_KV_Q8_0) {
        orc_q8_quantize_row(src, n, (orc_q8_block *)region + off / ORC_Q8_BLOCK);
    } else if (c->dtype == ORC_KV_F16) {
        uint16_t *d = (uint16_t *)region + off;
        for (int32_t i = 0; i < n; i++) d[i] = orc_f32_to_f16(src[i]);
    } else {
        memcpy((float *)region + off, src, sizeof(float) * (size_t)n);
    }
}

int32_t orc_cache_seq_len(const orc_cache *c, int32_t seq, int32_t layer)
{
    if (!c || seq < 0 || seq >= c->n_seq || layer < 0 || layer >= c->n_layer) return -1;
    return c->hw[(size_t)seq * c->n_layer + layer];
}

static int cmp_i64(const void *a, const void *b)
{
    int64_t x = *(const int64_t *)a, y = *(const int64_t *)b;
    return (x > y) - (x < y);
}

/* Store this step's K/V rows at the positions the caller passes, after rotating q
 * (optional, in place) and k.  Everything is checked before anything is written:
 * a position outside the region is an error, never a clamp ([MINFER-11] §3.2.3 and
 * §3.4 "Pitfalls & invariants"); two rows aimed at the same (sequence, position) in
 * one call are refused because their order would be ambiguous.
 * q: [nt][n_head][hd] (may be NULL); k, v: [nt][n_head_kv][hd_kv]. */
int orc_append_rope(orc_cache *c, int32_t layer, int32_t nt, const int32_t *seq_ids,
                    const int32_t *pos, float *q, int32_t n_head, int32_t hd,
                    const float *k, const float *v, float freq_base, float freq_scale,
                    int32_t style)
{
    if (!c || layer < 0 || layer >= c->n_layer || nt < 0) return ORC_E_ARG;
    if (nt == 0) return ORC_OK;
    if (!seq_ids || !pos || !k || !v) return ORC_E_ARG;
    if (style != ORC_ROPE_NEOX && style != ORC_ROPE_INTERLEAVED && style != ORC_ROPE_NONE)
        return ORC_E_ARG;
    if (style != ORC_ROPE_NONE &&
        (!(freq_base > 0.0f) || !isfinite(freq_base) || !(freq_scale > 0.0f) ||
         !isfinite(freq_scale)))
        return ORC_E_ARG;
    if (q) {
        if (n_head <= 0 || n_head % c->n_head_kv != 0) return ORC_E_ARG;
        if (hd <= 0 || (hd & 1) || hd > ORC_MAX_HEAD_DIM) return ORC_E_ARG;
        if (hd < c->hd_kv) return ORC_E_GEOMETRY;
    }
    for (int32_t t = 0; t < nt; t++)
        if (seq_ids[t] < 0 || seq_ids[t] >= c->n_seq) return ORC_E_ARG;
    for (int32_t t = 0; t < nt; t++)
        if (pos[t] < 0 || pos[t] >= c->capacity) return ORC_E_RANGE;
    int64_t *keys = (int64_t *)malloc(sizeof(int64_t) * (size_t)nt);
    if (!keys) return ORC_E_NOMEM;
    for (int32_t t = 0; t < nt; t++) keys[t] = ((int64_t)seq_ids[t] << 32) | (int64_t)pos[t];
    qsort(keys, (size_t)nt, sizeof(int64_t), cmp_i64);
    int dup = 0;
    for (int32_t t = 1; t < nt; t++) if (keys[t] == keys[t - 1]) dup = 1;
    free(keys);
    if (dup) return ORC_E_DUP;

    /* Checks passed: rotate q, then write every row. */
    if (q) {
        int st = orc_rope(q, nt, n_head, hd, pos, freq_base, freq_scale, style);
        if (st != ORC_OK) return st;
    }
    const int32_t nkt = c->n_head_kv * c->hd_kv;
    float *row = (float *)malloc(sizeof(float) * (size_t)nkt);
    if (!row) return ORC_E_NOMEM;
    for (int32_t t = 0; t < nt; t++) {
        memcpy(row, k + (size_t)t * nkt, sizeof(float) * (size_t)nkt);
        int st = orc_rope(row, 1, c->n_head_kv, c->hd_kv, &pos[t], freq_base, freq_scale, style);
        if (st != ORC_OK) { free(row); return st; }
        const size_t off = (size_t)pos[t] * nkt;
        store_values(c, orc_cache_region(c, 0, seq_ids[t], layer), off, row, nkt);
        store_values(c, orc_cache_region(c, 1, seq_ids[t], layer), off, v + (size_t)t * nkt, nkt);
        int32_t *hw = &c->hw[(size_t)seq_ids[t] * c->n_layer + layer];
        if (pos[t] + 1 > *hw) *hw = pos[t] + 1;
    }
    free(row);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Decode projections fused with the store ("13 · The decode loop and graph reuse"   */
/* §2.3: on a GPU build a decode step (nt = 1) merges the q/k/v matmuls, their biases, */
/* the two RoPEs and the two KV stores into one operation, and the fused and unfused   */
/* paths must give bit-identical results, §3.4 item 5).                               */
/* ------------------------------------------------------------------------------ */

/* out[t][j] = (sum_i x[t][i] * w[j][i]) + b[j].  Reading of the matmul's precision (the
 * pages fix only that fused and unfused agree bit for bit): the dot product is the f32
 * nearest to its exact value (here accumulated in binary128, where every f32 x f32
 * product is exact and 1024-term sums stay within ~1e-31 relative, then rounded once),
 * and the bias is added in f32 (one more rounding).  b may be NULL (no bias).
 * x: [nt][d]; w: [rows][d] (row j produces output j); out: [nt][rows]. */
int orc_project(const float *x, const float *w, const float *b, int32_t nt, int32_t rows,
                int32_t d, float *out)
{
    if (!x || !w || !out || nt < 0 || rows < 0 || d <= 0) return ORC_E_ARG;
    for (int32_t t = 0; t < nt; t++)
        for (int32_t j = 0; j < rows; j++) {
            __float128 acc = 0;
            const float *xr = x + (size_t)t * d, *wr = w + (size_t)j * d;
            for (int32_t i = 0; i < d; i++) acc += (__float128)xr[i] * (__float128)wr[i];
            float y = (float)acc;
            if (b) y = y + b[j];
            out[(size_t)t * rows + j] = y;
        }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* Attention ([MINFER-11] §2.1 "What attention computes", §2.4 GQA, §3.2.4 "GQA    */
/* attention", §3.2.5 softmax).                                                     */
/* ------------------------------------------------------------------------------ */

/* Sequential f32 dot product, one rounding per product and per sum. */
static float dot_f32(int32_t n, const float *a, const float *b)
{
    float s = 0.0f;
    for (int32_t i = 0; i < n; i++) s += a[i] * b[i];
    return s;
}

/* Kv head hk of row j of a region as f32 values: the region itself for an f32 cache,
 * the binary16 values widened into buf for an f16 cache, the head's Q8_0 blocks
 * dequantized into buf for a Q8_0 cache. */
static const float *head_row(const void *reg, int32_t dtype, size_t j, int32_t nkt, int32_t hk,
                             int32_t hd_kv, float *buf)
{
    const size_t off = j * (size_t)nkt + (size_t)hk * hd_kv;
    if (dtype == ORC_KV_F32) return (const float *)reg + off;
    if (dtype == ORC_KV_Q8_0) {
        orc_q8_dequantize_row((const orc_q8_block *)reg + off / ORC_Q8_BLOCK, hd_kv, buf);
        return buf;
    }
    const uint16_t *h = (const uint16_t *)reg + off;
    for (int32_t d = 0; d < hd_kv; d++) buf[d] = orc_f16_to_f32(h[d]);
    return buf;
}

/* One query row against vl rows of one kv head's slice of the regions: rows [0, vl), or,
 * when `cells` is given, rows cells[0 .. vl) in that order (an explicit window).
 *   score_j = (q . k_j) * scale                 (f32)
 *   e_j     = exp(score_j - max_j score_j)      (f32)
 *   sum     = sum_j e_j                          (f64)
 *   w_j     = e_j * (f32)(1 / sum)               (f32)
 *   out     = sum_j w_j * v_j, in j order        (f32)
 * Rows outside the window are the masked tail: their weight is exp(-inf) = 0 exactly and
 * their zero contribution is not formed. */
static void attend_row(const float *qrow, const void *kreg, const void *vreg, int32_t dtype,
                       int32_t nkt, int32_t hk, int32_t hd_kv, const int32_t *cells, int32_t vl,
                       float scale, float *scr, float *rowbuf, float *out)
{
    float mx = -INFINITY;
    for (int32_t j = 0; j < vl; j++) {
        const size_t row = cells ? (size_t)cells[j] : (size_t)j;
        const float *kr = head_row(kreg, dtype, row, nkt, hk, hd_kv, rowbuf);
        float s = dot_f32(hd_kv, qrow, kr) * scale;
        scr[j] = s;
        if (s > mx) mx = s;
    }
    double sum = 0.0;
    for (int32_t j = 0; j < vl; j++) {
        float e = expf(scr[j] - mx);
        scr[j] = e;
        sum += (double)e;
    }
    float inv = (float)(1.0 / sum);
    for (int32_t j = 0; j < vl; j++) scr[j] *= inv;
    for (int32_t d = 0; d < hd_kv; d++) out[d] = 0.0f;
    for (int32_t j = 0; j < vl; j++) {
        const size_t vrow = cells ? (size_t)cells[j] : (size_t)j;
        const float *vr = head_row(vreg, dtype, vrow, nkt, hk, hd_kv, rowbuf);
        float w = scr[j];
        for (int32_t d = 0; d < hd_kv; d++) out[d] += w * vr[d];
    }
}

/* The fused decode step: q = x Wq^T + bq, k = x Wk^T + bk, v = x Wv^T + bv (orc_project),
 * then exactly kv_append's work -- q rotated into q_out, k rotated and stored, v stored
 * -- so its results are the unfused path's by construction.
 * x: [nt][d_model]; wq: [n_head * hd][d_model]; wk, wv: [n_head_kv * hd_kv][d_model];
 * biases NULL or [rows]; q_out: [nt][n_head][hd]. */
int orc_qkv_rope_append(orc_cache *c, int32_t layer, int32_t nt, const int32_t *seq_ids,
                        const int32_t *pos, const float *x, int32_t d_model, const float *wq,
                        const float *bq, const float *wk, const float *bk, const float *wv,
                        const float *bv, int32_t n_head, int32_t hd, float *q_out,
                        float freq_base, float freq_scale, int32_t style)
{
    if (!c || layer < 0 || layer >= c->n_layer || nt < 0) return ORC_E_ARG;
    if (nt == 0) return ORC_OK;
    if (!x || !wq || !wk || !wv || !q_out || d_model <= 0) return ORC_E_ARG;
    if (n_head <= 0 || n_head % c->n_head_kv != 0) return ORC_E_ARG;
    if (hd <= 0 || (hd & 1) || hd > ORC_MAX_HEAD_DIM) return ORC_E_ARG;
    const int32_t nkt = c->n_head_kv * c->hd_kv;
    float *k = (float *)malloc(sizeof(float) * (size_t)nt * nkt);
    float *v = (float *)malloc(sizeof(float) * (size_t)nt * nkt);
    float *q = (float *)malloc(sizeof(float) * (size_t)nt * n_head * hd);
    int st = (!k || !v || !q) ? ORC_E_NOMEM : ORC_OK;
    if (st == ORC_OK) st = orc_project(x, wq, bq, nt, n_head * hd, d_model, q);
    if (st == ORC_OK) st = orc_project(x, wk, bk, nt, nkt, d_model, k);
    if (st == ORC_OK) st = orc_project(x, wv, bv, nt, nkt, d_model, v);
    /* orc_append_rope validates everything else before it writes anything. */
    if (st == ORC_OK)
        st = orc_append_rope(c, layer, nt, seq_ids, pos, q, n_head, hd, k, v, freq_base,
                             freq_scale, style);
    if (st == ORC_OK) memcpy(q_out, q, sizeof(float) * (size_t)nt * n_head * hd);
    free(k); free(v); free(q);
    return st;
}

static int check_heads(const orc_cache *c, int32_t n_head, int32_t hd)
{
    if (n_head <= 0 || n_head % c->n_head_kv != 0) return ORC_E_ARG;
    if (hd <= 0 || (hd & 1) || hd > ORC_MAX_HEAD_DIM) return ORC_E_ARG;
    if (hd < c->hd_kv) return ORC_E_GEOMETRY;
    return ORC_OK;
}

/* Work unit: one (token, query head) row.  Units never reduce against each other and
 * each owns its scratch, so the result is the same at any thread count.  Token t's window
 * is rows [0, pos[t]], or, when `cells` is given, the ncell[t] rows cells[t][..]. */
static int attend_units(const void *const *kregs, const void *const *vregs, int32_t dtype,
                        const int32_t *pos, const int32_t *const *cells, const int32_t *ncell,
                        int32_t nt, const float *q, int32_t n_head,
                        int32_t hd, int32_t n_head_kv, int32_t hd_kv, int32_t max_vl,
                        float scale, float *out, int32_t nthreads)
{
    const int32_t gqa = n_head / n_head_kv;
    const int32_t nkt = n_head_kv * hd_kv;
    const int64_t units = (int64_t)nt * n_head;
    int failed = 0;
#ifdef _OPENMP
    int nth = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nth)
#endif
    {
        float *scr = (float *)malloc(sizeof(float) * (size_t)(max_vl > 0 ? max_vl : 1));
        float *rowbuf = (float *)malloc(sizeof(float) * (size_t)hd_kv);
        if (!scr || !rowbuf) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
            failed = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t u = 0; u < units; u++) {
                int32_t t = (int32_t)(u / n_head), h = (int32_t)(u % n_head);
                int32_t hk = h / gqa;
                int32_t vl = cells ? ncell[t] : pos[t] + 1;
                attend_row(q + ((size_t)t * n_head + h) * hd, kregs[t], vregs[t], dtype, nkt,
                           hk, hd_kv, cells ? cells[t] : NULL, vl, scale, scr, rowbuf,
                           out + ((size_t)t * n_head + h) * hd_kv);
            }
        }
        free(scr);
        free(rowbuf);
    }
    (void)nthreads;
    return failed ? ORC_E_NOMEM : ORC_OK;
}

/* nt query tokens of one sequence.  Token t sees rows [0, pos[t]] of the layer's
 * regions: the causal mask is the window length, not a matrix.
 * q: [nt][n_head][hd] (rotated); out: [nt][n_head][hd_kv]. */
int orc_attn_prefill(const orc_cache *c, int32_t seq, int32_t layer, int32_t nt,
                     const int32_t *pos, const float *q, int32_t n_head, int32_t hd,
                     float scale, float *out, int32_t nthreads)
{
    if (!c || seq < 0 || seq >= c->n_seq || layer < 0 || layer >= c->n_layer || nt < 0)
        return ORC_E_ARG;
    if (nt == 0) return ORC_OK;
    if (!pos || !q || !out || !isfinite(scale)) return ORC_E_ARG;
    int st = check_heads(c, n_head, hd);
    if (st != ORC_OK) return st;
    int32_t max_vl = 0;
    for (int32_t t = 0; t < nt; t++) {
        if (pos[t] < 0 || pos[t] >= c->capacity) return ORC_E_RANGE;
        if (pos[t] + 1 > max_vl) max_vl = pos[t] + 1;
    }
    const void **kr = (const void **)malloc(sizeof(void *) * (size_t)nt);
    const void **vr = (const void **)malloc(sizeof(void *) * (size_t)nt);
    if (!kr || !vr) { free(kr); free(vr); return ORC_E_NOMEM; }
    const void *kreg = orc_cache_region((orc_cache *)c, 0, seq, layer);
    const void *vreg = orc_cache_region((orc_cache *)c, 1, seq, layer);
    for (int32_t t = 0; t < nt; t++) { kr[t] = kreg; vr[t] = vreg; }
    st = attend_units(kr, vr, c->dtype, pos, NULL, NULL, nt, q, n_head, hd, c->n_head_kv, c->hd_kv, max_vl,
                      scale, out, nthreads);
    free(kr); free(vr);
    return st;
}

/* One query token per batch entry b, at pos[b] of sequence seq_ids[b].  Entries only
 * read the cache, so two entries may name the same sequence.
 * q: [n_seq][n_head][hd]; out: [n_seq][n_head][hd_kv]. */
int orc_attn_decode(const orc_cache *c, int32_t layer, int32_t n_seq, const int32_t *seq_ids,
                    const int32_t *pos, const float *q, int32_t n_head, int32_t hd,
                    float scale, float *out, int32_t nthreads)
{
    if (!c || layer < 0 || layer >= c->n_layer || n_seq < 0) return ORC_E_ARG;
    if (n_seq == 0) return ORC_OK;
    if (!seq_ids || !pos || !q || !out || !isfinite(scale)) return ORC_E_ARG;
    int st = check_heads(c, n_head, hd);
    if (st != ORC_OK) return st;
    for (int32_t b = 0; b < n_seq; b++)
        if (seq_ids[b] < 0 || seq_ids[b] >= c->n_seq) return ORC_E_ARG;
    int32_t max_vl = 0;
    for (int32_t b = 0; b < n_seq; b++) {
        if (pos[b] < 0 || pos[b] >= c->capacity) return ORC_E_RANGE;
        if (pos[b] + 1 > max_vl) max_vl = pos[b] + 1;
    }
    const void **kr = (const void **)malloc(sizeof(void *) * (size_t)n_seq);
    const void **vr = (const void **)malloc(sizeof(void *) * (size_t)n_seq);
    if (!kr || !vr) { free(kr); free(vr); return ORC_E_NOMEM; }
    for (int32_t b = 0; b < n_seq; b++) {
        kr[b] = orc_cache_region((orc_cache *)c, 0, seq_ids[b], layer);
        vr[b] = orc_cache_region((orc_cache *)c, 1, seq_ids[b], layer);
    }
    st = attend_units(kr, vr, c->dtype, pos, NULL, NULL, n_seq, q, n_head, hd, c->n_head_kv, c->hd_kv,
                      max_vl, scale, out, nthreads);
    free(kr); free(vr);
    return st;
}

static int cmp_run(const void *a, const void *b)
{
    const int32_t *x = (const int32_t *)a, *y = (const int32_t *)b;
    return (x[0] > y[0]) - (x[0] < y[0]);
}

/* Decode over explicit windows ("13 · The decode loop and graph reuse" §2.2, Budget 3:
 * the cells a query may read are an input -- a list of runs -- resolved by the caller,
 * not a bound derived from positions; §3.4 "Pitfalls & invariants" item 4: rows past a
 * rolled-back cursor are never read because the window does not name them).
 * Query b attends, in its (seq_ids[b], layer) regions, the cells of its runs
 * r = run_off[b] .. run_off[b+1]-1, each run the rows [run_start[r], run_start[r] +
 * run_len[r]), taken in the listed order.  Reading of the run list (the pages name it but
 * do not define its encoding): every query has at least one run; every run is non-empty
 * and inside the region; the runs of one query name each cell at most once (a repeated
 * cell is refused, ORC_E_DUP, since it would count twice in the softmax).
 * q: [n][n_head][hd]; out: [n][n_head][hd_kv]. */
int orc_attn_decode_runs(const orc_cache *c, int32_t layer, int32_t n, const int32_t *seq_ids,
                         const int32_t *run_off, const int32_t *run_start,
                         const int32_t *run_len, const float *q, int32_t n_head, int32_t hd,
                         float scale, float *out, int32_t nthreads)
{
    if (!c || layer < 0 || layer >= c->n_layer || n < 0) return ORC_E_ARG;
    if (n == 0) return ORC_OK;
    if (!seq_ids || !run_off || !run_start || !run_len || !q || !out || !isfinite(scale))
        return ORC_E_ARG;
    int st = check_heads(c, n_head, hd);
    if (st != ORC_OK) return st;
    for (int32_t b = 0; b < n; b++)
        if (seq_ids[b] < 0 || seq_ids[b] >= c->n_seq) return ORC_E_ARG;
    if (run_off[0] != 0) return ORC_E_ARG;
    for (int32_t b = 0; b < n; b++)
        if (run_off[b + 1] <= run_off[b]) return ORC_E_ARG;   /* at least one run each */
    const int32_t nr = run_off[n];
    for (int32_t r = 0; r < nr; r++)
        if (run_len[r] <= 0) return ORC_E_ARG;
    for (int32_t r = 0; r < nr; r++)
        if (run_start[r] < 0 || (int64_t)run_start[r] + run_len[r] > c->capacity) return ORC_E_RANGE;
    /* Overlap: sort each query's runs by start and compare neighbours. */
    int32_t *tmp = (int32_t *)malloc(sizeof(int32_t) * 2 * (size_t)nr);
    int32_t *ncell = (int32_t *)malloc(sizeof(int32_t) * (size_t)n);
    int32_t **cells = (int32_t **)calloc((size_t)n, sizeof(int32_t *));
    const void **kr = (const void **)malloc(sizeof(void *) * (size_t)n);
    const void **vr = (const void **)malloc(sizeof(void *) * (size_t)n);
    st = ORC_OK;
    if (!tmp || !ncell || !cells || !kr || !vr) st = ORC_E_NOMEM;
    for (int32_t b = 0; st == ORC_OK && b < n; b++) {
        const int32_t r0 = run_off[b], r1 = run_off[b + 1];
        for (int32_t r = r0; r < r1; r++) {
            tmp[2 * r] = run_start[r];
            tmp[2 * r + 1] = run_len[r];
        }
        qsort(tmp + 2 * r0, (size_t)(r1 - r0), 2 * sizeof(int32_t), cmp_run);
        for (int32_t r = r0 + 1; r < r1; r++)
            if ((int64_t)tmp[2 * (r - 1)] + tmp[2 * (r - 1) + 1] > tmp[2 * r]) st = ORC_E_DUP;
    }
    int32_t max_vl = 0;
    for (int32_t b = 0; st == ORC_OK && b < n; b++) {
        int64_t total = 0;
        for (int32_t r = run_off[b]; r < run_off[b + 1]; r++) total += run_len[r];
        ncell[b] = (int32_t)total;   /* <= capacity: the runs are disjoint cells of a region */
        if (ncell[b] > max_vl) max_vl = ncell[b];
        cells[b] = (int32_t *)malloc(sizeof(int32_t) * (size_t)ncell[b]);
        if (!cells[b]) { st = ORC_E_NOMEM; break; }
        int32_t j = 0;
        for (int32_t r = run_off[b]; r < run_off[b + 1]; r++)
            for (int32_t i = 0; i < run_len[r]; i++) cells[b][j++] = run_start[r] + i;
        kr[b] = orc_cache_region((orc_cache *)c, 0, seq_ids[b], layer);
        vr[b] = orc_cache_region((orc_cache *)c, 1, seq_ids[b], layer);
    }
    if (st == ORC_OK)
        st = attend_units(kr, vr, c->dtype, NULL, (const int32_t *const *)cells, ncell, n, q,
                          n_head, hd, c->n_head_kv, c->hd_kv, max_vl, scale, out, nthreads);
    if (cells)
        for (int32_t b = 0; b < n; b++) free(cells[b]);
    free(cells); free(ncell); free(tmp); free(kr); free(vr);
    return st;
}

/* Threads the attention calls use when nthreads is 0. */
int32_t orc_max_threads(void)
{
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
