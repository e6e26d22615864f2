/*
 * kvc.h -- causal grouped-query attention over a per-layer KV cache, on MI355X (gfx950).
 *
 * One hot path, exposed as a C ABI of plain pointers and sizes:
 *   kv_alloc        size the per-(sequence, layer) K and V regions once, zeroed
 *   kv_append_rope  rotate q and k (RoPE) at positions given as data, write K/V rows
 *                   in place at those positions
 *   kv_qkv_rope_append  the decode step's q/k/v projections fused with RoPE and the store
 *   gqa_attn_prefill  nt query tokens of one sequence, token t attending rows [0, pos[t]]
 *   gqa_attn_decode   one query token per sequence for a batch of sequences
 *   gqa_attn_decode_runs  the same over explicit windows (lists of row runs)
 * plus kv_alloc_typed (binary16 or Q8_0 regions), kv_free, kv_view, kv_seq_len and
 * kv_last_error for storage format, ownership, inspection and error text.
 *
 * Sources (page titles; sections named per declaration):
 *   [MINFER-11] "11 · Attention, vec ops, and the KV cache"
 *   [ZEROCOPY]  "IV.2: Zero-copy KV cache"
 *   [MINFER-13] "13 · The decode loop and graph reuse"
 *
 * Conventions for every call
 *   - q, k, v and out are f32 (the cache regions are f32, binary16 or Q8_0, see
 *     kvc_kv_dtype).
 *     "device" pointers are HIP device memory; "host" pointers are
 *     ordinary host memory, read before the call returns (the caller may reuse them at
 *     once).  Device buffers must stay valid until the work queued on `stream` is done.
 *   - Device pointers must be 16-byte aligned and the tensors dense (row-major, no gaps).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls queue work and return;
 *     kv_alloc and kv_free wait for the device.  The other calls make the host wait only
 *     when handle-owned memory must grow or be reused:
 *       * a scratch buffer grows (split-K records of gqa_attn_prefill / gqa_attn_decode /
 *         gqa_attn_decode_runs, or the f32 window copy of a binary16 / Q8_0 prefill): the
 *         library waits for `stream` (hipStreamSynchronize) before freeing the old one;
 *       * the pinned staging ring wraps onto slots that queued kernels still read
 *         (hipEventSynchronize on those kernels), or grows for a call that needs more
 *         than it holds (every queued use is waited for first);
 *       * the first call with a new (head dim, base, freq_scale) allocates and builds
 *         its RoPE table (hipMalloc, one kernel).
 *     Sizes only grow, so after one call of each kind at its largest size no further
 *     call allocates or waits.  HIP graph capture: make those warm-up calls before
 *     capturing; a growth during capture fails with KVC_E_HIP (a capturing stream cannot
 *     be synchronised).  Calls on one handle must be issued from one host thread onto
 *     one stream (or be otherwise ordered): the handle's staging and scratch memory is
 *     reused call after call.
 *   - Store before attention: a row must be appended (on the same stream, earlier) before
 *     an attention call that reads it ([MINFER-11] §3.4).  Rows never written read as 0.
 *   - Every argument is checked on the host before any device work, and every
 *     allocation and staging a call needs is made before its first kernel is queued.
 *     On any non-OK status from those checks (KVC_E_ARG, KVC_E_GEOMETRY, KVC_E_RANGE,
 *     KVC_E_DUP, KVC_E_NOMEM, and KVC_E_HIP from an allocation or a wait) nothing is
 *     written: no cache row, no q element, no output element.  The one exception is a
 *     kernel launch that the HIP runtime refuses (KVC_E_HIP naming the kernels): the
 *     launches queued before it in the same call (a decode of more than 64 entries runs
 *     one launch per 64) may already have written their outputs.
 *     kv_last_error() then returns a message for the calling thread.
 *   - nt == 0 / n_seq == 0 is an OK no-op (after the handle and layer are checked).
 *
 * Limits of this implementation: hd_kv (the KV head dim) must be one of 16, 32, 64, 80, 96,
 * 112, 128, 160, 192, 256 (a Q8_0 cache: 32, 64, 128 or 256); the query head dim hd must
 * be even, <= 256 and >= hd_kv; positions < capacity <= 2^24.
 */
#ifndef KVC_H
#define KVC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvc_cache kvc_cache; /* opaque; owns the regions, tables and scratch */

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_E_ARG = 1,      /* bad pointer, size, index, style or unsupported head dim */
    KVC_E_GEOMETRY = 2, /* hd < hd_kv: a query head shorter than its key ([MINFER-11] §1, §3.3) */
    KVC_E_RANGE = 3,    /* a position < 0 or >= capacity: an error, never a clamp (§3.2.3) */
    KVC_E_DUP = 4,      /* one append names the same (sequence, position) twice */
    KVC_E_NOMEM = 5,    /* device or pinned host allocation failed */
    KVC_E_HIP = 6       /* a HIP runtime call failed (message holds hipGetErrorString) */
} kvc_status;

/* Which elements form a rotating pair ([MINFER-11] §3.2.2, the layout styles). */
typedef enum kvc_rope_style {
    KVC_ROPE_NEOX = 0,        /* (i, i + hd/2): Qwen2/Qwen3 */
    KVC_ROPE_INTERLEAVED = 1, /* (2i, 2i + 1): Llama */
    KVC_ROPE_NONE = 2         /* no rotation: a plain store of k and v, q untouched */
} kvc_rope_style;

/* Element format of the K and V regions.  F16 is the half-precision cache
 * ([MINFER-11] §2.5 "Storage" and §3.3): the store rounds each rotated k value and each
 * v value to IEEE binary16 (nearest, ties to even); attention widens them back to f32
 * and computes in f32.  It halves the bytes decode attention reads.
 * Q8_0 is the packed cache of the same section and of the FAQ on cache formats: each
 * row is cut into blocks of 32 values, 34 bytes each (3.76x fewer bytes than f32).  The
 * pages fix the size, not the arithmetic; the library takes the published GGML Q8_0
 * block: d = max|x| / 127 (f32 division), stored as binary16 (nearest, ties to even);
 * code = round(x * r) to nearest with halves away from zero, r = 1/d as an f32
 * division (r = 0 when d = 0); the value attention uses is f32(binary16 d) * code,
 * exact in f32, and the arithmetic after it is f32 as for the other formats.  Needs
 * hd_kv a multiple of 32 (each block inside one kv head).  Inputs to the store must be
 * finite; values beyond 127 * 65504 in magnitude overflow the scale. */
typedef enum kvc_kv_dtype {
    KVC_KV_F32 = 0,
    KVC_KV_F16 = 1,
    KVC_KV_Q8_0 = 2
} kvc_kv_dtype;

#define KVC_MAX_HEAD_DIM 256
#define KVC_MAX_CAPACITY (1 << 24)

/*
 * kv_alloc -- create a cache of n_seq x n_layer persistent regions.
 * [MINFER-11] §2.2 (each layer owns a K and a V region of n_kv_embd x n_ctx floats);
 * [ZEROCOPY] "A Vec with capacity is already a preallocated buffer" (reserve once);
 * [MINFER-13] §2.5 (the regions outlive every call that uses them).
 *
 *   out        host; receives the handle.
 *   n_seq      independent sequences (>= 1).
 *   n_layer    layers (>= 1).
 *   n_head_kv  KV heads per row (>= 1).
 *   hd_kv      KV head dim, one of 16, 32, 64, 80, 96, 112, 128, 160, 192, 256.
 *   capacity   rows per (sequence, layer) region, 1 .. 2^24.  Fixed for the handle's
 *              life: the regions never grow, move or get copied.
 *   stream     used for the zero fill; kv_alloc waits for it before returning.
 *
 * Layout in device memory: K[n_seq][n_layer][rows][n_head_kv * hd_kv], V likewise, with
 * rows = capacity rounded up to a multiple of 64 (the extra rows stay zero and are never
 * inside a window); row p of a region holds position p, kv head hk at columns
 * [hk*hd_kv, (hk+1)*hd_kv).  All rows start as +0.0f.
 * Errors: KVC_E_ARG (bad geometry or null out), KVC_E_NOMEM, KVC_E_HIP.  On error *out
 * is set to NULL and nothing stays allocated.
 */
kvc_status kv_alloc(kvc_cache **out, int32_t n_seq, int32_t n_layer, int32_t n_head_kv,
                    int32_t hd_kv, int32_t capacity, void *stream);

/*
 * kv_alloc_typed -- kv_alloc with an explicit region element format (kv_alloc is
 * kv_alloc_typed with KVC_KV_F32).  With KVC_KV_F16 every region element is 2 bytes;
 * everything else (layout, calls, errors) is as for kv_alloc.  With KVC_KV_Q8_0 a
 * region is rows * nkt int8 codes laid out [rows][nkt] (nkt = n_head_kv * hd_kv, the
 * code of value i of row p at byte p * nkt + i), followed directly by rows * nkt / 32
 * binary16 scales laid out [n_head_kv][rows / 4][hd_kv / 32][4] (the scale of value i of
 * row p, in kv head h = i / hd_kv and block b = (i % hd_kv) / 32, is entry
 * ((h * rows / 4 + p / 4) * hd_kv / 32 + b) * 4 + p % 4): the same 34 bytes per 32 values
 * as the interleaved block, as two planes so that code rows are aligned for vector loads,
 * with the scales of one block for 4 consecutive rows (4q .. 4q+3) in 8 contiguous bytes.
 * Zero bytes decode to +0.0.
 * Errors: as kv_alloc, plus KVC_E_ARG for an unknown format and KVC_E_GEOMETRY for a
 * Q8_0 cache whose hd_kv is not a multiple of 32, or is 96, 160 or 192 (this library's
 * Q8_0 kernels take the power-of-two head dims only).
 */
kvc_status kv_alloc_typed(kvc_cache **out, int32_t n_seq, int32_t n_layer, int32_t n_head_kv,
                          int32_t hd_kv, int32_t capacity, kvc_kv_dtype dtype, void *stream);

/*
 * kv_free -- wait for the device, then release every region, table and scratch buffer.
 * The regions live from kv_alloc to kv_free, across every call in between: the caller,
 * not any one call, decides when the cache ends ([MINFER-13] §2.5: the KV regions belong
 * to the cache and survive every rebuild of the step; [ZEROCOPY] "A Vec with capacity
 * is already a preallocated buffer": storage reserved once and kept).
 * Pointers from kv_view become invalid.  NULL is accepted (no-op).
 */
kvc_status kv_free(kvc_cache *c);

/*
 * kv_view -- borrow one (sequence, layer)'s regions without copying ([ZEROCOPY]
 * "Reading without copying": a live reference into the cache's own storage).
 *   k, v  host; each receives a device pointer to [capacity][n_head_kv * hd_kv] elements
 *         (f32, or binary16 for a KVC_KV_F16 cache; the region's first capacity rows),
 *         or to the start of a KVC_KV_Q8_0 region (codes, then scales at byte
 *         rows * n_head_kv * hd_kv, rows = capacity rounded up to 64; see
 *         kv_alloc_typed).
 *         The pointers never change for the handle's life and stay owned by it.
 * Errors: KVC_E_ARG for a NULL handle/pointer or seq/layer out of range.
 */
kvc_status kv_view(const kvc_cache *c, int32_t seq, int32_t layer, void **k, void **v);

/*
 * kv_seq_len -- high-water mark of one (sequence, layer): 1 + the largest position ever
 * appended there, 0 if none ([ZEROCOPY] the trait's seq_len).  Bookkeeping only: no
 * kernel reads it; attention windows come from the positions passed to each call.
 * Errors: KVC_E_ARG.
 */
kvc_status kv_seq_len(const kvc_cache *c, int32_t seq, int32_t layer, int32_t *len);

/*
 * kv_append_rope -- RoPE on q and k at the given positions, then write k and v rows in
 * place.  [MINFER-11] §2.3 and §3.2.2 (RoPE: speed_i = freq_scale / freq_base^(2i/d),
 * angle = position * speed_i, a 2-D rotation of each pair), §3.2.3 (the store: row t
 * goes to offset pos[t] * row width of its layer's region; a position outside the region
 * is an error); [ZEROCOPY] "The cache appends in place" (no reallocation, no copy of
 * existing rows).
 *
 *   layer       layer whose regions receive the rows.
 *   nt          tokens in this call.
 *   seq_ids     host [nt]: sequence of token t (0 .. n_seq-1).
 *   pos         host [nt]: position of token t (0 .. capacity-1).  (seq_ids[t], pos[t])
 *               pairs must be distinct within one call.
 *   q           device [nt][n_head][hd], rotated in place with head dim hd; may be NULL
 *               (then n_head and hd are ignored).
 *   n_head, hd  query heads (a multiple of n_head_kv) and query head dim (even,
 *               hd_kv <= hd <= 256).
 *   k, v        device [nt][n_head_kv][hd_kv].  k is rotated with head dim hd_kv and
 *               written to K[seq_ids[t]][layer][pos[t]]; v is written unchanged to V.
 *               The inputs k and v are not modified.
 *   freq_base, freq_scale  RoPE base and speed scale (finite, > 0; ignored for NONE).
 *   style       pair layout.
 *
 * Rounding: each speed and each cos/sin is the correctly rounded f32 of its exact value;
 * the angle is the f32 product f32(pos) * speed; each product and sum of the rotation is
 * rounded to f32 on its own (no fused multiply-add).  So rotated rows are bit-for-bit
 * reproducible on any machine.
 * Also raises the (seq, layer) high-water marks.
 * Errors: KVC_E_ARG, KVC_E_GEOMETRY (q given and hd < hd_kv), KVC_E_RANGE, KVC_E_DUP,
 * KVC_E_NOMEM, KVC_E_HIP.
 */
kvc_status kv_append_rope(kvc_cache *c, int32_t layer, int32_t nt, const int32_t *seq_ids,
                          const int32_t *pos, float *q, int32_t n_head, int32_t hd,
                          const float *k, const float *v, float freq_base, float freq_scale,
                          kvc_rope_style style, void *stream);

/*
 * kv_qkv_rope_append -- the decode step before attention, fused: the q, k and v
 * projections of nt input rows with their biases, RoPE on q and k, and the K/V store --
 * one kernel instead of three matmuls, three bias adds, two rotations and two stores
 * ([MINFER-13] §2.3: a GPU build fuses exactly these for one-token steps; §3.4 item 5:
 * fused and unfused results must be identical bit for bit).
 *
 *   x           device [nt][d_model] f32: the layer's normalised input rows.
 *   d_model     input width: a multiple of 4, at most 65536.
 *   wq          device [n_head * hd][d_model]: row j produces q value j (head j / hd).
 *   wk, wv      device [n_head_kv * hd_kv][d_model], likewise for k and v.
 *   bq, bk, bv  device [rows] biases, or NULL for none.
 *   q_out       device [nt][n_head][hd]: receives the rotated q.
 *   layer, nt, seq_ids, pos, n_head, hd, freq_base, freq_scale, style: as in
 *               kv_append_rope; nt is at most 64 (a decode batch).
 * Each projection value is the f32 nearest to the exact dot product of x's row and the
 * weight row, then plus the bias in f32 (a reading: the pages require only that fused
 * and unfused agree; this definition makes the result independent of summation order).
 * The k and v rows then go through exactly kv_append_rope's rotation and store, so the
 * cache equals what kv_append_rope writes from those projections, bit for bit, in every
 * region format; the high-water marks advance the same way.
 * Errors: as kv_append_rope (checked before any device work), plus KVC_E_ARG for NULL
 * inputs, a d_model that is not a multiple of 4 or too large, misaligned pointers (x,
 * weights, q_out 16-byte; biases 4-byte) and nt above 64.
 */
kvc_status kv_qkv_rope_append(kvc_cache *c, int32_t layer, int32_t nt, const int32_t *seq_ids,
                              const int32_t *pos, const float *x, int32_t d_model,
                              const float *wq, const float *bq, const float *wk, const float *bk,
                              const float *wv, const float *bv, int32_t n_head, int32_t hd,
                              float *q_out, float freq_base, float freq_scale,
                              kvc_rope_style style, void *stream);

/*
 * gqa_attn_prefill -- causal GQA attention for nt query tokens of one sequence.
 * [MINFER-11] §2.1 (score = q.k * scale over s <= t, softmax, weighted sum of v),
 * §2.4 (query head h reads kv head h / (n_head / n_head_kv)), §3.2.4 (the window of
 * token t is rows [0, pos[t]]: the mask is a length, not a matrix), §2.5 (online softmax
 * over tiles on a GPU).
 *
 *   seq, layer  the region pair read.
 *   nt          query tokens.
 *   pos         host [nt]: position of each query token (any order, repeats allowed).
 *   q           device [nt][n_head][hd], already rotated; the dot uses q[t][h][0:hd_kv].
 *   n_head, hd  as in kv_append_rope.
 *   scale       multiplies every dot product (the model's 1/sqrt(hd); finite).
 *   out         device [nt][n_head][hd_kv], overwritten.
 *
 * Positions (and, for short prompts, the work-unit table) are staged in pinned host
 * memory that the kernels read in place.  A prompt too short to fill the GPU has each
 * 64-query tile's key range split across workgroups whose (max, sum, output) records are
 * merged by log-sum-exp (§2.5's split, as in gqa_attn_decode); the records live in the
 * handle's scratch memory, which grows on demand (KVC_E_NOMEM if it cannot).  With a
 * binary16 or Q8_0 cache, K and V rows [0, 64 * ceil((max pos + 1) / 64)) are first
 * widened / dequantized into f32 scratch (8 bytes per value pair; same growth and error),
 * which the attention reads.
 * Errors: KVC_E_ARG, KVC_E_GEOMETRY, KVC_E_RANGE (a position >= capacity), KVC_E_NOMEM,
 * KVC_E_HIP.
 */
kvc_status gqa_attn_prefill(const kvc_cache *c, int32_t seq, int32_t layer, int32_t nt,
                            const int32_t *pos, const float *q, int32_t n_head, int32_t hd,
                            float scale, float *out, void *stream);

/*
 * gqa_attn_decode -- one query token per batch entry: entry b attends rows [0, pos[b]] of
 * sequence seq_ids[b].  Same mathematics as gqa_attn_prefill ([MINFER-11] §2.1, §2.4,
 * §3.2.4); long windows are split across workgroups and merged by log-sum-exp
 * ([MINFER-11] §2.5: split the KV axis across blocks, then reduce).
 *
 *   layer       the layer read.
 *   n_seq       batch entries.
 *   seq_ids     host [n_seq]: sequence of each entry (entries only read, so repeats are
 *               allowed).
 *   pos         host [n_seq]: position of each entry's query token.
 *   q           device [n_seq][n_head][hd], already rotated.
 *   n_head, hd, scale  as in gqa_attn_prefill.
 *   out         device [n_seq][n_head][hd_kv], overwritten.
 *
 * Positions and sequence ids travel in the kernel arguments (64 entries per launch).
 * The split-K partial records live in the handle's scratch memory, which grows on demand
 * (KVC_E_NOMEM if it cannot) before the first launch.
 * Errors: KVC_E_ARG, KVC_E_GEOMETRY, KVC_E_RANGE, KVC_E_NOMEM, KVC_E_HIP.
 */
kvc_status gqa_attn_decode(const kvc_cache *c, int32_t layer, int32_t n_seq,
                           const int32_t *seq_ids, const int32_t *pos, const float *q,
                           int32_t n_head, int32_t hd, float scale, float *out, void *stream);

/*
 * gqa_attn_decode_noalloc -- gqa_attn_decode for callers that cannot allocate memory
 * while they run: code recorded into a HIP graph, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, same kernels, same chunking and the same results
 * bit for bit; the split-K records go to a fixed scratch array of the library in device
 * memory instead of the handle's scratch, so the call never allocates, frees or waits
 * (no hipMalloc, hipFree, synchronisation or staging) and queues only the decode
 * kernels.
 *
 * Limit: the records of one launch (up to 64 entries) must fit the fixed scratch,
 * KVC_STATIC_SCRATCH_BYTES (16 MiB): chunks x n_head x (hd_kv + 4) floats.  The windows
 * of a call are cut into at most about 2048 x HPB / n_head_kv + n_seq chunks in all
 * (HPB, kv heads per workgroup: 2 for binary16 regions, and for Q8_0 regions with
 * n_head = 2 n_head_kv, when n_head_kv is even; else 1), fewer when longer chunks fill the
 * device in one round (e.g. 32 Qwen3-0.6B-shaped sequences of 8,192 rows, f32: about
 * 2.3 MB).  A call that needs more is refused with KVC_E_ARG before anything is queued.
 * Every call on one GPU shares that GPU's one copy of the array (it is held until the
 * process ends), so calls that overlap on one GPU -- on different streams, or from
 * different threads or handles without ordering -- race on it; calls ordered on one
 * stream do not.  Nothing in it needs clearing: every record a call reads is written
 * earlier in the same call.
 * Errors: as gqa_attn_decode (KVC_E_ARG also for a call beyond the limit); KVC_E_HIP if
 * the scratch array's address could not be found (looked up at kv_alloc).
 */
#define KVC_STATIC_SCRATCH_BYTES (16u << 20)
kvc_status gqa_attn_decode_noalloc(const kvc_cache *c, int32_t layer, int32_t n_seq,
                                   const int32_t *seq_ids, const int32_t *pos, const float *q,
                                   int32_t n_head, int32_t hd, float scale, float *out,
                                   void *stream);

/*
 * gqa_attn_decode_runs -- gqa_attn_decode over explicit windows: entry b attends the
 * rows its runs name instead of rows [0, pos[b]] ([MINFER-13] §2.2, Budget 3: the cells a
 * query may read are an input resolved by the caller, a list of runs, not a bound derived
 * from positions; §3.4 "Pitfalls & invariants" item 4: rows past a rolled-back cursor
 * are never read because no window names them).  Windows say which rows take part; they do not move
 * rows, so a caller that stores several sequences' rows in one region (at distinct
 * positions) reads each sequence's rows with its own runs.
 *
 *   layer, n_seq, seq_ids  as in gqa_attn_decode.
 *   run_off     host [n_seq + 1]: entry b's runs are r = run_off[b] .. run_off[b+1]-1;
 *               run_off[0] = 0 and every entry has at least one run.
 *   run_start   host [run_off[n_seq]]: first row of run r.
 *   run_len     host [run_off[n_seq]]: rows in run r (>= 1); rows
 *               [run_start[r], run_start[r] + run_len[r]) must lie in [0, capacity).
 *               The runs of one entry may come in any order but must not share a row.
 *   q, n_head, hd, scale, out  as in gqa_attn_decode.
 * The result is attention over the union of the entry's runs; the order of the runs
 * changes only the rounding (within the same tolerance as gqa_attn_decode).
 * The chunk table of every launch of the call is staged at once, before the first
 * launch, in pinned host memory that the kernels read in place.
 * Errors: KVC_E_ARG (also for a malformed run list), KVC_E_GEOMETRY, KVC_E_RANGE (a run
 * outside the region), KVC_E_DUP (two runs of one entry share a row), KVC_E_NOMEM,
 * KVC_E_HIP.
 */
kvc_status gqa_attn_decode_runs(const kvc_cache *c, int32_t layer, int32_t n_seq,
                                const int32_t *seq_ids, const int32_t *run_off,
                                const int32_t *run_start, const int32_t *run_len, const float *q,
                                int32_t n_head, int32_t hd, float scale, float *out, void *stream);

/*
 * kv_last_error -- text of the calling thread's last non-OK status ("" if none): the
 * message half of an error, beside the status code each call returns ([MINFER-11] §3.2.3:
 * a failing store returns an error carrying its reason, e.g. the position and n_ctx, and
 * the run stops rather than clamping).  The string is owned by the library and valid
 * until the thread's next call.
 */
const char *kv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
