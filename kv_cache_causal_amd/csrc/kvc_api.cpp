// The C ABI of kvc.h: handle, host validation, position staging, RoPE tables, launches.
//
// Per call: every argument is checked on the host (validate.cpp) before anything is
// queued.  Host-side integer arrays (positions, sequence ids, chunk offsets) ride in the
// kernel arguments when short, or in a pinned staging ring the kernels read in place
// when long; then the kernels are queued on the caller's stream.  The host waits for
// the device in kv_alloc (zero fill) and kv_free, and otherwise only when handle-owned
// memory grows or is reused: a scratch buffer replaced by a larger one (ensure_scratch),
// a staging slot still read by queued kernels (staging_push), or the staging ring grown
// (staging_release).  Every allocation and staging step of a call comes before its first
// launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <string>
#include <vector>

#include "kvc.h"
#include "kvc_internal.hpp"
#include "validate.hpp"

namespace {

thread_local std::string g_err;

kvc_status fail(kvc_status st, const std::string &msg)
{
    g_err = msg;
    return st;
}

kvc_status hip_fail(hipError_t e, const char *what)
{
    return fail(KVC_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

#define KVC_HIP(call)                                             \
    do {                                                          \
        hipError_t e_ = (call);                                   \
        if (e_ != hipSuccess) return hip_fail(e_, #call);         \
    } while (0)

struct RopeTable {
    int32_t hd;
    float base, fscale;
    float2 *dev;
};

// Pinned, coherent host ring for the integer arrays a call sends along when they do not
// fit the kernel arguments (positions and sequence ids of long appends and prefills).
// The kernels read a slot in place through its device-visible address: no copy is
// queued.  A slot is reused only after the event recorded behind the kernels that read
// it has completed, so the host never waits unless it runs a full ring ahead.
struct Staging {
    int32_t *host = nullptr;
    int32_t *dev = nullptr;   // device view of `host`
    size_t cap = 0;   // ints
    size_t head = 0;
    uint64_t lap = 0;
    struct Use {
        size_t off, n;
        uint64_t lap;
        hipEvent_t ev;
    };
    std::deque<Use> inflight;
    std::vector<hipEvent_t> pool;
};

}  // namespace

struct kvc_cache {
    kvc::Geometry g;
    int device = 0;
    int32_t kv_fmt = kvc::kFmtF32;
    char *K = nullptr, *V = nullptr;
    int64_t region_bytes = 0;  // bytes per (seq, layer) region
    int64_t scale_off = 0;     // Q8_0: byte offset of the block scales within a region
    std::vector<int32_t> hw;
    mutable Staging st;
    mutable std::vector<RopeTable> tables;
    mutable float *part = nullptr;  // split-K partials
    mutable size_t part_cap = 0;    // floats
    mutable float *dq = nullptr;    // binary16 / Q8_0 prefill: the window's K and V as f32
    mutable size_t dq_cap = 0;      // floats
};

namespace {

void staging_release(Staging &st)
{
    for (auto &u : st.inflight) {
        (void)hipEventSynchronize(u.ev);
        (void)hipEventDestroy(u.ev);
    }
    st.inflight.clear();
    for (auto ev : st.pool) (void)hipEventDestroy(ev);
    st.pool.clear();
    if (st.host) (void)hipHostFree(st.host);
    st.host = nullptr;
    st.dev = nullptr;
    st.cap = st.head = 0;
}

kvc_status staging_alloc(Staging &st, size_t ints)
{
    KVC_HIP(hipHostMalloc(reinterpret_cast<void **>(&st.host), ints * sizeof(int32_t),
                          hipHostMallocMapped | hipHostMallocCoherent));
    KVC_HIP(hipHostGetDevicePointer(reinterpret_cast<void **>(&st.dev), st.host, 0));
    st.cap = ints;
    st.head = 0;
    return KVC_OK;
}

// Copy `n` host ints into the ring.  Returns the device-visible address through *dev.
// The caller must call staging_commit after queueing the kernels that read it.
kvc_status staging_push(Staging &st, const std::vector<int32_t> &data, const int32_t **dev)
{
    const size_t n = (data.size() + 63) & ~size_t(63);  // keep slots 256-byte aligned
    if (n > st.cap) {
        size_t cap = st.cap ? st.cap : 65536;
        while (cap < n) cap *= 2;
        staging_release(st);
        kvc_status r = staging_alloc(st, cap);
        if (r != KVC_OK) return r;
    }
    if (st.head + n > st.cap) {
        st.head = 0;
        st.lap++;
    }
    const size_t a = st.head, e = a + n;
    while (!st.inflight.empty()) {
        Staging::Use &u = st.inflight.front();
        const bool stale = u.lap + 1 < st.lap;
        const bool overlaps = u.lap < st.lap && u.off < e;
        if (!stale && !overlaps) break;
        KVC_HIP(hipEventSynchronize(u.ev));
        st.pool.push_back(u.ev);
        st.inflight.pop_front();
    }
    std::memcpy(st.host + a, data.data(), data.size() * sizeof(int32_t));
    st.head = e;
    *dev = st.dev + a;
    st.inflight.push_back(Staging::Use{a, n, st.lap, nullptr});
    return KVC_OK;
}

kvc_status staging_commit(Staging &st, hipStream_t s)
{
    hipEvent_t ev;
    if (!st.pool.empty()) {
        ev = st.pool.back();
        st.pool.pop_back();
    } else {
        KVC_HIP(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
    }
    KVC_HIP(hipEventRecord(ev, s));
    st.inflight.back().ev = ev;
    return KVC_OK;
}

// Drop the slot pushed last when its kernels could not be queued.
void staging_abort(Staging &st)
{
    if (!st.inflight.empty() && st.inflight.back().ev == nullptr) st.inflight.pop_back();
}

// KVC_ROPE_EXACT=1 builds RoPE tables with every entry evaluated in double-double
// rather than only the few the f64 evaluation cannot certify (tests of that path; the
// entries are the same).
bool env_rope_exact()
{
    const char *e = std::getenv("KVC_ROPE_EXACT");
    return e && std::atoi(e) != 0;
}

kvc_status get_table(const kvc_cache *c, int32_t hd, float base, float fscale, hipStream_t s,
                     const float2 **out)
{
    for (const RopeTable &t : c->tables) {
        if (t.hd == hd && t.base == base && t.fscale == fscale) {
            *out = t.dev;
            return KVC_OK;
        }
    }
    RopeTable t{hd, base, fscale, nullptr};
    const size_t bytes = (size_t)c->g.capacity * (size_t)(hd / 2) * sizeof(float2);
    if (hipMalloc(reinterpret_cast<void **>(&t.dev), bytes) != hipSuccess)
        return fail(KVC_E_NOMEM, "RoPE table allocation failed");
    hipError_t e = kvc::launch_rope_table(t.dev, c->g.capacity, hd, base, fscale,
                                          env_rope_exact(), s);
    if (e != hipSuccess) {
        (void)hipFree(t.dev);
        return hip_fail(e, "rope table kernel");
    }
    c->tables.push_back(t);
    *out = t.dev;
    return KVC_OK;
}

float log2e_times(float scale) { return (float)((double)scale * 1.4426950408889634074); }

// Optional override of the decode chunk size (rows), read at each call; 0 = automatic.
int32_t env_split_rows()
{
    const char *e = std::getenv("KVC_SPLIT_ROWS");
    return e ? std::max(0, std::atoi(e)) : 0;
}

// KVC_PREFILL_SEG sets the prefill's key tiles per segment: unset or 0 lets the plan
// choose, n > 0 forces segments of n tiles, a negative value forbids splitting (tuning
// and tests of both paths; results agree within rounding).
int32_t env_prefill_seg()
{
    const char *e = std::getenv("KVC_PREFILL_SEG");
    return e ? std::atoi(e) : 0;
}

// Grow a scratch buffer of the handle to `need` floats.  The old buffer may still be
// read by queued kernels on `s`, so it is freed after a sync.
kvc_status ensure_scratch(float *&buf, size_t &buf_cap, size_t need, hipStream_t s,
                          const char *what)
{
    if (need <= buf_cap) return KVC_OK;
    if (buf) {
        KVC_HIP(hipStreamSynchronize(s));
        (void)hipFree(buf);
        buf = nullptr;
    }
    const size_t cap = std::max(need, buf_cap * 2);
    buf_cap = 0;
    if (hipMalloc(reinterpret_cast<void **>(&buf), cap * sizeof(float)) != hipSuccess)
        return fail(KVC_E_NOMEM, std::string(what) + " scratch allocation failed");
    buf_cap = cap;
    return KVC_OK;
}

// The split-K partials buffer, shared by decode and prefill.
kvc_status ensure_part(const kvc_cache *c, size_t need, hipStream_t s)
{
    return ensure_scratch(c->part, c->part_cap, need, s, "split-K");
}

// Split-K decode of n_seq validated entries.  Entry b's window is rows [0, pos[b]]
// (run_off == nullptr) or the union of its runs run_off[b] .. run_off[b+1]-1.  The
// split-K records go to the handle's scratch (grown on demand), or, with fixed != nullptr,
// to the fixed_cap floats at `fixed` (a call that needs more is refused, nothing queued).
kvc_status decode_driver(const kvc_cache *c, int32_t layer, int32_t n_seq, const int32_t *seq_ids,
                         const int32_t *pos, const int32_t *run_off, const int32_t *run_start,
                         const int32_t *run_len, const float *q, int32_t n_head, int32_t hd,
                         float scale, float *out, hipStream_t s, float *fixed = nullptr,
                         size_t fixed_cap = 0)
{
    const bool runs = run_off != nullptr;
    auto window_rows = [&](int32_t b) -> int64_t {
        if (!runs) return (int64_t)pos[b] + 1;
        int64_t t = 0;
        for (int32_t r = run_off[b]; r < run_off[b + 1]; r++) t += run_len[r];
        return t;
    };
    // Chunk size (plan.cpp); KVC_SPLIT_ROWS overrides it (tuning only, never the result).
    const int32_t hpb = kvc::decode_heads_per_block(c->kv_fmt, c->g.n_head_kv,
                                                    n_head / c->g.n_head_kv);
    const int32_t br = kvc::decode_block_rows(c->g.hd_kv, n_head / c->g.n_head_kv, c->kv_fmt, hpb);
    int64_t total_rows = 0;
    for (int32_t b = 0; b < n_seq; b++) total_rows += window_rows(b);
    const int32_t forced = env_split_rows();
    int64_t rows = kvc::decode_chunk_rows(total_rows * c->g.n_head_kv, br, hpb, forced);
    if (forced <= 0 && n_seq <= kvc::kInlineEntries) {
        // One launch: chunks whose workgroups all run at once, when such chunks balance.
        const int32_t slots = kvc::decode_resident_blocks(
            c->device, c->g.hd_kv, n_head / c->g.n_head_kv, c->kv_fmt, hpb, n_seq);
        if (!runs) {
            int64_t len[kvc::kInlineEntries];
            for (int32_t b = 0; b < n_seq; b++) len[b] = (int64_t)pos[b] + 1;
            rows = kvc::decode_one_round_rows(len, n_seq, c->g.n_head_kv, hpb, slots, br, rows,
                                              kvc::decode_one_round_excess(c->kv_fmt));
        } else {
            std::vector<int64_t> len(run_len + run_off[0], run_len + run_off[n_seq]);
            rows = kvc::decode_one_round_rows(len.data(), (int32_t)len.size(), c->g.n_head_kv,
                                              hpb, slots, br, rows,
                                              kvc::decode_one_round_excess(c->kv_fmt));
        }
    }
    // Chunks of entry b: its window cut into pieces of at most `rows` rows (each run on
    // its own for an explicit window).
    auto chunks_of = [&](int32_t b) -> int64_t {
        if (!runs) return ((int64_t)pos[b] + rows) / rows;
        int64_t ch = 0;
        for (int32_t r = run_off[b]; r < run_off[b + 1]; r++) ch += (run_len[r] + rows - 1) / rows;
        return ch;
    };

    // Launches of up to kInlineEntries entries; the partials buffer fits the largest.
    const int32_t E = kvc::kInlineEntries;
    int64_t max_chunks = 0;
    for (int32_t b0 = 0; b0 < n_seq; b0 += E) {
        int64_t ch = 0;
        for (int32_t b = b0; b < std::min(n_seq, b0 + E); b++) ch += chunks_of(b);
        max_chunks = std::max(max_chunks, ch);
    }
    if (max_chunks > (1 << 30)) return fail(KVC_E_ARG, "too many split-K chunks");
    const size_t need = (size_t)max_chunks * n_head * (c->g.hd_kv + 4);
    kvc_status pst = KVC_OK;
    if (fixed) {
        if (need > fixed_cap)
            return fail(KVC_E_ARG, "the call needs " + std::to_string(need) +
                                       " floats of split-K records; the fixed scratch holds " +
                                       std::to_string(fixed_cap) +
                                       " (fewer entries or shorter windows per call)");
    } else if ((pst = ensure_part(c, need, s)) != KVC_OK) {
        return pst;
    }
    float *part = fixed ? fixed : c->part;

    // Explicit windows: the (first row, rows) table of every chunk of every launch, staged
    // once before the first launch, so no staging step can fail after a launch.
    const int32_t *pieces_dev = nullptr;
    if (runs) {
        std::vector<int32_t> pieces;
        for (int32_t b = 0; b < n_seq; b++)
            for (int32_t r = run_off[b]; r < run_off[b + 1]; r++)
                for (int64_t o = 0; o < run_len[r]; o += rows) {
                    pieces.push_back(run_start[r] + (int32_t)o);
                    pieces.push_back((int32_t)std::min<int64_t>(rows, run_len[r] - o));
                }
        if ((pst = staging_push(c->st, pieces, &pieces_dev)) != KVC_OK) return pst;
    }

    int64_t chunk0 = 0;   // chunks of the entries before this launch's first
    for (int32_t b0 = 0; b0 < n_seq; b0 += E) {
        const int32_t n = std::min(E, n_seq - b0);
        kvc::DecodeParams p{};
        p.q = q + (int64_t)b0 * n_head * hd;
        p.out = out + (int64_t)b0 * n_head * c->g.hd_kv;
        p.part = part;
        p.kc = c->K;
        p.vc = c->V;
        p.region_bytes = c->region_bytes;
        p.scale_off = c->scale_off;
        p.n = n;
        p.n_head = n_head;
        p.hd = hd;
        p.n_head_kv = c->g.n_head_kv;
        p.hd_kv = c->g.hd_kv;
        p.n_layer = c->g.n_layer;
        p.layer = layer;
        p.kv_fmt = c->kv_fmt;
        p.rows_per_chunk = (int32_t)rows;
        p.hpb = hpb;
        p.qscale = log2e_times(scale);
        int32_t chunks = 0;
        for (int32_t i = 0; i < n; i++) {
            p.pos[i] = runs ? 0 : pos[b0 + i];
            p.seq[i] = seq_ids[b0 + i];
            p.cbase[i] = chunks;
            chunks += (int32_t)chunks_of(b0 + i);
        }
        p.cbase[n] = chunks;
        p.total_chunks = chunks;
        p.pieces = runs ? pieces_dev + 2 * chunk0 : nullptr;
        chunk0 += chunks;
        hipError_t e = kvc::launch_decode(p, s);
        if (e != hipSuccess) {
            // Record the slot's release behind whatever was queued before the failure.
            if (runs) (void)staging_commit(c->st, s);
            return hip_fail(e, "decode kernels");
        }
    }
    return runs ? staging_commit(c->st, s) : KVC_OK;
}

}  // namespace

extern "C" {

const char *kv_last_error(void) { return g_err.c_str(); }

kvc_status kv_alloc(kvc_cache **out, int32_t n_seq, int32_t n_layer, int32_t n_head_kv,
                    int32_t hd_kv, int32_t capacity, void *stream)
{
    return kv_alloc_typed(out, n_seq, n_layer, n_head_kv, hd_kv, capacity, KVC_KV_F32, stream);
}

kvc_status kv_alloc_typed(kvc_cache **out, int32_t n_seq, int32_t n_layer, int32_t n_head_kv,
                          int32_t hd_kv, int32_t capacity, kvc_kv_dtype dtype, void *stream)
{
    if (!out) return fail(KVC_E_ARG, "out is NULL");
    *out = nullptr;
    std::string msg;
    kvc_status st = kvc::check_alloc(n_seq, n_layer, n_head_kv, hd_kv, capacity, (int32_t)dtype,
                                     msg);
    if (st != KVC_OK) return fail(st, msg);

    kvc_cache *c = new (std::nothrow) kvc_cache();
    if (!c) return fail(KVC_E_NOMEM, "handle allocation failed");
    c->g = kvc::Geometry{n_seq, n_layer, n_head_kv, hd_kv, capacity};
    c->kv_fmt = (int32_t)dtype;
    const int64_t rows = ((int64_t)capacity + kvc::kRegionRowAlign - 1) / kvc::kRegionRowAlign *
                         kvc::kRegionRowAlign;
    const int64_t vals = rows * n_head_kv * hd_kv;
    if (dtype == KVC_KV_Q8_0) {
        c->scale_off = vals;                                    // int8 codes first
        c->region_bytes = vals + vals / kvc::kQ8Block * 2;      // then binary16 scales
    } else {
        c->region_bytes = vals * (dtype == KVC_KV_F16 ? 2 : 4);
    }
    c->hw.assign((size_t)n_seq * n_layer, 0);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const size_t bytes = (size_t)n_seq * n_layer * (size_t)c->region_bytes;

    auto cleanup = [&](kvc_status code, const std::string &m) {
        if (c->K) (void)hipFree(c->K);
        if (c->V) (void)hipFree(c->V);
        staging_release(c->st);
        delete c;
        return fail(code, m);
    };
    hipError_t e = hipGetDevice(&c->device);
    if (e != hipSuccess) return cleanup(KVC_E_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (hipMalloc(reinterpret_cast<void **>(&c->K), bytes) != hipSuccess ||
        hipMalloc(reinterpret_cast<void **>(&c->V), bytes) != hipSuccess) {
        (void)hipGetLastError();
        return cleanup(KVC_E_NOMEM, "KV region allocation of 2 x " + std::to_string(bytes) +
                                        " bytes failed");
    }
    if ((e = hipMemsetAsync(c->K, 0, bytes, s)) != hipSuccess ||
        (e = hipMemsetAsync(c->V, 0, bytes, s)) != hipSuccess)
        return cleanup(KVC_E_HIP, std::string("zero fill: ") + hipGetErrorString(e));
    if (staging_alloc(c->st, 65536) != KVC_OK) return cleanup(KVC_E_NOMEM, "staging allocation failed");
    if ((e = hipStreamSynchronize(s)) != hipSuccess)
        return cleanup(KVC_E_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
    // Look up (once per device) the fixed scratch of gqa_attn_decode_noalloc while this
    // device is current, so that entry point itself makes no runtime call to find it.  A
    // failure here only disables that entry point, which then reports it.
    float *fixed = nullptr;
    (void)kvc::static_scratch_addr(c->device, &fixed);
    (void)hipGetLastError();
    *out = c;
    return KVC_OK;
}

kvc_status kv_free(kvc_cache *c)
{
    if (!c) return KVC_OK;
    hipError_t e = hipDeviceSynchronize();
    staging_release(c->st);
    for (RopeTable &t : c->tables) (void)hipFree(t.dev);
    if (c->part) (void)hipFree(c->part);
    if (c->dq) (void)hipFree(c->dq);
    (void)hipFree(c->K);
    (void)hipFree(c->V);
    delete c;
    if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
    return KVC_OK;
}

kvc_status kv_view(const kvc_cache *c, int32_t seq, int32_t layer, void **k, void **v)
{
    if (!c || !k || !v) return fail(KVC_E_ARG, "NULL handle or output pointer");
    if (seq < 0 || seq >= c->g.n_seq || layer < 0 || layer >= c->g.n_layer)
        return fail(KVC_E_ARG, "seq/layer out of range");
    const size_t off = ((size_t)seq * c->g.n_layer + layer) * (size_t)c->region_bytes;
    *k = c->K + off;
    *v = c->V + off;
    return KVC_OK;
}

kvc_status kv_seq_len(const kvc_cache *c, int32_t seq, int32_t layer, int32_t *len)
{
    if (!c || !len) return fail(KVC_E_ARG, "NULL handle or output pointer");
    if (seq < 0 || seq >= c->g.n_seq || layer < 0 || layer >= c->g.n_layer)
        return fail(KVC_E_ARG, "seq/layer out of range");
    *len = c->hw[(size_t)seq * c->g.n_layer + layer];
    return KVC_OK;
}

kvc_status kv_append_rope(kvc_cache *c, int32_t layer, int32_t nt, const int32_t *seq_ids,
                          const int32_t *pos, float *q, int32_t n_head, int32_t hd,
                          const float *k, const float *v, float freq_base, float freq_scale,
                          kvc_rope_style style, void *stream)
{
    if (!c) return fail(KVC_E_ARG, "NULL handle");
    std::string msg;
    kvc_status st = kvc::check_append(c->g, layer, nt, seq_ids, pos, q, n_head, hd, k, v,
                                      freq_base, freq_scale, (int32_t)style, msg);
    if (st != KVC_OK) return fail(st, msg);
    if (nt == 0) return KVC_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    const float2 *tab_q = nullptr, *tab_k = nullptr;
    if (style != KVC_ROPE_NONE) {
        if ((st = get_table(c, c->g.hd_kv, freq_base, freq_scale, s, &tab_k)) != KVC_OK) return st;
        if (q && (st = get_table(c, hd, freq_base, freq_scale, s, &tab_q)) != KVC_OK) return st;
    }
    kvc::AppendParams p{};
    const bool inline_args = nt <= kvc::kInlineTokens;
    const int32_t *dev = nullptr;
    if (inline_args) {
        std::memcpy(p.ipos, pos, sizeof(int32_t) * nt);
        std::memcpy(p.iseq, seq_ids, sizeof(int32_t) * nt);
    } else {
        std::vector<int32_t> ints((size_t)nt * 2);
        std::memcpy(ints.data(), pos, sizeof(int32_t) * nt);
        std::memcpy(ints.data() + nt, seq_ids, sizeof(int32_t) * nt);
        if ((st = staging_push(c->st, ints, &dev)) != KVC_OK) return st;
    }

    p.q = style == KVC_ROPE_NONE ? nullptr : q;
    p.k = k;
    p.v = v;
    p.kc = c->K;
    p.vc = c->V;
    p.pos = inline_args ? nullptr : dev;
    p.seq = inline_args ? nullptr : dev + nt;
    p.tab_q = tab_q;
    p.tab_k = tab_k;
    p.region_bytes = c->region_bytes;
    p.scale_off = c->scale_off;
    p.nt = nt;
    p.n_head = n_head;
    p.hd = hd;
    p.n_head_kv = c->g.n_head_kv;
    p.hd_kv = c->g.hd_kv;
    p.n_layer = c->g.n_layer;
    p.layer = layer;
    p.style = (int32_t)style;
    p.kv_fmt = c->kv_fmt;
    hipError_t e = kvc::launch_append(p, s);
    if (e != hipSuccess) {
        if (!inline_args) staging_abort(c->st);
        return hip_fail(e, "append kernel");
    }
    if (!inline_args && (st = staging_commit(c->st, s)) != KVC_OK) return st;
    for (int32_t t = 0; t < nt; t++) {
        int32_t &w = c->hw[(size_t)seq_ids[t] * c->g.n_layer + layer];
        w = std::max(w, pos[t] + 1);
    }
    return KVC_OK;
}

kvc_status kv_qkv_rope_append(kvc_cache *c, int32_t layer, int32_t nt, const int32_t *seq_ids,
                              const int32_t *pos, const float *x, int32_t d_model,
                              const float *wq, const float *bq, const float *wk, const float *bk,
                              const float *wv, const float *bv, int32_t n_head, int32_t hd,
                              float *q_out, float freq_base, float freq_scale,
                              kvc_rope_style style, void *stream)
{
    if (!c) return fail(KVC_E_ARG, "NULL handle");
    std::string msg;
    kvc_status st = kvc::check_qkv(c->g, layer, nt, seq_ids, pos, x, d_model, wq, bq, wk, bk, wv,
                                   bv, n_head, hd, q_out, freq_base, freq_scale, (int32_t)style,
                                   msg);
    if (st != KVC_OK) return fail(st, msg);
    if (nt == 0) return KVC_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    kvc::QkvParams p{};
    if (style != KVC_ROPE_NONE) {
        if ((st = get_table(c, c->g.hd_kv, freq_base, freq_scale, s, &p.tab_k)) != KVC_OK) return st;
        if ((st = get_table(c, hd, freq_base, freq_scale, s, &p.tab_q)) != KVC_OK) return st;
    }
    std::memcpy(p.ipos, pos, sizeof(int32_t) * nt);
    std::memcpy(p.iseq, seq_ids, sizeof(int32_t) * nt);
    p.x = x;
    p.w[0] = wq;
    p.w[1] = wk;
    p.w[2] = wv;
    p.b[0] = bq;
    p.b[1] = bk;
    p.b[2] = bv;
    p.q_out = q_out;
    p.kc = c->K;
    p.vc = c->V;
    p.region_bytes = c->region_bytes;
    p.scale_off = c->scale_off;
    p.d = d_model;
    p.nt = nt;
    p.n_head = n_head;
    p.hd = hd;
    p.n_head_kv = c->g.n_head_kv;
    p.hd_kv = c->g.hd_kv;
    p.n_layer = c->g.n_layer;
    p.layer = layer;
    p.style = (int32_t)style;
    p.kv_fmt = c->kv_fmt;
    const int32_t ppu = kvc::qkv_pairs_per_unit(c->kv_fmt);
    p.units_q = n_head * ((hd / 2 + ppu - 1) / ppu);
    p.units_kv = c->g.n_head_kv * ((c->g.hd_kv / 2 + ppu - 1) / ppu);
    hipError_t e = kvc::launch_qkv(p, s);
    if (e != hipSuccess) return hip_fail(e, "fused projection kernel");
    for (int32_t t = 0; t < nt; t++) {
        int32_t &w = c->hw[(size_t)seq_ids[t] * c->g.n_layer + layer];
        w = std::max(w, pos[t] + 1);
    }
    return KVC_OK;
}

kvc_status gqa_attn_prefill(const kvc_cache *c, int32_t seq, int32_t layer, int32_t nt,
                            const int32_t *pos, const float *q, int32_t n_head, int32_t hd,
                            float scale, float *out, void *stream)
{
    if (!c) return fail(KVC_E_ARG, "NULL handle");
    std::string msg;
    kvc_status st = kvc::check_prefill(c->g, seq, layer, nt, pos, q, n_head, hd, scale, out, msg);
    if (st != KVC_OK) return fail(st, msg);
    if (nt == 0) return KVC_OK;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    // Work units (plan.cpp); positions travel only when they are not one contiguous run,
    // the unit table only when it is too long for the kernel arguments.
    const kvc::PrefillPlan pl = kvc::plan_prefill(pos, nt, n_head, c->g.n_head_kv, c->g.hd_kv,
                                                    env_prefill_seg());
    const bool units_inline = pl.units_per_hgroup <= kvc::kInlineUnits;
    std::vector<int32_t> ints;
    if (!pl.contiguous) ints.assign(pos, pos + nt);
    const size_t units_at = (ints.size() + 7) & ~size_t(7);   // 32-byte aligned
    if (!units_inline) {
        ints.resize(units_at, 0);
        ints.insert(ints.end(), pl.units.begin(), pl.units.end());
    }
    if (pl.max_seg > 1) {
        st = ensure_part(c, (size_t)pl.max_seg * nt * n_head * (c->g.hd_kv + 4), s);
        if (st != KVC_OK) return st;
    }
    // binary16 and Q8_0: the kernels read an f32 copy of rows [0, dq_rows) (whole 64-row
    // groups up to the largest position), written by a widening / dequantization pass on
    // the same stream.
    int32_t dq_rows = 0;
    if (c->kv_fmt != kvc::kFmtF32) {
        const int32_t top = *std::max_element(pos, pos + nt) + 1;
        dq_rows = (top + kvc::kRegionRowAlign - 1) / kvc::kRegionRowAlign * kvc::kRegionRowAlign;
        const size_t nkt = (size_t)c->g.n_head_kv * c->g.hd_kv;
        st = ensure_scratch(c->dq, c->dq_cap, 2 * (size_t)dq_rows * nkt, s, "f32 window copy");
        if (st != KVC_OK) return st;
    }
    const int32_t *dev = nullptr;
    const bool staged = !ints.empty();
    if (staged && (st = staging_push(c->st, ints, &dev)) != KVC_OK) return st;
    const size_t off = ((size_t)seq * c->g.n_layer + layer) * (size_t)c->region_bytes;
    kvc::PrefillParams p{};
    p.pos = pl.contiguous ? nullptr : dev;
    p.pos0 = pos[0];
    p.units = units_inline ? nullptr : dev + units_at;
    if (units_inline) std::copy(pl.units.begin(), pl.units.end(), p.iunits);
    p.part = pl.max_seg > 1 ? c->part : nullptr;
    p.dq = dq_rows ? c->dq : nullptr;
    p.dq_rows = dq_rows;
    p.GB = pl.GB;
    p.TQ = pl.TQ;
    p.n_qtiles = pl.n_qtiles;
    p.n_hsub = pl.n_hsub;
    p.units_per_hgroup = pl.units_per_hgroup;
    p.max_seg = pl.max_seg;
    p.q = q;
    p.out = out;
    p.kc = c->K + off;
    p.vc = c->V + off;
    p.kv_fmt = c->kv_fmt;
    p.scale_off = c->scale_off;
    p.nt = nt;
    p.n_head = n_head;
    p.hd = hd;
    p.n_head_kv = c->g.n_head_kv;
    p.hd_kv = c->g.hd_kv;
    p.capacity = c->g.capacity;
    p.qscale = log2e_times(scale);
    hipError_t e = kvc::launch_prefill(p, s);
    if (e != hipSuccess) {
        if (staged) staging_abort(c->st);
        return hip_fail(e, "prefill kernel");
    }
    return staged ? staging_commit(c->st, s) : KVC_OK;
}

kvc_status gqa_attn_decode(const kvc_cache *c, int32_t layer, int32_t n_seq,
                           const int32_t *seq_ids, const int32_t *pos, const float *q,
                           int32_t n_head, int32_t hd, float scale, float *out, void *stream)
{
    if (!c) return fail(KVC_E_ARG, "NULL handle");
    std::string msg;
    kvc_status st = kvc::check_decode(c->g, layer, n_seq, seq_ids, pos, q, n_head, hd, scale,
                                      out, msg);
    if (st != KVC_OK) return fail(st, msg);
    if (n_seq == 0) return KVC_OK;
    return decode_driver(c, layer, n_seq, seq_ids, pos, nullptr, nullptr, nullptr, q, n_head, hd,
                         scale, out, reinterpret_cast<hipStream_t>(stream));
}

kvc_status gqa_attn_decode_noalloc(const kvc_cache *c, int32_t layer, int32_t n_seq,
                                   const int32_t *seq_ids, const int32_t *pos, const float *q,
                                   int32_t n_head, int32_t hd, float scale, float *out,
                                   void *stream)
{
    if (!c) return fail(KVC_E_ARG, "NULL handle");
    std::string msg;
    kvc_status st = kvc::check_decode(c->g, layer, n_seq, seq_ids, pos, q, n_head, hd, scale,
                                      out, msg);
    if (st != KVC_OK) return fail(st, msg);
    if (n_seq == 0) return KVC_OK;
    float *fixed = nullptr;
    hipError_t e = kvc::static_scratch_addr(c->device, &fixed);
    if (e != hipSuccess) return hip_fail(e, "fixed decode scratch (hipGetSymbolAddress)");
    return decode_driver(c, layer, n_seq, seq_ids, pos, nullptr, nullptr, nullptr, q, n_head, hd,
                         scale, out, reinterpret_cast<hipStream_t>(stream), fixed,
                         kvc::kStaticScratchFloats);
}

kvc_status gqa_attn_decode_runs(const kvc_cache *c, int32_t layer, int32_t n_seq,
                                const int32_t *seq_ids, const int32_t *run_off,
                                const int32_t *run_start, const int32_t *run_len, const float *q,
                                int32_t n_head, int32_t hd, float scale, float *out, void *stream)
{
    if (!c) return fail(KVC_E_ARG, "NULL handle");
    std::string msg;
    kvc_status st = kvc::check_decode_runs(c->g, layer, n_seq, seq_ids, run_off, run_start,
                                           run_len, q, n_head, hd, scale, out, msg);
    if (st != KVC_OK) return fail(st, msg);
    if (n_seq == 0) return KVC_OK;
    return decode_driver(c, layer, n_seq, seq_ids, nullptr, run_off, run_start, run_len, q,
                         n_head, hd, scale, out, reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
