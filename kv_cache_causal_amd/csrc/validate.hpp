// Host-side argument checks for every entry point of kvc.h.  Pure C++ (no HIP): the same
// source is compiled into the library and into a host-only test shim, so each error path
// can be exercised without a GPU.
//
// Every check runs before any device work; a non-OK status means nothing is written.
// Sources: "11 · Attention, vec ops, and the KV cache" §3.2.3 (a store position outside
// the region is an error, never a clamp), §3.2.4 and §3.3 (hd < hd_kv is refused),
// §2.4 (query heads map onto kv heads by integer division, so the counts must divide).
#pragma once

#include <cstdint>
#include <string>

#include "kvc.h"

namespace kvc {

struct Geometry {
    int32_t n_seq = 0, n_layer = 0, n_head_kv = 0, hd_kv = 0, capacity = 0;
};

// hd_kv values the attention kernels are built for.
bool supported_kv_head_dim(int32_t hd_kv);

kvc_status check_alloc(int32_t n_seq, int32_t n_layer, int32_t n_head_kv, int32_t hd_kv,
                       int32_t capacity, int32_t dtype, std::string &msg);

kvc_status check_append(const Geometry &g, int32_t layer, int32_t nt, const int32_t *seq_ids,
                        const int32_t *pos, const void *q, int32_t n_head, int32_t hd,
                        const void *k, const void *v, float freq_base, float freq_scale,
                        int32_t style, std::string &msg);

kvc_status check_prefill(const Geometry &g, int32_t seq, int32_t layer, int32_t nt,
                         const int32_t *pos, const void *q, int32_t n_head, int32_t hd,
                         float scale, const void *out, std::string &msg);

kvc_status check_decode(const Geometry &g, int32_t layer, int32_t n_seq, const int32_t *seq_ids,
                        const int32_t *pos, const void *q, int32_t n_head, int32_t hd,
                        float scale, const void *out, std::string &msg);

// Limits of the fused decode step: input width and tokens per call.
constexpr int32_t kMaxModelDim = 65536;
constexpr int32_t kMaxFusedTokens = 64;

kvc_status check_qkv(const Geometry &g, int32_t layer, int32_t nt, const int32_t *seq_ids,
                     const int32_t *pos, const void *x, int32_t d_model, const void *wq,
                     const void *bq, const void *wk, const void *bk, const void *wv,
                     const void *bv, int32_t n_head, int32_t hd, const void *q_out,
                     float freq_base, float freq_scale, int32_t style, std::string &msg);

kvc_status check_decode_runs(const Geometry &g, int32_t layer, int32_t n_seq,
                             const int32_t *seq_ids, const int32_t *run_off,
                             const int32_t *run_start, const int32_t *run_len, const void *q,
                             int32_t n_head, int32_t hd, float scale, const void *out,
                             std::string &msg);

}  // namespace kvc
