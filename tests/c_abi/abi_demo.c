/*
 * The library used from plain C, with no Python or torch in the process: device memory
 * from the HIP runtime, every call through include/kvc.h.  One sequence, one layer:
 * RoPE + append of an nt-token prompt, its causal prefill, then RoPE + append of one more
 * token and its decode; then one call that must fail (a position outside the region).
 *
 * usage: abi_demo <inputs> <outputs>
 *   inputs  int32 header {n_head, hd, n_head_kv, hd_kv, capacity, nt}, then f32 arrays
 *           q[nt][n_head][hd], k[nt][n_head_kv][hd_kv], v[nt][n_head_kv][hd_kv], then the
 *           decode token's q[n_head][hd], k[n_head_kv][hd_kv], v[n_head_kv][hd_kv].
 *           Positions are 0..nt-1 for the prompt and nt for the decode token.
 *   outputs f32 arrays: rotated prompt q, prefill out[nt][n_head][hd_kv], rotated decode
 *           q, decode out[n_head][hd_kv], the K and V regions' first nt + 1 rows; then
 *           int32 {status of the failing call, 1 if kv_last_error() said something}.
 * Exit status 0 on success, 1 on any unexpected failure (the message goes to stderr).
 */
#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kvc.h"

#define CHECK_HIP(x)                                                                    \
    do {                                                                                \
        hipError_t e_ = (x);                                                            \
        if (e_ != hipSuccess) {                                                         \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                     \
            return 1;                                                                   \
        }                                                                               \
    } while (0)
#define CHECK_KVC(x)                                                                    \
    do {                                                                                \
        kvc_status s_ = (x);                                                            \
        if (s_ != KVC_OK) {                                                             \
            fprintf(stderr, "%s: status %d: %s\n", #x, (int)s_, kv_last_error());       \
            return 1;                                                                   \
        }                                                                               \
    } while (0)

static int read_all(FILE *f, void *dst, size_t bytes)
{
    return fread(dst, 1, bytes, f) == bytes ? 0 : 1;
}

/* Host buffer of n floats read from f, copied to a new device buffer. */
static int upload(FILE *f, size_t n, float **dev)
{
    float *h = (float *)malloc(n * sizeof(float));
    if (!h || read_all(f, h, n * sizeof(float))) return 1;
    if (hipMalloc((void **)dev, n * sizeof(float)) != hipSuccess) return 1;
    if (hipMemcpy(*dev, h, n * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) return 1;
    free(h);
    return 0;
}

static int download(FILE *f, const void *dev, size_t bytes)
{
    void *h = malloc(bytes);
    if (!h || hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost) != hipSuccess) return 1;
    if (fwrite(h, 1, bytes, f) != bytes) return 1;
    free(h);
    return 0;
}

int main(int argc, char **argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: abi_demo <inputs> <outputs>\n");
        return 1;
    }
    FILE *in = fopen(argv[1], "rb");
    if (!in) return 1;
    int32_t hdr[6];
    if (read_all(in, hdr, sizeof(hdr))) return 1;
    const int32_t n_head = hdr[0], hd = hdr[1], n_head_kv = hdr[2], hd_kv = hdr[3];
    const int32_t capacity = hdr[4], nt = hdr[5];
    const size_t nq = (size_t)n_head * hd, nkv = (size_t)n_head_kv * hd_kv;
    float *q, *k, *v, *q1, *k1, *v1, *out, *out1;
    if (upload(in, nt * nq, &q) || upload(in, nt * nkv, &k) || upload(in, nt * nkv, &v) ||
        upload(in, nq, &q1) || upload(in, nkv, &k1) || upload(in, nkv, &v1)) {
        fprintf(stderr, "reading or uploading the inputs failed\n");
        return 1;
    }
    fclose(in);
    CHECK_HIP(hipMalloc((void **)&out, nt * (size_t)n_head * hd_kv * sizeof(float)));
    CHECK_HIP(hipMalloc((void **)&out1, (size_t)n_head * hd_kv * sizeof(float)));

    int32_t *pos = (int32_t *)malloc(sizeof(int32_t) * (size_t)(nt + 1));
    int32_t *seq = (int32_t *)calloc((size_t)nt + 1, sizeof(int32_t));
    for (int32_t t = 0; t <= nt; t++) pos[t] = t;
    const float scale = 0.125f;

    kvc_cache *c = NULL;
    CHECK_KVC(kv_alloc(&c, 1, 1, n_head_kv, hd_kv, capacity, NULL));
    CHECK_KVC(kv_append_rope(c, 0, nt, seq, pos, q, n_head, hd, k, v, 1e6f, 1.0f,
                             KVC_ROPE_NEOX, NULL));
    CHECK_KVC(gqa_attn_prefill(c, 0, 0, nt, pos, q, n_head, hd, scale, out, NULL));
    CHECK_KVC(kv_append_rope(c, 0, 1, seq, pos + nt, q1, n_head, hd, k1, v1, 1e6f, 1.0f,
                             KVC_ROPE_NEOX, NULL));
    CHECK_KVC(gqa_attn_decode(c, 0, 1, seq, pos + nt, q1, n_head, hd, scale, out1, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    int32_t len = 0;
    CHECK_KVC(kv_seq_len(c, 0, 0, &len));
    if (len != nt + 1) {
        fprintf(stderr, "kv_seq_len %d, expected %d\n", len, nt + 1);
        return 1;
    }
    /* A position outside the region is an error, reported before any device work. */
    const int32_t bad = capacity;
    const int32_t st = (int32_t)gqa_attn_decode(c, 0, 1, seq, &bad, q1, n_head, hd, scale, out1,
                                                NULL);
    const int32_t said = kv_last_error()[0] != '\0';

    void *kr = NULL, *vr = NULL;
    CHECK_KVC(kv_view(c, 0, 0, &kr, &vr));
    FILE *o = fopen(argv[2], "wb");
    if (!o) return 1;
    if (download(o, q, nt * nq * sizeof(float)) ||
        download(o, out, nt * (size_t)n_head * hd_kv * sizeof(float)) ||
        download(o, q1, nq * sizeof(float)) ||
        download(o, out1, (size_t)n_head * hd_kv * sizeof(float)) ||
        download(o, kr, (size_t)(nt + 1) * nkv * sizeof(float)) ||
        download(o, vr, (size_t)(nt + 1) * nkv * sizeof(float))) {
        fprintf(stderr, "writing the outputs failed\n");
        return 1;
    }
    if (fwrite(&st, sizeof(st), 1, o) != 1 || fwrite(&said, sizeof(said), 1, o) != 1) return 1;
    fclose(o);
    CHECK_KVC(kv_free(c));
    hipFree(q); hipFree(k); hipFree(v); hipFree(q1); hipFree(k1); hipFree(v1);
    hipFree(out); hipFree(out1);
    free(pos);
    free(seq);
    return 0;
}
