// Measurement helper for the benchmark (built as lib/libkvc_probe.so; not part of the
// attention library or its C ABI): a plain streaming read of a device buffer.
//
// Two uses: (1) the measured read ceiling that decode bandwidth is reported against,
// beside the 8 TB/s specification -- a grid-stride float4 read of a large buffer with
// ordinary or nontemporal loads, summed so the loads cannot be dropped; (2) a cache
// flush between timed calls: reading (not writing) a buffer larger than the 256 MB
// Infinity Cache evicts earlier data without leaving dirty lines for the next call to
// write back.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// U float4 loads per thread per trip, `stride` apart (1 or 2: measured faster than 4 or
// 8, which spread a wave's loads in flight over as many distant DRAM pages).
template <bool NT, int U>
__global__ void __launch_bounds__(256) stream_read_kernel(const floatx4 *__restrict__ a, int64_t n,
                                                          float *__restrict__ sink)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (; i + (U - 1) * stride < n; i += U * stride) {
        floatx4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            if constexpr (NT) v[u] = __builtin_nontemporal_load(a + i + u * stride);
            else v[u] = a[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < U; u++) acc += v[u];
    }
    for (; i < n; i += stride) acc += a[i];
    const float s = acc[0] + acc[1] + acc[2] + acc[3];
    // One value per workgroup, written only if it can never be true for finite data, so
    // the sum is live but the sink (blocks floats) is written at most rarely.
    if (s == 1.5e38f) sink[blockIdx.x] = s;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, buffer 16-byte aligned) of device memory at `buf` with
// `blocks` workgroups of 256 threads (0: 2048); `sink` holds at least `blocks` floats.
// nontemporal != 0 streams past the caches; unroll is 1 or 2 loads per thread per trip.
// Queued on `stream`; returns a hipError_t.
int kvc_probe_stream_read(const void *buf, int64_t bytes, float *sink, int32_t blocks,
                          int32_t nontemporal, int32_t unroll, void *stream)
{
    if (!buf || !sink || bytes < 16 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15) ||
        (unroll != 1 && unroll != 2))
        return (int)hipErrorInvalidValue;
    const int nb = blocks > 0 ? blocks : 2048;
    const int64_t n = bytes / 16;
    const floatx4 *a = static_cast<const floatx4 *>(buf);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (nontemporal && unroll == 2) stream_read_kernel<true, 2><<<nb, 256, 0, s>>>(a, n, sink);
    else if (nontemporal) stream_read_kernel<true, 1><<<nb, 256, 0, s>>>(a, n, sink);
    else if (unroll == 2) stream_read_kernel<false, 2><<<nb, 256, 0, s>>>(a, n, sink);
    else stream_read_kernel<false, 1><<<nb, 256, 0, s>>>(a, n, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
