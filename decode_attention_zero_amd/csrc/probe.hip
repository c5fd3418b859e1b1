// Streaming-read probe of the decode-attention library: the read ceiling of
// a memory region (host-pinned over the host link, or HBM) as a kernel sees
// it, used as the denominator of the host-link roofline. Grid-stride 16-byte
// loads, U loads in flight per lane, optionally nontemporal.
#include "device_common.h"

namespace dkv {
namespace {

template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, uint64_t nvec,
                                                          uint32_t *sink) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t x = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t j = i + (uint64_t)u * stride;
            v[u] = j < nvec ? (NT ? load_stream(p + j) : p[j]) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (x == 0x9E3779B9u) sink[0] = x;   // keeps the loads alive
}

template <bool NT>
hipError_t launch(const uint4 *p, uint64_t nvec, int grid, int unroll, uint32_t *sink, hipStream_t st) {
    switch (unroll) {
        case 1: stream_read_kernel<1, NT><<<grid, 256, 0, st>>>(p, nvec, sink); break;
        case 2: stream_read_kernel<2, NT><<<grid, 256, 0, st>>>(p, nvec, sink); break;
        case 4: stream_read_kernel<4, NT><<<grid, 256, 0, st>>>(p, nvec, sink); break;
        case 8: stream_read_kernel<8, NT><<<grid, 256, 0, st>>>(p, nvec, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Page-run read: wave w streams run (w mod runs) of the pages of item
// w / runs, RUN16 16-byte loads per lane per run (one run in flight).
template <int RUN16>
__global__ __launch_bounds__(64) void page_read_kernel(const char *__restrict__ base, int pages_per_item,
                                                       int page_bytes, int runs, int skew, uint32_t *sink) {
    const int w = blockIdx.x;
    const int item = w / runs;
    const int run = w - item * runs;
    const int lane = threadIdx.x;
    const char *p0 = base + (size_t)item * pages_per_item * page_bytes + (size_t)run * RUN16 * 1024 + lane * 16;
    const int r = skew ? (int)(((int64_t)item * 13) % pages_per_item) : 0;
    uint32_t x = 0;
    for (int k = 0; k < pages_per_item; ++k) {
        int p = k + r;
        if (p >= pages_per_item) p -= pages_per_item;
        const char *q = p0 + (size_t)p * page_bytes;
        uint4 v[RUN16];
#pragma unroll
        for (int j = 0; j < RUN16; ++j) v[j] = load_stream(q + j * 1024);
#pragma unroll
        for (int j = 0; j < RUN16; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

hipError_t launch_page_read(const void *ptr, int pages_per_item, int page_bytes, int runs, int waves, int skew,
                            uint32_t *sink, hipStream_t st) {
    const char *p = reinterpret_cast<const char *>(ptr);
    switch (page_bytes / runs / 1024) {
        case 4: page_read_kernel<4><<<waves, 64, 0, st>>>(p, pages_per_item, page_bytes, runs, skew, sink); break;
        case 8: page_read_kernel<8><<<waves, 64, 0, st>>>(p, pages_per_item, page_bytes, runs, skew, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *ptr, uint64_t bytes, int grid, int unroll, bool nontemporal,
                              uint32_t *sink, hipStream_t st) {
    const uint4 *p = reinterpret_cast<const uint4 *>(ptr);
    return nontemporal ? launch<true>(p, bytes / 16, grid, unroll, sink, st)
                       : launch<false>(p, bytes / 16, grid, unroll, sink, st);
}

}  // namespace dkv
