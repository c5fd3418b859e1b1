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

}  // namespace

hipError_t launch_stream_read(const void *ptr, uint64_t bytes, int grid, int unroll, bool nontemporal,
                              uint32_t *sink, hipStream_t st) {
    const uint4 *p = reinterpret_cast<const uint4 *>(ptr);
    return nontemporal ? launch<true>(p, bytes / 16, grid, unroll, sink, st)
                       : launch<false>(p, bytes / 16, grid, unroll, sink, st);
}

}  // namespace dkv
