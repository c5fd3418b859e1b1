// Advancing a batch by one decoded token, on the device: ctx_lens[b] += 1,
// and in a layout with a sliding hot window, the page that the next slot
// opens is given an HBM page while the oldest page of the window is demoted
// to its host page. Hot KV in HBM and cold KV read in place from host memory
// is the placement the DirectKV digest ("长上下文 LLM 的零拷贝 KV Cache 卸载
// （OSDI 2026）") proposes in its limits / future-work section; doing the move
// in a kernel with fixed addresses keeps the whole decode step capturable in
// one HIP graph, the property the "KV Cache 内存层级" overview (2.1 去搬运：
// DirectKV) says staging copies lose.
#include "device_common.h"

namespace dkv {
namespace {

// One workgroup per sequence. Page P = ctx_lens[b] / 16 after the advance
// is the page the next decode step writes into. When it is a new page
// (ctx_lens[b] + 1 a multiple of 16), HBM ring slot P % W moves to it; the
// page that held that slot, P - W, is copied to its host page first (every
// layer), and the page table is repointed. Blocks touch only their own
// sequence's entries, so no ordering between blocks is needed; the next
// kernel on the stream sees the new table.
__global__ __launch_bounds__(256) void kv_advance_kernel(AdvanceArgs a) {
    const int b = blockIdx.x;
    const int L = a.ctx_lens[b];
    if (L < 0 || L + 1 >= a.capacity[b]) {       // no room for the next slot
        if (threadIdx.x == 0) atomicOr(a.status, 1u);
        return;
    }
    const int Ln = L + 1;
    if (a.windowed && Ln % kPageTokens == 0) {
        const int P = Ln / kPageTokens;
        const int W = a.window[b];
        const int old = P - W;
        for (int layer = 0; layer < a.n_layers; ++layer) {
            const size_t row = (size_t)layer * a.batch + b;
            uint64_t *pt = a.page_table + row * a.max_pages;
            const uint64_t hbm = a.ring[row * a.max_window + P % W];
            if (old >= 0) {
                const uint64_t host = a.host_pages[row * a.max_pages + old];
                const uint4 *src = reinterpret_cast<const uint4 *>(hbm);
                uint4 *dst = reinterpret_cast<uint4 *>(host);
                const int n16 = (int)(a.page_bytes / 16);
                for (int i = threadIdx.x; i < n16; i += blockDim.x) dst[i] = src[i];
                if (threadIdx.x == 0) pt[old] = host;
            }
            if (threadIdx.x == 0) pt[P] = hbm;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) a.ctx_lens[b] = Ln;
}

}  // namespace

hipError_t launch_advance(const AdvanceArgs &a, hipStream_t st) {
    if (a.batch <= 0) return hipErrorInvalidValue;
    kv_advance_kernel<<<a.batch, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace dkv
