// Set-up writes of cached tokens from device buffers: K/V rows that a
// device-side producer (a prefill on the GPU, say) left in HBM are scattered
// straight into their pages, host or HBM, by vector stores from the GPU --
// the pages' write path of the history KV into CPU memory (KV Offload wiki,
// Offload 的基本机制: swap-out moves KV blocks from HBM to host DRAM), here
// written directly in the page layout the attention kernel reads.
#include "device_common.h"

namespace dkv {
namespace {

// One workgroup per token slot; each thread copies 16-byte pieces of the
// token's K and V rows (Hkv * 2 rows of head_dim bf16) to the slot's page.
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a) {
    const int slot = a.start + (int)blockIdx.x;
    char *page = reinterpret_cast<char *>(a.page_table[slot / kPageTokens]);
    const int tin = slot % kPageTokens;
    const int pieces = a.head_dim / 8;                  // 16-byte pieces per row
    const int per_kv = a.n_kv_heads * pieces;
    for (int i = threadIdx.x; i < 2 * per_kv; i += blockDim.x) {
        const int c = i / per_kv;                       // 0 = K, 1 = V
        const int g = (i - c * per_kv) / pieces;
        const int p = i - c * per_kv - g * pieces;
        const uint16_t *src = (c == 0 ? a.k : a.v) + ((size_t)blockIdx.x * a.n_kv_heads + g) * a.head_dim + p * 8;
        char *dst = page + ((size_t)((g * 2 + c) * kPageTokens + tin) * a.head_dim + p * 8) * 2;
        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, int n_tokens, hipStream_t st) {
    if (n_tokens <= 0) return hipSuccess;
    kv_append_kernel<<<n_tokens, 256, 0, st>>>(a);
    return hipGetLastError();
}

}  // namespace dkv
