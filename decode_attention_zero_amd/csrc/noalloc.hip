// decode_step_noalloc: the decode step on a file-scope device array instead
// of the layout's own scratch, for callers that cannot allocate device
// memory. The array is sized for every layout whose step needs at most
// kStaticScratchBytes (projection slabs, fp32 queries, split partials and
// the work-queue counter; the five workloads this library is measured on
// need 0.15 to 19 MB). Each GPU holds its own copy until the process ends.
#include <mutex>

#include "dkv_internal.h"

constexpr size_t kStaticScratchBytes = size_t(32) << 20;

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on each device, looked up once per device with
// that device current. In host code `scratch` names a host-side shadow, not
// device memory, so only these addresses are handed to kernels.
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(char **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = static_cast<char *>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t decode_step_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

dkv_status decode_step_noalloc(dkv_layout *kv_layout, int32_t layer, const uint16_t *q_in, const uint16_t *W_qkv,
                               const int32_t *ctx_lens, uint16_t *attn_out, dkv_stream_t stream) {
    char *base = nullptr;
    const hipError_t e = scratch_address(&base);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return dkv::report_hip_error(e, "decode_step_noalloc: address of the static scratch array");
    }
    return dkv::decode_step_on_scratch(kv_layout, layer, q_in, W_qkv, ctx_lens, attn_out, stream, base,
                                       kStaticScratchBytes, "decode_step_noalloc");
}

}  // extern "C"
