// Host-side checks of the runtime and the CPU comparator, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code only and
// run without a GPU: pure host functions over their whole input range, the
// argument checks of every entry point that can fail before touching the
// device, the host-CPU attention on ragged pages, and the host-DRAM probe.
// Prints OK and exits 0 when every expectation holds.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "dkv.h"
#include "dkv_probe.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::printf("FAILED: %s (line %d)\n", #cond, __LINE__);      \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

int main() {
    const dkv_shape s{4096, 32, 8, 128, 1, 16};
    // Placement over a range of capacities and tails.
    for (int cap = 1; cap < 300; cap += 7)
        for (int tail = 0; tail < 400; tail += 13) {
            int32_t n = -1, f = -1;
            EXPECT(kv_placement(cap, tail, &n, &f) == DKV_OK);
            EXPECT(n == (cap + 15) / 16 && f >= 0 && f <= n);
        }
    int32_t n, f;
    EXPECT(kv_placement(0, 0, &n, &f) != DKV_OK);
    EXPECT(kv_placement(10, -1, &n, &f) != DKV_OK);
    EXPECT(kv_placement(10, 0, nullptr, &f) != DKV_OK);
    // Page offsets: in range and distinct for every element of a page.
    const int64_t pb = kv_page_bytes(&s);
    EXPECT(pb == 8 * 2 * 16 * 128 * 2);
    std::vector<char> seen((size_t)pb / 2, 0);
    for (int t = 0; t < 16; ++t)
        for (int g = 0; g < 8; ++g)
            for (int c = 0; c < 2; ++c)
                for (int i = 0; i < 128; ++i) {
                    const int64_t off = kv_page_offset(&s, t, g, c, i);
                    EXPECT(off >= 0 && off + 2 <= pb && off % 2 == 0);
                    if (off >= 0 && off + 2 <= pb) {
                        EXPECT(!seen[(size_t)off / 2]);
                        seen[(size_t)off / 2] = 1;
                    }
                }
    EXPECT(kv_page_offset(&s, 16, 0, 0, 0) == -1 && kv_page_offset(&s, 0, 8, 0, 0) == -1);
    EXPECT(kv_page_offset(&s, 0, 0, 2, 0) == -1 && kv_page_offset(&s, 0, 0, 0, 128) == -1);
    const dkv_shape bad{4096, 30, 8, 128, 1, 16};
    EXPECT(kv_page_bytes(&bad) == 0 && kv_page_bytes(nullptr) == 0);
    // Argument checks that fail before any device call.
    dkv_pool *pool = nullptr;
    EXPECT(kv_alloc_host(nullptr, 4, 0, &pool) == DKV_E_INVALID_ARG && pool == nullptr);
    EXPECT(kv_alloc_host(&s, 0, 0, &pool) == DKV_E_INVALID_ARG);
    EXPECT(kv_alloc_hbm(&bad, 4, &pool) == DKV_E_INVALID_ARG);
    EXPECT(kv_alloc_host(&s, (int64_t)1 << 40, 0, &pool) == DKV_E_OUT_OF_MEMORY && pool == nullptr);
    EXPECT(kv_alloc_hbm(&s, INT64_MAX, &pool) == DKV_E_OUT_OF_MEMORY && pool == nullptr);
    EXPECT(kv_pool_free(nullptr) == DKV_OK && kv_layout_free(nullptr) == DKV_OK);
    // A pointer that no kv_layout_create returned is refused without being read.
    int64_t not_a_layout[4] = {0, 0, 0, 0};
    dkv_layout *stranger = reinterpret_cast<dkv_layout *>(not_a_layout);
    int32_t tier = -7;
    EXPECT(kv_layout_split_tokens(stranger) == 0 && kv_layout_split_kernel(stranger) == -1 &&
           kv_layout_split_waves(stranger) == -1);
    EXPECT(kv_layout_set_split_kernel(stranger, 0) == DKV_E_INVALID_ARG);
    EXPECT(kv_layout_page_tier(stranger, 0, 0, &tier) == DKV_E_INVALID_ARG && tier == -7);
    EXPECT(kv_layout_timing_enable(stranger, 1, 4) == DKV_E_INVALID_ARG);
    EXPECT(kv_layout_timing_read(stranger, nullptr, nullptr, nullptr, nullptr, nullptr) == DKV_E_INVALID_ARG);
    EXPECT(kv_layout_check_status(stranger) == DKV_E_INVALID_ARG);
    EXPECT(kv_layout_free(stranger) == DKV_E_INVALID_ARG);
    EXPECT(std::strlen(dkv_last_error()) > 0);
    dkv_layout *layout = nullptr;
    const int32_t cap1[1] = {4};
    EXPECT(kv_layout_create(&bad, 1, cap1, nullptr, nullptr, nullptr, &layout) != DKV_OK && layout == nullptr);
    EXPECT(decode_step(nullptr, 0, nullptr, nullptr, nullptr, nullptr, nullptr) == DKV_E_INVALID_ARG);
    EXPECT(kv_advance(nullptr, nullptr, nullptr) == DKV_E_INVALID_ARG);
    EXPECT(dkv_gemm_bf16_nt(nullptr, nullptr, nullptr, 128, 128, 64, 0, nullptr) == DKV_E_INVALID_ARG);
    // Host-CPU attention on ragged pages: 3 sequences (0, 5 and 37 tokens).
    const dkv_shape s2{512, 8, 2, 64, 1, 16};
    const int64_t pb2 = kv_page_bytes(&s2);
    std::vector<std::vector<uint16_t>> store;
    const int32_t ctx[3] = {0, 5, 37};
    std::vector<const void *> table(3 * 3, nullptr);
    for (int b = 0; b < 3; ++b)
        for (int p = 0; p < (ctx[b] + 15) / 16; ++p) {
            store.emplace_back((size_t)pb2 / 2);
            for (size_t e = 0; e < store.back().size(); ++e)
                store.back()[e] = (uint16_t)(0x3C00 + (e * 7 + b * 13 + p) % 512);   // values in [2^-7, 2^-6)
            table[(size_t)b * 3 + p] = store.back().data();
        }
    std::vector<float> q(3 * 8 * 64), out(3 * 8 * 64);
    for (size_t e = 0; e < q.size(); ++e) q[e] = std::sin((double)e);
    std::vector<uint16_t> kn(3 * 2 * 64, 0x3F80), vn(3 * 2 * 64, 0x4000);
    int32_t used = 0;
    EXPECT(dkv_cpu_attention_pages(table.data(), 3, &s2, 3, q.data(), kn.data(), vn.data(), ctx, out.data(), 4,
                                   &used) == DKV_OK);
    EXPECT(used == 4);
    for (int i = 0; i < 8 * 64; ++i) EXPECT(out[i] == 2.0f);     // empty cache: the fresh V exactly
    for (float v : out) EXPECT(std::isfinite(v));
    const void *holes[3] = {nullptr, nullptr, nullptr};
    const int32_t one[1] = {1};
    EXPECT(dkv_cpu_attention_pages(holes, 3, &s2, 1, q.data(), kn.data(), vn.data(), one, out.data(), 1,
                                   nullptr) == DKV_E_INVALID_ARG);
    const int32_t huge[1] = {INT32_MAX};                         // rounds up to pages without overflow
    EXPECT(dkv_cpu_attention_pages(holes, 3, &s2, 1, q.data(), kn.data(), vn.data(), huge, out.data(), 1,
                                   nullptr) == DKV_E_INVALID_ARG);
    // Host-DRAM probe.
    std::vector<uint64_t> words(1 << 16);
    uint64_t want = 0;
    for (size_t i = 0; i < words.size(); ++i) want += words[i] = i * 2654435761u;
    uint64_t sum = 0;
    EXPECT(dkv_cpu_stream_read(words.data(), words.size() * 8, 3, &sum) == DKV_OK && sum == want);
    EXPECT(dkv_cpu_stream_read(words.data(), 100, 3, &sum) == DKV_E_INVALID_ARG);
    // The cold-read probe refuses a region count below 1 before touching the device.
    float ms = -1.0f;
    EXPECT(dkv_probe_stream_read_cycled(words.data(), 64, 0, 1, 1, 1, &ms) == DKV_E_INVALID_ARG && ms == -1.0f);
    // The page-run probe refuses shapes that do not divide before touching the device.
    EXPECT(dkv_probe_page_read(words.data(), 65536, 65536, 8, 12, 0, 1, &ms) == DKV_E_INVALID_ARG);   // 12 % 8
    EXPECT(dkv_probe_page_read(words.data(), 65536, 65536, 4, 8, 0, 1, &ms) == DKV_E_INVALID_ARG);    // 16 KiB runs
    EXPECT(dkv_probe_page_read(words.data(), 65536, 65536, 8, 16, 0, 1, &ms) == DKV_E_INVALID_ARG && ms == -1.0f);  // 1 page, 2 items
    std::printf(failures ? "FAILED %d\n" : "OK\n", failures);
    return failures ? 1 : 0;
}
