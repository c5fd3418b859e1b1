// Decode attention computed by the host CPU over host-resident KV pages: the
// comparator for moving the attention to the KV instead of the KV to the GPU
// ("KV Cache 内存层级" overview, 2.2 挪计算：NEO: decoding attention is bound
// by memory bandwidth on either processor, and host DRAM bandwidth is within a
// small factor of the GPU's, so the CPU can take it over). It answers, on this
// machine, whether host cores next to DRAM beat the GPU reading the same
// pages over PCIe. Measurement only: decode_step never calls it.
//
// Work item = (sequence b, KV head g, a run of up to 64 pages). A thread
// streams the item's pages once for the G query heads of the group and keeps
// an online softmax state (log2 domain, q pre-scaled by log2(e)/sqrt(d), fp32)
// per head; the items of (b, g) and the fresh token are then merged in item
// order. Page layout: head-major runs, K rows then V rows of 16 tokens each,
// element (t, g, c, i) at ((g * 2 + c) * 16 + t) * d * 2 + 2 * i bytes.
//
// Host-only C++, built with the system compiler; the per-page loops are
// compiled for AVX-512, AVX2 and baseline x86-64 and chosen at load time.
#include "cpu_attention.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace dkv {
namespace {

constexpr int kPage = 16;
constexpr int kItemPages = 64;     // pages per work item (1024 tokens)
constexpr int kMaxGroup = 8;
constexpr int kMaxDim = 128;

inline float bf16_value(uint16_t bits) {
    const uint32_t u = (uint32_t)bits << 16;
    float f;
    std::memcpy(&f, &u, sizeof f);
    return f;
}

// Online-softmax state of one work item: G heads x d.
struct ItemState {
    float m[kMaxGroup], l[kMaxGroup];
    float acc[kMaxGroup * kMaxDim];
};

// Adds tokens [0, n) of one page run (K rows at `k`, V rows at `v`, row
// stride d) to the state of the G heads whose scaled queries are `qs`.
__attribute__((target_clones("avx512f", "avx2", "default")))
void add_page(const uint16_t *k, const uint16_t *v, int n, int G, int d, const float *qs, ItemState &st) {
    float s[kPage][kMaxGroup];
    float row[kMaxDim];
    for (int t = 0; t < n; ++t) {
        const uint16_t *kr = k + (size_t)t * d;
#pragma omp simd
        for (int i = 0; i < d; ++i) row[i] = bf16_value(kr[i]);
        for (int h = 0; h < G; ++h) {
            const float *qh = qs + h * d;
            float dot = 0.0f;
#pragma omp simd reduction(+ : dot)
            for (int i = 0; i < d; ++i) dot += qh[i] * row[i];
            s[t][h] = dot;
        }
    }
    for (int h = 0; h < G; ++h) {
        float mx = st.m[h];
        for (int t = 0; t < n; ++t) mx = std::max(mx, s[t][h]);
        if (mx > st.m[h]) {
            const float alpha = std::exp2(st.m[h] - mx);   // 0 while the state is empty
            st.l[h] *= alpha;
            float *a = st.acc + h * d;
#pragma omp simd
            for (int i = 0; i < d; ++i) a[i] *= alpha;
            st.m[h] = mx;
        }
    }
    for (int t = 0; t < n; ++t) {
        const uint16_t *vr = v + (size_t)t * d;
#pragma omp simd
        for (int i = 0; i < d; ++i) row[i] = bf16_value(vr[i]);
        for (int h = 0; h < G; ++h) {
            const float p = std::exp2(s[t][h] - st.m[h]);
            st.l[h] += p;
            float *a = st.acc + h * d;
#pragma omp simd
            for (int i = 0; i < d; ++i) a[i] += p * row[i];
        }
    }
}

void run_item(const CpuAttentionJob &j, int b, int g, int item, const float *qs, ItemState &st) {
    const int G = j.n_q_heads / j.n_kv_heads, d = j.head_dim;
    for (int h = 0; h < G; ++h) {
        st.m[h] = -INFINITY;
        st.l[h] = 0.0f;
    }
    std::fill(st.acc, st.acc + G * d, 0.0f);
    const int L = j.ctx_lens[b];
    const int p0 = item * kItemPages;
    const int p1 = std::min((L + kPage - 1) / kPage, p0 + kItemPages);
    const size_t tile = (size_t)kPage * d;        // elements of one K or V tile
    for (int p = p0; p < p1; ++p) {
        const uint16_t *run = reinterpret_cast<const uint16_t *>(j.pages[(size_t)b * j.max_pages + p]) +
                              (size_t)g * 2 * tile;
        add_page(run, run + tile, std::min(kPage, L - p * kPage), G, d, qs, st);
    }
}

}  // namespace

int cpu_attention_run(const CpuAttentionJob &j) {
    const int B = j.batch, Hq = j.n_q_heads, Hkv = j.n_kv_heads, d = j.head_dim;
    const int G = Hq / Hkv;
    int max_items = 0;
    for (int b = 0; b < B; ++b)
        max_items = std::max(max_items, (j.ctx_lens[b] + kPage * kItemPages - 1) / (kPage * kItemPages));
    const int64_t n_items = (int64_t)B * Hkv * max_items;

    // Scaled queries, log2 units.
    const float scale = (float)(1.4426950408889634 / std::sqrt((double)d));
    std::vector<float> qs((size_t)B * Hq * d);
    for (size_t i = 0; i < qs.size(); ++i) qs[i] = j.q[i] * scale;

    std::vector<ItemState> states((size_t)std::max<int64_t>(n_items, 1));
    std::atomic<int64_t> next{0};
    auto worker = [&]() {
        for (int64_t it = next.fetch_add(1); it < n_items; it = next.fetch_add(1)) {
            const int item = (int)(it % max_items);
            const int g = (int)((it / max_items) % Hkv);
            const int b = (int)(it / ((int64_t)max_items * Hkv));
            run_item(j, b, g, item, qs.data() + ((size_t)b * Hq + (size_t)g * G) * d, states[(size_t)it]);
        }
    };
    const int n_threads = std::max(1, j.n_threads);
    std::vector<std::thread> pool;
    for (int t = 1; t < n_threads; ++t) pool.emplace_back(worker);
    worker();
    for (auto &t : pool) t.join();

    // Merge each head's items in order, then the fresh token.
    for (int b = 0; b < B; ++b) {
        const int items = (j.ctx_lens[b] + kPage * kItemPages - 1) / (kPage * kItemPages);
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G, hl = h % G;
            const float *qh = qs.data() + ((size_t)b * Hq + h) * d;
            const uint16_t *kn = j.k_new + ((size_t)b * Hkv + g) * d;
            const uint16_t *vn = j.v_new + ((size_t)b * Hkv + g) * d;
            float s_new = 0.0f;
            for (int i = 0; i < d; ++i) s_new += qh[i] * bf16_value(kn[i]);
            float M = s_new;
            for (int it = 0; it < items; ++it)
                M = std::max(M, states[((size_t)b * Hkv + g) * max_items + it].m[hl]);
            float l = std::exp2(s_new - M);
            float o[kMaxDim];
            for (int i = 0; i < d; ++i) o[i] = l * bf16_value(vn[i]);
            for (int it = 0; it < items; ++it) {
                const ItemState &st = states[((size_t)b * Hkv + g) * max_items + it];
                const float w = std::exp2(st.m[hl] - M);
                l += w * st.l[hl];
                for (int i = 0; i < d; ++i) o[i] += w * st.acc[hl * d + i];
            }
            float *dst = j.out + ((size_t)b * Hq + h) * d;
            for (int i = 0; i < d; ++i) dst[i] = o[i] / l;
        }
    }
    return n_threads;
}

uint64_t cpu_stream_read(const void *p, uint64_t bytes, int n_threads) {
    const uint64_t *w = static_cast<const uint64_t *>(p);
    const uint64_t n = bytes / 8;
    n_threads = std::max(1, n_threads);
    std::vector<uint64_t> sums((size_t)n_threads, 0);
    auto worker = [&](int t) {
        const uint64_t lo = n * t / n_threads, hi = n * (t + 1) / n_threads;
        uint64_t s0 = 0, s1 = 0, s2 = 0, s3 = 0;
        uint64_t i = lo;
        for (; i + 4 <= hi; i += 4) {
            s0 += w[i];
            s1 += w[i + 1];
            s2 += w[i + 2];
            s3 += w[i + 3];
        }
        for (; i < hi; ++i) s0 += w[i];
        sums[(size_t)t] = s0 + s1 + s2 + s3;
    };
    std::vector<std::thread> pool;
    for (int t = 1; t < n_threads; ++t) pool.emplace_back(worker, t);
    worker(0);
    for (auto &t : pool) t.join();
    uint64_t total = 0;
    for (uint64_t s : sums) total += s;
    return total;
}

}  // namespace dkv
