// Host-CPU attention over a layout's host pages: the comparator for the
// design that computes attention on the CPU, next to host DRAM, instead of
// streaming the KV over the link. Host-only code (no HIP types).
#pragma once

#include <stdint.h>

namespace dkv {

struct CpuAttentionJob {
    int32_t batch, n_q_heads, n_kv_heads, head_dim;
    int32_t max_pages;              // row length of `pages`
    const char *const *pages;       // [batch][max_pages] CPU addresses of the cached tokens' pages
    const int32_t *ctx_lens;        // [batch] cached tokens
    const float *q;                 // [batch][Hq][d] fp32, unscaled
    const uint16_t *k_new, *v_new;  // [batch][Hkv][d] bf16 bits
    float *out;                     // [batch][Hq][d] fp32
    int32_t n_threads;
};

// Runs the job on n_threads host threads; returns the number of threads used.
int cpu_attention_run(const CpuAttentionJob &job);

// Sums `bytes` bytes (a multiple of 64) of host memory as 64-bit words on
// n_threads threads; the sum keeps the reads from being optimised away.
uint64_t cpu_stream_read(const void *p, uint64_t bytes, int n_threads);

}  // namespace dkv
