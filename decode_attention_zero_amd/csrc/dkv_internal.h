// Internal declarations shared by the runtime and the kernels of the
// zero-copy decode-attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dkv.h"

namespace dkv {

constexpr int kPageTokens = DKV_PAGE_TOKENS;

// Split-attention kernel variants: one wavefront per work item with a
// register double buffer, or a producer wavefront streaming page runs into an
// LDS ring for consumer wavefronts.
constexpr int kSplitRegisters = 0;
constexpr int kSplitLds = 1;
// Comparator: one wavefront per query head, each KV head fetched G times.
constexpr int kSplitNaive = 2;
// Register double buffer with the group's scores and output update on the
// matrix cores (the default from groups of kMfmaMinGroup query heads).
constexpr int kSplitMfma = 3;
constexpr int kMfmaMinGroup = 4;

// Everything one decode step's kernels read or write. Built on the host by
// decode_step from the layout and the caller's pointers; passed by value.
struct StepArgs {
    // shape
    int32_t batch;
    int32_t hidden;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t n_qkv;          // (Hq + 2 Hkv) * d
    int32_t max_pages;      // page-table row length
    int32_t split_tokens;   // tokens per attention work item (multiple of 16)
    int32_t max_splits;     // partial slots per (sequence, query head)
    float qscale;           // log2(e) / sqrt(head_dim): scores come out in log2 units
    int32_t split_variant;  // kSplitRegisters, kSplitLds, kSplitNaive or kSplitMfma
    int32_t split_waves;    // register kernel: > 0 = that many wavefronts loop over the items
    int32_t proj_mfma_min_batch;  // batches from this size on project on MFMA, below on VALU
    int32_t lds_ring;       // LDS producer/consumer kernel: ring slots (2, 3 or 4)
    int32_t lds_poison;     // LDS producer/consumer kernel: 1 = fill each freed slot with NaN first
    // this layer's page table [batch][max_pages] of device addresses
    const uint64_t *page_table;
    const int32_t *capacity;  // [batch] slots per sequence (device)
    // caller's buffers
    const uint16_t *x;        // [batch][hidden] bf16
    const uint16_t *w;        // [n_qkv][hidden] bf16
    const int32_t *ctx_lens;  // [batch]
    void *out;                // [batch][Hq * d] bf16 or fp32
    int32_t out_f32;
    // layout-owned scratch
    float *q;                 // [batch][Hq][d] fp32, scaled by log2(e) / sqrt(d)
    uint16_t *kv_new;         // [batch][Hkv][2][d] bf16 (fresh K then V)
    float *part_o;            // [batch][Hq][max_splits][d] unnormalised outputs
    float2 *part_ml;          // [batch][Hq][max_splits] (running max, sum of weights)
    uint32_t *status;         // range flag (bit 0: a ctx_lens entry out of range)
    uint32_t *item_counter;   // looping split kernels: next work item to take (zeroed by the
                              // step's projection kernel before the split kernel runs)
};

// What kv_advance's kernel reads and writes (see kv_advance in dkv.h).
struct AdvanceArgs {
    int32_t batch;
    int32_t n_layers;
    int32_t max_pages;
    int32_t max_window;
    int64_t page_bytes;
    int32_t windowed;            // 0: only advance ctx_lens
    uint64_t *page_table;        // [n_layers][batch][max_pages]
    const uint64_t *host_pages;  // [n_layers][batch][max_pages] (windowed)
    const uint64_t *ring;        // [n_layers][batch][max_window] (windowed)
    const int32_t *window;       // [batch] (windowed)
    const int32_t *capacity;     // [batch]
    int32_t *ctx_lens;           // [batch], advanced in place
    uint32_t *status;
};

hipError_t launch_advance(const AdvanceArgs &a, hipStream_t stream);

// From this batch size the matrix-core projection splits the hidden dimension
// into at most kProjMaxSplits ranges and adds their fp32 partials in a second
// kernel; the partials take kProjMaxSplits * batch * n_qkv floats of
// layout-owned scratch (`proj_part` below).
constexpr int kProjSplitkMinBatch = 16;
constexpr int kProjMaxSplits = 8;

// Enqueues the decode step's kernels on `stream`. With `events` non-null,
// records events[0] before the projection, events[1] after it, events[2]
// after the split attention and events[3] after the combine. `proj_part` is
// the projection's partial-sum scratch (null for batches that do not use it).
hipError_t launch_decode_step(const StepArgs &a, float *proj_part, hipStream_t stream, hipEvent_t *events);

// The three kernels of a step (each returns hipErrorInvalidValue for a shape
// outside its compiled variants, before launching anything).
hipError_t launch_projection(const StepArgs &a, float *proj_part, hipStream_t stream);
hipError_t launch_split(const StepArgs &a, hipStream_t stream);
hipError_t launch_combine(const StepArgs &a, hipStream_t stream);

// GEMM C = A x B^T (bf16 in, fp32 out) with a row-major or CPU-aware tile order.
hipError_t launch_gemm_nt(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K,
                          bool cpu_aware, hipStream_t stream);

// Streaming-read probe (grid-stride, 16 B per lane per load, optionally
// nontemporal).
hipError_t launch_stream_read(const void *ptr, uint64_t bytes, int grid, int unroll,
                              bool nontemporal, uint32_t *sink, hipStream_t stream);

}  // namespace dkv
