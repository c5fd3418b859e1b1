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
// Producer wavefront streaming page runs into an LDS ring for a matrix-core
// consumer wavefront (groups of kMfmaMinGroup and more, head_dim 128).
constexpr int kSplitLdsMfma = 4;

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
    int32_t max_splits;     // splits of the cached tokens per sequence, at most
    int32_t part_slots;     // partial slots per (sequence, query head): max_splits + 1; sequence b's
                            // fresh token takes slot ceil(ctx_lens[b] / split_tokens), after its splits
    int32_t item_slots;     // work items the capacities allow: the sum over sequences of
                            // ceil((capacity[b] - 1) / split_tokens), at least 1
    float qscale;           // log2(e) / sqrt(head_dim): scores come out in log2 units
    int32_t split_variant;  // kSplitRegisters, kSplitLds, kSplitNaive, kSplitMfma or kSplitLdsMfma
    int32_t split_waves;    // register kernel: > 0 = that many wavefronts loop over the items
    int32_t proj_mfma_min_batch;  // batches from this size on project on MFMA, below on VALU
    int32_t proj_splitk_min_batch;  // MFMA batches from this size on split the hidden dimension
                                    // over workgroups (split-k); below, one workgroup per row block
    int32_t proj_ranges;          // split-k ranges of the hidden dimension (1, 2, 4, 8; 0 = by size)
    int32_t lds_ring;       // LDS producer/consumer kernels: ring slots (2, 3 or 4; 0 = the kernel's default)
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
    // scratch (the layout's, or the static array of decode_step_noalloc)
    float *proj_part;         // [ranges][batch][n_qkv] fp32 projection sums, one slab per range of
                              // the hidden dimension (one range below kProjSplitkMinBatch)
    float *q;                 // [batch][Hq][d] fp32, scaled by log2(e) / sqrt(d)
    float *part_o;            // [batch][Hq][part_slots][d] unnormalised outputs
    float2 *part_ml;          // [batch][Hq][part_slots] (running max, sum of weights)
    uint32_t *status;         // range flag (bit 0: a ctx_lens entry out of range)
    uint32_t *item_counter;   // looping split kernels: next work item to take (zeroed by the
                              // step's fresh-token kernel before the split kernel runs)
    uint32_t *item_list;      // [1 + batch * max_splits]: [0] = n, the number of (sequence, split)
                              // pairs with tokens this step; [1 + j] = (b << 16) | s, sequence-major.
                              // Written by the fresh-token kernel from ctx_lens; the split kernels
                              // take their work items from it.
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

// What kv_append's device path reads and writes: tokens [start, start + n)
// of one sequence and layer, from device buffers k, v [n][Hkv][d] bf16
// (16-byte aligned) into the pages of `page_table` (that sequence's row).
struct AppendArgs {
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t start;
    const uint64_t *page_table;
    const uint16_t *k;
    const uint16_t *v;
};

hipError_t launch_append(const AppendArgs &a, int n_tokens, hipStream_t stream);

// From this batch size (by default: every batch that projects on the matrix
// cores) the projection splits the hidden dimension into at most
// kProjMaxSplits ranges, each writing its own fp32 slab of
// StepArgs::proj_part; otherwise the projection writes one slab. The
// fresh-token kernel adds the slabs of its group's rows in range order.
// Scratch always has room for kProjMaxSplits slabs.
constexpr int kProjSplitkMinBatch = 8;
constexpr int kProjMaxSplits = 8;

// Scratch bytes of one decode step (each buffer 256-byte aligned in the order
// proj_part, q, part_o, part_ml, item counter, item list), so that one carve
// serves the layout-owned scratch and the static array of decode_step_noalloc
// alike.
struct ScratchPlan {
    size_t proj_part, q, part_o, part_ml, item_counter, item_list, total;
};
ScratchPlan scratch_plan(int batch, int n_q_heads, int n_kv_heads, int head_dim, int part_slots);
// Points a's scratch fields into `base` (an allocation of plan.total bytes).
void carve_scratch(StepArgs &a, char *base, const ScratchPlan &plan);

// Records a failed HIP call as the thread's last error; returns DKV_E_HIP.
dkv_status report_hip_error(hipError_t e, const char *what);

// Runs decode_step on `scratch` (capacity bytes of device memory) instead of
// the layout's own scratch: DKV_E_CAPACITY, with nothing enqueued, when the
// layout's step needs more. `who` names the entry point in error messages.
dkv_status decode_step_on_scratch(dkv_layout *layout, int32_t layer, const uint16_t *q_in, const uint16_t *W,
                                  const int32_t *ctx_lens, uint16_t *attn_out, dkv_stream_t stream, char *scratch,
                                  size_t capacity, const char *who);

// Enqueues the decode step's kernels on `stream`. With `events` non-null,
// records events[0] before the projection, events[1] after it, events[2]
// after the fresh-token kernel, events[3] after the split attention and
// events[4] after the combine.
hipError_t launch_decode_step(const StepArgs &a, hipStream_t stream, hipEvent_t *events, bool split_only);

// The four kernels of a step (each returns hipErrorInvalidValue for a shape
// outside its compiled variants, before launching anything). The projection
// reports how many slabs of proj_part it wrote.
// The projection form a step of these arguments runs (only the batch, the
// shape and the layout's thresholds matter): 0 VALU GEMV, 1 one-tile streamed
// MFMA, 2 split-k MFMA, 3 tiled MFMA.
enum ProjectionForm { kProjGemv = 0, kProjStream = 1, kProjSplitk = 2, kProjTiled = 3 };
int projection_form(const StepArgs &a);
hipError_t launch_projection(const StepArgs &a, int *ranges, hipStream_t stream);
hipError_t launch_fresh(const StepArgs &a, int ranges, hipStream_t stream);
hipError_t launch_split(const StepArgs &a, hipStream_t stream);
hipError_t launch_combine(const StepArgs &a, hipStream_t stream);

// GEMM C = A x B^T (bf16 in, fp32 out) with a row-major or CPU-aware tile order.
// B-stationary GEMM (each 128 x 512 tile of B fetched once): partial sums of
// C per 512-wide k tile in `workspace`, then added in k order.
uint64_t gemm_bstationary_workspace_bytes(int M, int N, int K);
hipError_t launch_gemm_nt_bstationary(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K,
                                      float *workspace, hipStream_t stream);
hipError_t launch_gemm_nt(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K,
                          bool cpu_aware, hipStream_t stream);

// Streaming-read probe (grid-stride, 16 B per lane per load, optionally
// nontemporal).
hipError_t launch_stream_read(const void *ptr, uint64_t bytes, int grid, int unroll,
                              bool nontemporal, uint32_t *sink, hipStream_t stream);
// Page-run read probe: `waves` wavefronts, wave w reading run w mod runs of
// pages_per_item consecutive pages of page_bytes each (item w / runs).
hipError_t launch_page_read(const void *ptr, int pages_per_item, int page_bytes, int runs, int waves, int skew,
                            uint32_t *sink, hipStream_t stream);

}  // namespace dkv
