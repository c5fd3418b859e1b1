/*
 * dkv_probe.h -- measurement helpers of the zero-copy decode-attention
 * library: the streaming-read ceiling of a memory region as seen by a GPU
 * kernel, used as the denominator of the host-link roofline.
 *
 * The pages put the bottleneck of direct CPU-memory access on sustained link
 * bandwidth ("KV Cache 内存层级" overview, 2.1 去搬运：DirectKV: on a fast
 * link the deciding factor becomes sustained bandwidth, not single-access
 * latency) and warn that on PCIe-only platforms the kernel cannot beat the
 * physical link (DirectKV digest, 核心方法). This probe measures that link.
 */
#ifndef DKV_PROBE_H
#define DKV_PROBE_H

#include <stdint.h>

#include "dkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Device address, size in bytes and tier (0 host, 1 HBM) of a pool's
 * memory. Any output pointer may be NULL. */
dkv_status kv_pool_info(const dkv_pool *pool, void **device_base, int64_t *bytes,
                        int32_t *tier);

/* Times a streaming read of `bytes` bytes at device address `ptr` (host
 * mapped memory or HBM): a grid-stride kernel of `grid` x 256 threads,
 * 16-byte loads, `unroll` (1, 2, 4 or 8) loads in flight per thread; a
 * negative `unroll` (-1, -2, -4, -8) uses nontemporal loads instead. One
 * warm-up run, then `reps` timed runs on a private stream; *ms_median gets
 * the median in milliseconds. Synchronous. bytes must be a multiple of 16
 * and ptr 16-byte aligned. */
dkv_status dkv_probe_stream_read(const void *ptr, uint64_t bytes, int32_t grid,
                                 int32_t unroll, int32_t reps, float *ms_median);

/* The same read of `bytes` bytes, cold: timed run r reads region
 * r mod n_regions of n_regions consecutive regions at `ptr` (n_regions x
 * bytes in all), so that with n_regions x bytes beyond the GPU's caches
 * (256 MiB of last-level cache on MI355X) every timed run fetches its bytes
 * from memory, as a kernel that reads a fresh operand once per step does.
 * The warm-up run reads the last region. Same arguments and errors
 * otherwise; n_regions >= 1. */
dkv_status dkv_probe_stream_read_cycled(const void *ptr, uint64_t bytes, int32_t n_regions,
                                        int32_t grid, int32_t unroll, int32_t reps, float *ms_median);

/* The read ceiling in the split-attention kernel's own access pattern, with
 * no arithmetic: `bytes` at `ptr` are `page_bytes` pages of `runs` runs each
 * (page_bytes / runs bytes per run, a multiple of 1024); `waves` wavefronts
 * (a multiple of `runs`) each stream one run of every page of their share
 * (wave w reads run w mod runs of items w / runs, each item an equal stretch
 * of consecutive pages), with one run's nontemporal 16-byte loads in flight.
 * With skew != 0 each item starts at page (item x 13) mod its length and
 * wraps around. One warm-up run, then `reps` timed runs on a private stream;
 * *ms_median gets the median. DKV_E_INVALID_ARG when the shapes do not
 * divide (bytes by page_bytes, page_bytes by runs x 1024, the pages by the
 * items). */
dkv_status dkv_probe_page_read(const void *ptr, uint64_t bytes, int32_t page_bytes, int32_t runs,
                               int32_t waves, int32_t skew, int32_t reps, float *ms_median);

/* Comparator for measurement: the staging design the pages set against
 * zero-copy (KV Offload wiki, Offload 的基本机制: swap-in copies KV into a GPU
 * buffer before attention runs; KV-hierarchy overview, 2.1: staging costs a
 * reserved GPU buffer and doubled link traffic). Copies the first `bytes`
 * bytes of pool `src` into pool `dst` with hipMemcpyAsync (the copy engines)
 * on `stream`. Two fresh pools of the same page shape, handed to layouts of
 * the same capacities created in the same order, hold every page at the same
 * offset, so staging a host-placed layout's pool into the HBM-placed layout's
 * pool gives the latter the same KV. Errors: DKV_E_INVALID_ARG (null pool,
 * different page sizes, or bytes < 0 or beyond either pool). */
dkv_status kv_pool_copy(dkv_pool *dst, const dkv_pool *src, int64_t bytes, dkv_stream_t stream);

/* The QKV projection kernel the layout's decode steps run, fixed at creation
 * by the batch, the shape and the thresholds (DKV_PROJ_MFMA_MIN_BATCH,
 * DKV_PROJ_SPLITK_MIN_BATCH): 0 the VALU GEMV (below 8 sequences), 1 the
 * one-tile streamed MFMA kernel (on request, up to 16), 2 the split-k MFMA
 * kernel, 3 the tiled MFMA kernel (from 192 sequences, once its workgroups
 * fill half the CUs). -1 for a NULL or freed layout. Measurement and
 * reporting only. */
int32_t kv_layout_projection_kernel(const dkv_layout *layout);

/* Per-kernel timing of a layout's decode steps. While enabled, decode_step
 * records HIP events on its stream before and after each of its kernels
 * (enable = 1: projection, fresh token, split attention, combine) or only
 * around the split-attention kernel (enable = 2: two events per step, which
 * disturb short steps less; the other kernels then read as 0 ms), for up to
 * max_steps steps; enabling creates those events, so do it outside graph
 * capture. Disabling (enable = 0) destroys them. Errors: DKV_E_INVALID_ARG
 * (null or freed layout, enable not 0, 1 or 2, max_steps <= 0 when
 * enabling). */
dkv_status kv_layout_timing_enable(dkv_layout *layout, int32_t enable, int32_t max_steps);

/* Synchronises, then returns the milliseconds each kernel took summed over
 * the steps recorded since the last read (*n_steps of them), and restarts
 * the count. Any output pointer may be NULL. */
dkv_status kv_layout_timing_read(dkv_layout *layout, double *ms_projection, double *ms_fresh,
                                 double *ms_split, double *ms_combine, int32_t *n_steps);

/* ---------------------------------------------------------------------------
 * GEMM with an operand in host memory: the experiment behind CPU-aware tiling
 * ("KV Cache 内存层级" overview, opening section, Fig. 2(a): a 10240-square GEMM
 * is 17x slower reading CPU memory directly than with a swap buffer; 2.1 去搬
 * 运：DirectKV: CPU-aware tiling fetches each B tile over the link once and
 * re-reads the HBM operand instead). Measurement only; not on the decode path.
 * ------------------------------------------------------------------------- */

/* Pinned host buffer of `bytes` bytes (hipHostMalloc, mapped, portable;
 * flags as kv_alloc_host: DKV_HOST_COHERENT or DKV_HOST_NONCOHERENT).
 * *host_ptr is the CPU address, *device_ptr the address kernels use. The
 * caller frees it with dkv_host_buffer_free. Errors: DKV_E_INVALID_ARG,
 * DKV_E_OUT_OF_MEMORY. */
dkv_status dkv_host_buffer_alloc(uint64_t bytes, uint32_t flags, void **host_ptr, void **device_ptr);
dkv_status dkv_host_buffer_free(void *host_ptr);

/* Asynchronous copy of `bytes` bytes between any two addresses the HIP
 * runtime knows (pinned host, HBM), on the copy engines, on `stream`: the
 * swap-in of the staging design. Errors: DKV_E_INVALID_ARG, DKV_E_HIP. */
dkv_status dkv_copy(void *dst, const void *src, uint64_t bytes, dkv_stream_t stream);

/* C[M][N] (fp32, device) = A[M][K] (bf16, device) x B[N][K]^T (bf16; HBM or a
 * mapped host buffer), fp32 accumulation on the matrix cores, enqueued on
 * `stream`. tile_order 0 = row-major tile order (naive zero-copy: B column
 * blocks are fetched again for every row block), 1 = CPU-aware order (each
 * XCD owns every 8th column block and runs all row blocks of one column
 * block back to back, so B crosses the link once). Same bits either way.
 * Requires M, N multiples of 128, K a multiple of 64, 16-byte aligned
 * pointers, and for tile_order 1 N / 128 a multiple of 8.
 * Errors: DKV_E_INVALID_ARG (checked before anything is enqueued). */
dkv_status dkv_gemm_bf16_nt(const uint16_t *A, const uint16_t *B, float *C, int32_t M, int32_t N,
                            int32_t K, int32_t tile_order, dkv_stream_t stream);

/* The B-stationary form of the same product ("KV Cache 内存层级" overview,
 * 2.1 去搬运：DirectKV: CPU-aware tiling keeps the remote operand's tile
 * resident so that it crosses the link once, at the price of sending partial
 * results through HBM): each 128 x 512 tile of B is fetched once into one
 * workgroup's LDS and all of A streams past it; the fp32 partial C of each
 * 512-wide k tile goes to `workspace`, and a second kernel adds the k tiles
 * in order into C. Every entry is one fp32 sum per k tile plus the adds of
 * the tiles' sums, so its bits can differ from dkv_gemm_bf16_nt's within the
 * fp32 summation bound (identical when every partial sum is exact).
 * workspace: device memory of at least
 * dkv_gemm_bstationary_workspace_bytes(M, N, K) = (K / 512) * M * N * 4
 * bytes, caller-owned. Requires M a multiple of 64, N of 128, K of 512 and
 * 16-byte aligned pointers. Errors: DKV_E_INVALID_ARG, DKV_E_CAPACITY (too
 * small a workspace); both before anything is enqueued. */
dkv_status dkv_gemm_bf16_nt_bstationary(const uint16_t *A, const uint16_t *B, float *C, int32_t M, int32_t N,
                                        int32_t K, float *workspace, uint64_t workspace_bytes,
                                        dkv_stream_t stream);
uint64_t dkv_gemm_bstationary_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* ---------------------------------------------------------------------------
 * Attention on the host CPU: the comparator for moving decoding attention to
 * where the KV lives instead of moving the KV to the GPU ("KV Cache 内存层级"
 * overview, 2.2 挪计算：NEO: decoding attention is memory-bandwidth-bound on
 * both processors and host DRAM bandwidth is within a small factor of the
 * GPU's). Measurement only; decode_step never calls these.
 * ------------------------------------------------------------------------- */

/* Attention of one decode step of `layer`, computed by n_threads host
 * threads that read the cached K/V in place from the layout's host pages
 * (every page holding tokens [0, ctx_lens[b]) must be a host page), with the
 * fresh token's K/V appended: for each sequence b and query head h (KV head
 * h / G), softmax over ctx_lens[b] + 1 tokens of (q . k) / sqrt(d), applied
 * to the values, fp32 arithmetic.
 *   q            host [B][Hq][d] fp32 (unscaled)
 *   k_new, v_new host [B][Hkv][d] bf16 bits
 *   ctx_lens     host [B], each in [0, capacity - 1]
 *   out          host [B][Hq][d] fp32, written
 * Synchronises the device first (pages written by earlier steps are
 * complete). *threads_used (may be NULL) gets the thread count.
 * Errors: DKV_E_INVALID_ARG (null pointer, bad layer or thread count, an HBM
 * page among the cached tokens), DKV_E_CAPACITY, DKV_E_HIP. */
dkv_status dkv_cpu_attention(const dkv_layout *layout, int32_t layer, const float *q,
                             const uint16_t *k_new, const uint16_t *v_new, const int32_t *ctx_lens,
                             float *out, int32_t n_threads, int32_t *threads_used);

/* The same computation on plain host page pointers, no GPU needed:
 * pages[b * max_pages + p] is the CPU address of page p of sequence b in the
 * page layout above (NULL allowed past the cached tokens), every other
 * argument as in dkv_cpu_attention; `batch` sequences of `shape` (its
 * n_layers is ignored). Errors: DKV_E_INVALID_ARG (null pointer, bad shape,
 * thread count, or a missing page among the cached tokens). */
dkv_status dkv_cpu_attention_pages(const void *const *pages, int32_t max_pages, const dkv_shape *shape,
                                   int32_t batch, const float *q, const uint16_t *k_new,
                                   const uint16_t *v_new, const int32_t *ctx_lens, float *out,
                                   int32_t n_threads, int32_t *threads_used);

/* Reads `bytes` bytes (a multiple of 64) of host memory at `host_ptr` on
 * n_threads host threads as 64-bit words and returns their wrapping sum in
 * *checksum (may be NULL): the host-DRAM streaming-read rate, timed by the
 * caller. Errors: DKV_E_INVALID_ARG. */
dkv_status dkv_cpu_stream_read(const void *host_ptr, uint64_t bytes, int32_t n_threads,
                               uint64_t *checksum);

#ifdef __cplusplus
}
#endif

#endif /* DKV_PROBE_H */
