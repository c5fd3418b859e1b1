/*
 * dkv.h -- C ABI of the zero-copy decode-attention library for MI355X (gfx950).
 *
 * One decode step of one transformer layer: a fused QKV projection of the
 * batch's hidden states, followed by softmax attention of every query head
 * over its sequence's cached K/V plus the freshly projected token. The KV
 * cache lives in pages; each page is either host memory (pinned, mapped into
 * the GPU's address space) or HBM, and the attention kernel reads host pages
 * in place over the host link -- no staging buffer, no copy into HBM.
 *
 * What the method is, from the pages this library follows:
 *  - "长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）" (DirectKV digest,
 *    awesome-system-papers), 核心方法 (core method): the attention kernel
 *    reads CPU pinned/unified memory directly instead of staging KV into HBM;
 *    the KV layout is rearranged for coalesced remote reads; the QKV
 *    projection that generates the new K/V is fused with the attention that
 *    consumes it. 局限与后续工作 (limits and future work): keep hot KV in HBM
 *    and read cold KV directly from CPU memory.
 *  - "KV Cache 内存层级" series overview (10100.com), 2.1 去搬运：DirectKV:
 *    staging costs a reserved GPU buffer, doubled interconnect traffic and
 *    dynamic copy addresses that break graph replay; one launch does the QKV
 *    projection and the attention.
 *
 * Conventions used by every entry point
 *  - All functions return a dkv_status; 0 is success, negative is failure.
 *    A failing call leaves its outputs untouched (unless stated otherwise)
 *    and sets a thread-local message readable with dkv_last_error().
 *  - bf16 values are passed as uint16_t bit patterns (upper half of an
 *    IEEE-754 binary32).
 *  - "device pointer" = memory the GPU can address (HBM from hipMalloc, or
 *    mapped host memory); "host pointer" = ordinary CPU memory.
 *  - dkv_stream_t is a hipStream_t passed as an opaque pointer (NULL = the
 *    null stream). Work is enqueued on it; nothing synchronises unless said.
 *  - Handles are not thread-safe: one thread at a time per handle.
 *  - No C++ exception leaves the library: host memory or threads running
 *    out inside a call is reported as DKV_E_OUT_OF_MEMORY, with nothing
 *    left allocated or taken by the failed call.
 */
#ifndef DKV_H
#define DKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dkv_status {
    DKV_OK = 0,
    DKV_E_INVALID_ARG = -1,   /* null/misaligned pointer, bad shape or range */
    DKV_E_OUT_OF_MEMORY = -2, /* a pool or workspace allocation failed */
    DKV_E_CAPACITY = -3,      /* tokens or pages beyond what was allocated */
    DKV_E_HIP = -4,           /* a HIP runtime call failed (message has it) */
    DKV_E_UNSUPPORTED = -5    /* shape outside the compiled kernel variants */
} dkv_status;

typedef void *dkv_stream_t;

/* Model shape. Supported kernel variants: head_dim 64 or 128; n_q_heads a
 * multiple of n_kv_heads with group size n_q_heads / n_kv_heads in {1, 2, 4,
 * 8}; hidden a multiple of 512; page_tokens == 16 (DKV_PAGE_TOKENS). */
typedef struct dkv_shape {
    int32_t hidden;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t n_layers;
    int32_t page_tokens;
} dkv_shape;

#define DKV_PAGE_TOKENS 16

/* ---------------------------------------------------------------------------
 * KV page layout (one page = DKV_PAGE_TOKENS consecutive tokens of one
 * sequence and one layer, all KV heads):
 *
 *     page[g][c][t][i]   g < n_kv_heads, c = 0 (K) / 1 (V), t < 16, i < head_dim
 *
 * i.e. head-major: each (page, KV head) is one contiguous run of
 * 2 * 16 * head_dim * 2 bytes (8 KiB at head_dim 128), K rows then V rows.
 * Page bytes = n_kv_heads * 2 * 16 * head_dim * 2; pools are 4 KiB-aligned,
 * so every run starts on a 128-byte boundary. Following the core-method
 * section of the DirectKV digest (layout rearranged for coalesced remote
 * access) and the Beluga note on the "KV Offload" wiki (CXL section: a
 * 16-token GQA block splits into 128 fragments unless head-contiguous).
 * ------------------------------------------------------------------------- */

/* Byte size of one page for `shape`; 0 on an invalid shape. */
int64_t kv_page_bytes(const dkv_shape *shape);

/* Byte offset, inside a page, of element (t, g, c, i) as above; -1 when any
 * index is out of range. Pure host function (no GPU needed). */
int64_t kv_page_offset(const dkv_shape *shape, int32_t token_in_page,
                       int32_t kv_head, int32_t kv_select, int32_t dim);

/* Placement policy (DirectKV digest, 局限与后续工作: hot KV in HBM, cold KV
 * read in place from host memory). A sequence with room for
 * `capacity_tokens` slots has n_pages = ceil(capacity_tokens / 16) pages;
 * the last ceil(hbm_tail_tokens / 16) of them (at most n_pages) are HBM,
 * the rest host. Pure host function. Outputs: *n_pages, *first_hbm_page
 * (== *n_pages when no page is in HBM). */
dkv_status kv_placement(int32_t capacity_tokens, int32_t hbm_tail_tokens,
                        int32_t *n_pages, int32_t *first_hbm_page);

/* ---------------------------------------------------------------------------
 * Pools
 * ------------------------------------------------------------------------- */
typedef struct dkv_pool dkv_pool;

#define DKV_HOST_COHERENT 0u     /* default: fine-grained, uncached on the GPU */
#define DKV_HOST_NONCOHERENT 1u  /* coarse-grained, may be cached in GPU L2 */

/* Host-pinned page pool of n_pages pages of kv_page_bytes(shape), allocated
 * with hipHostMalloc (mapped, portable) on the current device's host NUMA
 * node; the GPU reads it in place (DirectKV digest, 核心方法: the attention
 * kernel reads KV in CPU pinned/unified memory directly, with no staging
 * buffer in HBM). The pool owns the memory until kv_pool_free. Errors:
 * DKV_E_INVALID_ARG (null/shape/n_pages <= 0), DKV_E_OUT_OF_MEMORY (pinning
 * failed, or n_pages pages would exceed 2^50 bytes). */
dkv_status kv_alloc_host(const dkv_shape *shape, int64_t n_pages, uint32_t flags,
                         dkv_pool **out);

/* HBM page pool (hipMalloc) of n_pages pages, for the hot part of the KV
 * (DirectKV digest, 局限与后续工作: hot KV stays in HBM, cold KV is read
 * directly from CPU memory). Same ownership and errors as kv_alloc_host. */
dkv_status kv_alloc_hbm(const dkv_shape *shape, int64_t n_pages, dkv_pool **out);

/* Pages of the pool not yet handed to a layout. */
dkv_status kv_pool_free_pages(const dkv_pool *pool, int64_t *n_free);

/* Frees the pool's memory. The caller must first free every layout that
 * borrows pages from it (DKV_E_INVALID_ARG otherwise, and nothing is freed).
 * NULL is accepted and ignored; a pool freed already (or never returned by
 * kv_alloc_*) gives DKV_E_INVALID_ARG, as does any call that is handed one. */
dkv_status kv_pool_free(dkv_pool *pool);

/* ---------------------------------------------------------------------------
 * Layouts: page tables + placement + workspace for one batch
 * ------------------------------------------------------------------------- */
typedef struct dkv_layout dkv_layout;

/* Creates the KV layout of a batch of `batch` sequences for all
 * shape->n_layers layers: fixed page tables and scratch, set up once, so that
 * every decode step runs on stable addresses ("KV Cache 内存层级" overview,
 * 2.1 去搬运：DirectKV: staging's per-step copy addresses break graph
 * replay; DirectKV digest, 核心方法: a KV layout arranged for the remote
 * reads). Sequence b gets room for capacity_tokens[b] slots
 * (cached tokens plus the token the next decode_step writes) in every layer;
 * its pages are placed by kv_placement(capacity_tokens[b],
 * hbm_tail_tokens[b]) and taken from host_pool / hbm_pool (hbm_pool may be
 * NULL when no page goes to HBM; hbm_tail_tokens may be NULL for "none").
 * Allocates, once: the device page tables [n_layers][batch][max_pages] of
 * 64-bit device addresses, and every scratch buffer decode_step needs, so
 * that decode_step itself allocates and copies nothing.
 * capacity_tokens and hbm_tail_tokens are host arrays of length `batch`.
 * The layout borrows its pools: they must outlive it.
 * Errors: DKV_E_INVALID_ARG, DKV_E_CAPACITY (a pool has too few free
 * pages), DKV_E_OUT_OF_MEMORY, DKV_E_HIP. */
dkv_status kv_layout_create(const dkv_shape *shape, int32_t batch,
                            const int32_t *capacity_tokens,
                            const int32_t *hbm_tail_tokens,
                            dkv_pool *host_pool, dkv_pool *hbm_pool,
                            dkv_layout **out);

/* A layout whose HBM part is a sliding hot window instead of a fixed tail
 * (DirectKV digest, 局限与后续工作: hot KV in HBM, cold KV read in place from
 * host memory). Sequence b gets room for capacity_tokens[b] slots in every
 * layer, a host page for every one of its ceil(capacity / 16) pages, and
 * W_b = min(pages, ceil(window_tokens[b] / 16)) HBM pages. The W_b pages up
 * to and including the one holding slot ctx_lens[b] (the slot the next
 * decode_step writes) are HBM-resident; page p always uses HBM page p % W_b
 * of the sequence's window. kv_advance slides the window as the sequence
 * grows. Host arrays of length `batch`: capacity_tokens (> 0), window_tokens
 * (> 0), ctx_lens (in [0, capacity)). Both pools are required. Allocation,
 * ownership and errors as kv_layout_create. */
dkv_status kv_layout_create_windowed(const dkv_shape *shape, int32_t batch,
                                     const int32_t *capacity_tokens,
                                     const int32_t *window_tokens,
                                     const int32_t *ctx_lens,
                                     dkv_pool *host_pool, dkv_pool *hbm_pool,
                                     dkv_layout **out);

/* Returns the layout's pages to their pools and frees its device memory.
 * Synchronises the device first. NULL is accepted and ignored; a layout freed
 * already (or never returned by kv_layout_create*) gives DKV_E_INVALID_ARG,
 * as does any call that is handed one. */
dkv_status kv_layout_free(dkv_layout *layout);

/* Tier of page `page` of sequence `seq` (same in every layer) as the page
 * table holds it now (synchronises the device first): 0 = host, 1 = HBM.
 * Errors: DKV_E_INVALID_ARG for out-of-range indices. */
dkv_status kv_layout_page_tier(const dkv_layout *layout, int32_t seq, int32_t page,
                               int32_t *tier);

/* Stores n_tokens tokens of one sequence and layer at slots
 * [start_token, start_token + n_tokens), rearranged from logical order into
 * the page layout: the write of history KV into its tier (KV Offload wiki,
 * 为什么需要 Offload and Offload 的基本机制: a long context's KV moves out of
 * HBM into host DRAM), here straight into the pages the attention reads.
 * k and v point to [n_tokens][n_kv_heads][head_dim] bf16 in logical order,
 * both HOST memory (ordinary or pinned) or both DEVICE memory (hipMalloc or
 * managed; then 16-byte aligned):
 *  - host buffers: host pages are written by the CPU directly, HBM pages
 *    through a synchronous copy on `stream`;
 *  - device buffers: one kernel on `stream` scatters the rows into their
 *    pages, host or HBM, after the work already on `stream`.
 * Returns when the tokens are in place (it synchronises `stream`). This is
 * the set-up path (prefill / tests), not part of a decode step. The buffers
 * stay the caller's. Errors: DKV_E_INVALID_ARG (null, misaligned device
 * buffers, or one host and one device buffer), DKV_E_CAPACITY (slots beyond
 * capacity), DKV_E_HIP. */
dkv_status kv_append(dkv_layout *layout, int32_t layer, int32_t seq,
                     int32_t start_token, int32_t n_tokens,
                     const uint16_t *k, const uint16_t *v, dkv_stream_t stream);

/* Reads slots [start_token, start_token + n_tokens) back into HOST buffers
 * k_out / v_out ([n_tokens][n_kv_heads][head_dim] bf16). Synchronises the
 * device first, so a decode_step's write-back is visible. Test/debug path. */
dkv_status kv_read(const dkv_layout *layout, int32_t layer, int32_t seq,
                   int32_t start_token, int32_t n_tokens,
                   uint16_t *k_out, uint16_t *v_out);

/* ---------------------------------------------------------------------------
 * The decode step (DirectKV digest, 核心方法; KV-hierarchy overview, 2.1)
 * ------------------------------------------------------------------------- */

/* One decode step of layer `layer` for every sequence of the layout:
 *   y_b     = W_qkv . q_in[b]          fp32 accumulation of bf16 products
 *   q       = y_b[0 : Hq*d]            kept in fp32
 *   k_new,
 *   v_new   = y_b[Hq*d : (Hq+Hkv)*d], y_b[(Hq+Hkv)*d : (Hq+2Hkv)*d],
 *             rounded once to bf16 (nearest even) and written once into
 *             slot ctx_lens[b] of the sequence's pages (host or HBM)
 *   attn_out[b][h*d : (h+1)*d] = softmax((q_h . K_j) / sqrt(d)) . V_j over
 *             the ctx_lens[b] cached tokens and the fresh one, with
 *             KV head g = h / (Hq/Hkv); fp32 softmax state and sums, rounded
 *             to bf16 (nearest even). From groups of 4 query heads the
 *             group's score and output products run on the matrix cores,
 *             which take q and the probabilities as two bf16 terms each
 *             (x ~ bf16(x) + bf16(x - bf16(x)), ~2^-17 relative).
 * Arguments (all device pointers, caller-owned, never retained):
 *   q_in     [batch][hidden] bf16 hidden states of this layer (16-byte aligned)
 *   W_qkv    [(Hq + 2 Hkv) * d][hidden] bf16, row-major, rows ordered
 *            [Q heads | K heads | V heads], each head's d rows contiguous
 *            (16-byte aligned)
 *   ctx_lens [batch] int32: cached tokens per sequence before this step
 *            (0 allowed; 4-byte aligned). Not modified; the caller advances it.
 *   attn_out [batch][Hq * d] bf16 (2-byte aligned)
 * The call enqueues kernels on `stream` and returns; it allocates nothing,
 * copies nothing and does not synchronise, so it can be captured in a HIP
 * graph (the stable-address property the KV-hierarchy overview, 2.1, says
 * staging loses). Host-side checks (null/misaligned pointers, layer range)
 * fail with DKV_E_INVALID_ARG before anything is enqueued. ctx_lens lives
 * on the device, so its range is checked by the kernels: a sequence with
 * ctx_lens[b] < 0 or ctx_lens[b] >= its capacity writes nothing to the
 * cache, gets attn_out rows of NaN, and raises the flag that
 * kv_layout_check_status reports. A layout's steps share its scratch (the
 * projection's output, the split partials, the step's list of work items
 * and the work queue of the looping split kernel), so steps of one layout
 * must be ordered (one stream, or events between streams); steps of
 * different layouts may overlap. */
dkv_status decode_step(dkv_layout *kv_layout, int32_t layer,
                       const uint16_t *q_in, const uint16_t *W_qkv,
                       const int32_t *ctx_lens, uint16_t *attn_out,
                       dkv_stream_t stream);

/* Same step with fp32 attn_out [batch][Hq * d] (no output rounding). For
 * tests that need a gate tighter than bf16 output rounding allows. */
dkv_status decode_step_f32(dkv_layout *kv_layout, int32_t layer,
                           const uint16_t *q_in, const uint16_t *W_qkv,
                           const int32_t *ctx_lens, float *attn_out,
                           dkv_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * step as decode_step, with the same arguments, errors and results (identical
 * bits), whose scratch (projection sums, queries, split partials, work-item
 * list, work-queue counter) is a file-scope device array of
 * decode_step_noalloc_scratch_bytes()
 * bytes (32 MiB) instead of the layout's. The call allocates nothing; its
 * first call on a device looks the array's address up once. A layout whose
 * step needs more scratch than the array holds gets DKV_E_CAPACITY and
 * nothing is enqueued. Every value of the array that a step uses is written
 * earlier in the same step (the work-item list and the zeroed work-queue
 * counter by the step's fresh-token kernel), so no clearing is needed
 * between calls. All calls on one GPU
 * share its one array: calls that overlap on a GPU (different streams without
 * ordering, other threads) race and give undefined results; order them. */
dkv_status decode_step_noalloc(dkv_layout *kv_layout, int32_t layer,
                               const uint16_t *q_in, const uint16_t *W_qkv,
                               const int32_t *ctx_lens, uint16_t *attn_out,
                               dkv_stream_t stream);

/* Size in bytes of decode_step_noalloc's static scratch array. */
size_t decode_step_noalloc_scratch_bytes(void);

/* Advances every sequence by one decoded token, on the device: for each b
 * with ctx_lens[b] + 1 < capacity, ctx_lens[b] += 1 (in place; ctx_lens is
 * the device array decode_step reads). In a windowed layout, when the new
 * value starts a page (a multiple of 16), that page takes the HBM page of
 * the window's oldest page, whose contents are first copied to its own host
 * page (every layer), and the page table is repointed; the slots from the
 * new ctx_lens[b] on are assumed to hold nothing yet. A sequence that has no
 * room for another slot is left as it is and raises the flag that
 * kv_layout_check_status reports. Enqueued on `stream` after the step that
 * wrote slot ctx_lens[b]; it allocates nothing, copies nothing from the host
 * and does not synchronise, so a decode step and kv_advance can be captured
 * together in one HIP graph and replayed step after step. Host-side checks:
 * DKV_E_INVALID_ARG for a null or misaligned pointer. */
dkv_status kv_advance(dkv_layout *kv_layout, int32_t *ctx_lens, dkv_stream_t stream);

/* Synchronises the device and reports (then clears) the in-kernel range
 * flag: DKV_OK, or DKV_E_CAPACITY if some decode_step since the last check
 * saw a ctx_lens entry outside [0, capacity - 1]. */
dkv_status kv_layout_check_status(dkv_layout *kv_layout);

/* Split size (tokens per attention work item) the layout uses; a multiple
 * of 16 fixed at creation, independent of placement. */
int32_t kv_layout_split_tokens(const dkv_layout *kv_layout);

/* Split-attention kernel the layout's decode steps use. All but the naive
 * comparator read each page run once per step for the whole group of query
 * heads:
 *   0 = one wavefront per work item with a register double buffer, VALU
 *       arithmetic (the default below groups of 4 query heads);
 *   1 = a producer wavefront that streams page runs with LDS DMA into a ring
 *       for consumer wavefronts that own the group's query heads (same
 *       arithmetic as 0; identical bits up to groups of 4);
 *   3 = the register double buffer with the group's scores and output update
 *       on the matrix cores (the default from groups of 4; queries and
 *       probabilities enter as two bf16 terms each, see the kernel source);
 *   2 = the naive zero-copy comparator (one wavefront per query head, so
 *       each KV head's pages are read once per query head of its group), for
 *       measurement only, with the arithmetic of the group's default kernel
 *       and so the same bits as it;
 *   4 = a producer wavefront streaming page runs with LDS DMA into a ring for
 *       a consumer wavefront with the arithmetic of 3 (same bits as 3; groups
 *       of 4 and 8, head_dim 128).
 * Chosen at creation (producer/consumer DirectKV digest, 核心方法; the
 * "KV Cache 内存层级" overview, 2.1); the environment variable
 * DKV_SPLIT_KERNEL=regs|lds|naive|mfma|ldsmfma, read by kv_layout_create,
 * selects one (mfma from groups of 4, ldsmfma from groups of 4 at head_dim
 * 128). -1 for a NULL layout. */
int32_t kv_layout_split_kernel(const dkv_layout *kv_layout);

/* Wavefronts the register split kernel runs on: 0 = one per work item
 * (sequence, KV head, token split); n > 0 = n wavefronts, each looping over
 * every n-th item. Layouts whose host pages dominate the step default to
 * 256, which keeps the host link's request queue short (more outstanding
 * reads lower its bandwidth); layouts that are all or nearly all HBM (below
 * ~4 % host pages) default to 0, since HBM needs far more reads in flight.
 * The environment variable
 * DKV_SPLIT_WAVES=<n>, read by kv_layout_create, overrides it. Same bits
 * either way. -1 for a NULL layout. */
int32_t kv_layout_split_waves(const dkv_layout *kv_layout);

/* Switches the layout's split-attention kernel (0 to 4 as above) for the
 * decode steps enqueued after the call. Errors: DKV_E_INVALID_ARG for a NULL
 * layout, an unknown kernel, or 3 / 4 on a shape they do not serve. */
dkv_status kv_layout_set_split_kernel(dkv_layout *kv_layout, int32_t kernel);

/* Thread-local message of the last failing call on this thread. */
const char *dkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DKV_H */
