// Host runtime and C ABI of the zero-copy decode-attention library:
// KV page pools (host-pinned or HBM), per-batch layouts (page tables,
// placement, scratch), set-up copies, validation and the decode-step launch.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <thread>
#include <unordered_set>
#include <vector>

#include "cpu_attention.h"
#include "dkv_internal.h"
#include "dkv_probe.h"

namespace {

thread_local std::string g_last_error;

// Handles (pools and layouts) that are alive. The free calls and the calls
// that use a handle check it here, so a double free or a call on a freed
// handle fails with DKV_E_INVALID_ARG instead of touching freed memory
// (unless a newer handle has taken the same address).
std::mutex g_handles_mu;
std::unordered_set<const void *> g_handles;

void track(const void *h) {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    g_handles.insert(h);
}

bool untrack(const void *h) {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    return g_handles.erase(h) == 1;
}

bool live(const void *h) {
    std::lock_guard<std::mutex> lock(g_handles_mu);
    return g_handles.count(h) == 1;
}

// Records the message of a failing call; never throws (a message that
// cannot be stored is dropped), so it is safe on every error path.
dkv_status fail(dkv_status st, const char *fmt, ...) noexcept {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    try {
        g_last_error = buf;
    } catch (...) {
        g_last_error.clear();
    }
    return st;
}

dkv_status hip_fail(hipError_t e, const char *what) {
    return fail(DKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Entry points that allocate host memory or start threads run their body
// through this: a std::bad_alloc (or any other exception of the C++ runtime,
// such as thread creation failing) becomes DKV_E_OUT_OF_MEMORY with a
// message, so nothing unwinds across the C ABI.
template <class F>
dkv_status guarded(const char *who, F &&body) {
    try {
        return body();
    } catch (const std::bad_alloc &) {
        return fail(DKV_E_OUT_OF_MEMORY, "%s: host memory exhausted", who);
    } catch (const std::exception &ex) {
        return fail(DKV_E_OUT_OF_MEMORY, "%s: host resources exhausted (%s)", who, ex.what());
    }
}

// HIP events a timed decode step records: before the projection, after it,
// after the fresh-token kernel, after the split attention, after the combine.
constexpr int kTimingEvents = 5;

// Largest pool, in bytes, a request may ask for (1 PiB): keeps page counts
// times page bytes far from overflow.
constexpr uint64_t kMaxPoolBytes = 1ull << 50;

#define HIP_TRY(call)                                        \
    do {                                                     \
        hipError_t e_ = (call);                              \
        if (e_ != hipSuccess) return hip_fail(e_, #call);    \
    } while (0)

bool shape_ok(const dkv_shape *s) {
    if (!s) return false;
    if (s->hidden <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 ||
        s->n_layers <= 0)
        return false;
    if (s->page_tokens != DKV_PAGE_TOKENS) return false;
    if (s->n_q_heads % s->n_kv_heads != 0) return false;
    return true;
}

bool shape_supported(const dkv_shape *s) {
    const int G = s->n_q_heads / s->n_kv_heads;
    return (s->head_dim == 64 || s->head_dim == 128) && (G == 1 || G == 2 || G == 4 || G == 8) &&
           s->hidden % 512 == 0;
}

int64_t page_bytes_of(const dkv_shape *s) {
    return (int64_t)s->n_kv_heads * 2 * DKV_PAGE_TOKENS * s->head_dim * 2;
}

int64_t row_offset(const dkv_shape *s, int t, int g, int c) {
    return ((int64_t)(g * 2 + c) * DKV_PAGE_TOKENS + t) * s->head_dim * 2;
}

}  // namespace

struct dkv_pool {
    dkv_shape shape;
    int32_t tier;            // 0 host, 1 HBM
    int64_t n_pages;
    int64_t page_bytes;
    char *host_base;         // CPU address (host tier), else nullptr
    char *dev_base;          // GPU address of page 0
    std::vector<uint8_t> used;
    int64_t n_free;
    int64_t scan;            // allocation cursor
    int64_t n_layouts;       // layouts holding pages of this pool
};

struct dkv_layout {
    dkv_shape shape;
    int32_t batch;
    std::vector<int32_t> capacity;
    std::vector<int32_t> n_pages;
    std::vector<int32_t> first_hbm;    // static placement: pages [first_hbm, n_pages) are HBM
    int32_t max_pages;
    int32_t split_tokens;
    int32_t max_splits;
    int32_t item_slots;                // sum over sequences of ceil((capacity - 1) / split_tokens), >= 1
    int32_t split_variant;             // dkv::kSplitRegisters, kSplitLds, kSplitNaive or kSplitMfma
    int32_t split_waves;               // > 0: the register kernel runs on that many looping wavefronts
    int32_t proj_mfma_min_batch;       // batches from this size on project on the matrix cores
    int32_t proj_splitk_min_batch;     // MFMA batches from this size on use the split-k projection
    int32_t proj_ranges;               // split-k ranges (0: chosen from the shape)
    int32_t lds_ring;                  // LDS producer/consumer kernel: ring slots
    int32_t lds_poison;                // LDS producer/consumer kernel: NaN-fill freed slots
    dkv_pool *host_pool;
    dkv_pool *hbm_pool;
    std::vector<std::pair<dkv_pool *, int64_t>> owned;   // every page the layout holds
    uint64_t *d_page_table;            // [n_layers][batch][max_pages] current device address of each page
    int32_t *d_capacity;
    char *d_scratch = nullptr;         // one allocation carved by dkv::carve_scratch (projection slabs,
                                       // queries, split partials, work-queue counter)
    dkv::ScratchPlan scratch{};
    uint32_t *d_status;
    // sliding hot window (kv_layout_create_windowed); windowed == 0 otherwise
    int32_t windowed = 0;
    std::vector<int32_t> window;       // HBM window pages per sequence
    int32_t max_window = 0;
    uint64_t *d_host_pages = nullptr;  // [n_layers][batch][max_pages] host page of every page
    uint64_t *d_ring = nullptr;        // [n_layers][batch][max_window] HBM pages of the window
    int32_t *d_window = nullptr;       // [batch] window pages per sequence
    // per-kernel timing (measurement mode only)
    std::vector<hipEvent_t> timing_events;   // kTimingEvents per recorded step
    int32_t timing_recorded = 0;
    int32_t timing_mode = 0;                 // 0 off, 1 every kernel, 2 the split kernel only
};

namespace {

size_t pt_index(const dkv_layout *L, int layer, int b, int p) {
    return ((size_t)layer * L->batch + b) * L->max_pages + p;
}

bool take_pages(dkv_pool *pool, int64_t n, std::vector<int64_t> &out) {
    if (pool->n_free < n) return false;
    out.clear();
    out.reserve(n);
    int64_t i = pool->scan;
    for (int64_t cnt = 0; cnt < pool->n_pages && (int64_t)out.size() < n; ++cnt) {
        if (!pool->used[i]) out.push_back(i);
        i = (i + 1) % pool->n_pages;
    }
    if ((int64_t)out.size() < n) return false;
    for (int64_t idx : out) pool->used[idx] = 1;
    pool->n_free -= n;
    pool->scan = i;
    return true;
}

void give_back(dkv_pool *pool, int64_t idx) {
    if (pool && idx >= 0 && pool->used[idx]) {
        pool->used[idx] = 0;
        ++pool->n_free;
    }
}

uint64_t page_addr(const dkv_pool *pool, int64_t idx) {
    return (uint64_t)(uintptr_t)(pool->dev_base + idx * pool->page_bytes);
}

void free_device(dkv_layout *L) {
    for (void *p : {(void *)L->d_page_table, (void *)L->d_capacity, (void *)L->d_scratch, (void *)L->d_status,
                    (void *)L->d_host_pages, (void *)L->d_ring, (void *)L->d_window})
        if (p) (void)hipFree(p);
}

void release_pages(dkv_layout *L) {
    for (auto &pi : L->owned) give_back(pi.first, pi.second);
    L->owned.clear();
}

// Current device addresses of pages [p_first, p_last] of (layer, seq), read
// from the device page table (the authority: kv_advance moves pages there).
hipError_t table_row(const dkv_layout *L, int layer, int b, int p_first, int p_last, std::vector<uint64_t> &row) {
    row.resize((size_t)(p_last - p_first + 1));
    return hipMemcpy(row.data(), L->d_page_table + pt_index(L, layer, b, p_first), row.size() * sizeof(uint64_t),
                     hipMemcpyDeviceToHost);
}

// CPU address of a page that lives in the host pool, nullptr for an HBM page.
char *host_view(const dkv_layout *L, uint64_t addr) {
    const dkv_pool *hp = L->host_pool;
    if (!hp) return nullptr;
    const uint64_t base = (uint64_t)(uintptr_t)hp->dev_base;
    if (addr < base || addr >= base + (uint64_t)(hp->n_pages * hp->page_bytes)) return nullptr;
    return hp->host_base + (addr - base);
}

// The split size T: the longest power of two of at most 8192 tokens whose
// work items both
//  * spread over the chip: at least 1536 full items (batch x KV heads x
//    floor(longest cached context / T)); a short tail split, such as decode
//    headroom past the cached tokens, is not counted), and
//  * fit one round of the 3072 wavefronts the matrix-core split kernel keeps
//    resident (3 per SIMD): at most 3072 items in all, tails included (KV
//    heads x the sum over sequences of ceil((capacity - 1) / T)).
// Without such a T: the smallest T whose items still fit one round (the most
// parallel single round), or 8192 when even that takes two rounds (the
// fewest rounds). A second round leaves waves idling at its end: 32
// sequences of 57344 tokens, all in HBM: 1792 items of 8192 tokens 1.09 ms
// (6.9 TB/s), 3584 items of 4096 tokens 1.28 ms. A longer split is a longer
// contiguous page stream per wavefront, fewer partials to write and
// combine, and fewer waves starting up; with every page in HBM on MI355X
// (one wave per item): 1 GiB at batch 8 (2048 items at 1024 tokens),
// 1024 / 2048 / 4096 tokens: 0.169 / 0.198 / 0.297 ms (too few items);
// an 8 GiB layer at batch 16, 131072 tokens, group 8: 1024 / 2048 / 8192
// tokens: 1.415 / 1.348 / 1.252 ms (6.07 -> 6.86 TB/s), group 4: 1.40 /
// 1.35 / 1.25-1.31 ms. The choice depends on the shape and capacities
// only, never on placement.
int32_t choose_split_tokens(int32_t batch, int32_t n_kv_heads, const int32_t *capacity) {
    if (const char *env = getenv("DKV_SPLIT_TOKENS")) {
        const int v = atoi(env);
        if (v >= DKV_PAGE_TOKENS && v % DKV_PAGE_TOKENS == 0) return v;
    }
    constexpr int64_t kMinFullItems = 1536, kResidentWaves = 3072;
    int32_t max_cap = 1;
    for (int b = 0; b < batch; ++b) max_cap = std::max(max_cap, capacity[b]);
    const int64_t max_cached = std::max(1, max_cap - 1);
    auto items = [&](int64_t t) {
        int64_t n = 0;
        for (int b = 0; b < batch; ++b) n += (capacity[b] - 1 + t - 1) / t;
        return n * n_kv_heads;
    };
    int32_t one_round = 0;       // the smallest T whose items fit one round
    for (int32_t t = 8192; t >= DKV_PAGE_TOKENS; t /= 2) {
        const int64_t n = items(t);
        if (n > kResidentWaves) break;          // smaller T only add items
        if ((int64_t)batch * n_kv_heads * (max_cached / t) >= kMinFullItems) return t;
        one_round = t;
    }
    return one_round ? one_round : 8192;
}

// Split-attention kernel variant. Every default streams pages through a
// register double buffer, which measured faster on MI355X than the LDS
// producer/consumer ring in the all-HBM placement (1 GiB of KV at group 4:
// 189 us vs 258 us; group 8: 18.8 ms vs 27.6 ms for 64 GiB) and the same on
// the host link. From groups of 4 the group's products run on the matrix
// cores (all-HBM, 1 GiB at group 4: 161 us vs 174 us on VALU; 8 GiB layers
// at group 8: 1.41 ms vs 2.0 ms); smaller groups keep the VALU form. The LDS
// ring with a matrix-core consumer ties with the register kernel at best
// (all-HBM: 4 GiB at group 4, 0.617 vs 0.619 ms; 1 GiB, 0.168 vs 0.163 ms;
// 9.1 GB of ragged contexts, 1.62 vs 1.33 ms). DKV_SPLIT_KERNEL=regs|lds|
// mfma|ldsmfma overrides it; DKV_SPLIT_KERNEL=naive selects the naive
// zero-copy comparator (one work item per query head).
bool lds_mfma_supported(int32_t group, int32_t head_dim) {
    return group >= dkv::kMfmaMinGroup && head_dim == 128;
}

int32_t choose_split_variant(int32_t group, int32_t head_dim) {
    if (const char *env = getenv("DKV_SPLIT_KERNEL")) {
        if (!strcmp(env, "lds")) return dkv::kSplitLds;
        if (!strcmp(env, "regs")) return dkv::kSplitRegisters;
        if (!strcmp(env, "naive")) return dkv::kSplitNaive;
        if (!strcmp(env, "mfma") && group >= dkv::kMfmaMinGroup) return dkv::kSplitMfma;
        if (!strcmp(env, "ldsmfma") && lds_mfma_supported(group, head_dim)) return dkv::kSplitLdsMfma;
    }
    return group >= dkv::kMfmaMinGroup ? dkv::kSplitMfma : dkv::kSplitRegisters;
}

// Wavefronts of the split kernel. On the host link the number of reads in
// flight matters beyond Little's law: 256 looping wavefronts keep it at its
// ceiling, one wavefront per item (thousands) loses ~2.5 %. HBM needs many
// more reads in flight (~16 MiB), so 256 waves starve it. Measured on MI355X
// (1 GiB at batch 8): host-resident 19.13 ms with one wave per item vs 18.69
// ms with 128-384 waves (18.74 ms with 512, 19.1 ms from 768 up); HBM-resident
// 0.18 ms per item vs ~0.8 ms on 256 waves (~1.34 TB/s). The layout takes
// whichever launch its page counts predict to be faster:
//   looping:  max(host / 57.5 GB/s, HBM / 1.34 TB/s)
//   per item: max(host / 56.1 GB/s, HBM / 6.0 TB/s)
// so a layout keeps one wavefront per item below ~4 % host bytes.
// DKV_SPLIT_WAVES=<n> overrides (0: one wavefront per item).
constexpr int32_t kHostSplitWaves = 256;

int32_t choose_split_waves(int64_t host_pages, int64_t hbm_pages) {
    if (const char *env = getenv("DKV_SPLIT_WAVES")) {
        const int v = atoi(env);
        if (v >= 0) return v;
    }
    if (host_pages == 0) return 0;
    const double h = (double)host_pages, m = (double)hbm_pages;   // page bytes cancel out
    const double t_looping = std::max(h / 57.5, m / 1340.0);
    const double t_per_item = std::max(h / 56.1, m / 6000.0);
    return t_looping < t_per_item ? kHostSplitWaves : 0;
}

// Batch size from which the QKV projection runs on the matrix cores (the
// split-k kernel), below which it takes the VALU GEMV: from 8 sequences,
// where x fills half of every 16-column MFMA tile or more, the projection is
// a real dense contraction. Below that the tiles would be mostly padding,
// although the matrix cores would still save a little time: measured on
// MI355X (W cycled through copies so that every step reads it from HBM,
// decode-step HIP events, hidden 4096 / 8192, GEMV vs split-k MFMA), batch
// 1, 13.33 / 33.5 vs 13.31 / 35.3 us; batch 2, 14.07 / 35.5 vs 13.48 / 35.6;
// batch 3, 14.85 / 37.0 vs 13.54 / 35.2; batch 4, 15.5 / 38.6 vs 13.38 /
// 35.6; at batch 8, 21.2 vs 13.6 us at hidden 4096. DKV_PROJ_MFMA_MIN_BATCH=<n>
// overrides it.
constexpr int32_t kProjMfmaMinBatch = 8;

// The split-k projection's batch threshold and range count; the defaults
// are measured choices (proj.hip), the environment variables
// DKV_PROJ_SPLITK_MIN_BATCH=<n> and DKV_PROJ_RANGES=1|2|4|8 override them.
int32_t choose_proj_splitk_min_batch() {
    if (const char *env = getenv("DKV_PROJ_SPLITK_MIN_BATCH")) {
        const int v = atoi(env);
        if (v >= 1) return v;
    }
    return dkv::kProjSplitkMinBatch;
}

int32_t choose_proj_ranges() {
    if (const char *env = getenv("DKV_PROJ_RANGES")) {
        const int v = atoi(env);
        if (v == 1 || v == 2 || v == 4 || v == 8) return v;
    }
    return 0;
}

int32_t choose_proj_mfma_min_batch() {
    if (const char *env = getenv("DKV_PROJ_MFMA_MIN_BATCH")) {
        const int v = atoi(env);
        if (v >= 1) return v;
    }
    return kProjMfmaMinBatch;
}

// Parallel copy helper for host pages: runs f(first, last) over [0, n) in
// contiguous chunks on up to 16 threads.
template <class F>
void parallel_for(int64_t n, F f) {
    const int64_t nthreads = std::min<int64_t>(16, std::max<int64_t>(1, n / 64));
    if (nthreads <= 1) {
        f(0, n);
        return;
    }
    std::vector<std::thread> ts;
    const int64_t chunk = (n + nthreads - 1) / nthreads;
    for (int64_t i = 0; i < nthreads; ++i) {
        const int64_t a = i * chunk, e = std::min(n, a + chunk);
        if (a < e) ts.emplace_back([=] { f(a, e); });
    }
    for (auto &t : ts) t.join();
}

// Pool bookkeeping (the struct, its page map and its registry entry) comes
// first, so that nothing is left to undo if one of them throws.
std::unique_ptr<dkv_pool> new_pool(const dkv_shape *shape, int64_t n_pages, int32_t tier) {
    std::unique_ptr<dkv_pool> p(new dkv_pool());
    p->shape = *shape;
    p->tier = tier;
    p->n_pages = n_pages;
    p->page_bytes = page_bytes_of(shape);
    p->host_base = nullptr;
    p->dev_base = nullptr;
    p->used.assign((size_t)n_pages, 0);
    p->n_free = n_pages;
    p->scan = 0;
    p->n_layouts = 0;
    return p;
}

bool pool_too_large(const dkv_shape *shape, int64_t n_pages) {
    return (uint64_t)n_pages > kMaxPoolBytes / (uint64_t)page_bytes_of(shape);
}

}  // namespace

namespace dkv {

namespace {
size_t align256(size_t n) { return (n + 255) & ~size_t(255); }
}  // namespace

ScratchPlan scratch_plan(int batch, int n_q_heads, int n_kv_heads, int head_dim, int part_slots) {
    ScratchPlan p{};
    const size_t B = (size_t)batch, Hq = (size_t)n_q_heads, D = (size_t)head_dim;
    const size_t n_qkv = (Hq + 2 * (size_t)n_kv_heads) * D;
    p.proj_part = align256((size_t)kProjMaxSplits * B * n_qkv * sizeof(float));
    p.q = align256(B * Hq * D * sizeof(float));
    p.part_o = align256(B * Hq * (size_t)part_slots * D * sizeof(float));
    p.part_ml = align256(B * Hq * (size_t)part_slots * sizeof(float2));
    p.item_counter = 256;
    p.item_list = align256((1 + B * (size_t)(part_slots - 1)) * sizeof(uint32_t));
    p.total = p.proj_part + p.q + p.part_o + p.part_ml + p.item_counter + p.item_list;
    return p;
}

void carve_scratch(StepArgs &a, char *base, const ScratchPlan &p) {
    char *c = base;
    a.proj_part = reinterpret_cast<float *>(c);
    c += p.proj_part;
    a.q = reinterpret_cast<float *>(c);
    c += p.q;
    a.part_o = reinterpret_cast<float *>(c);
    c += p.part_o;
    a.part_ml = reinterpret_cast<float2 *>(c);
    c += p.part_ml;
    a.item_counter = reinterpret_cast<uint32_t *>(c);
    c += p.item_counter;
    a.item_list = reinterpret_cast<uint32_t *>(c);
}

hipError_t launch_decode_step(const StepArgs &a, hipStream_t st, hipEvent_t *ev, bool split_only) {
    const int G = a.n_q_heads / a.n_kv_heads;
    if (!((a.head_dim == 128 || a.head_dim == 64) && (G == 1 || G == 2 || G == 4 || G == 8)))
        return hipErrorInvalidValue;
    hipError_t e;
    int ranges = 1;
    hipEvent_t *every = split_only ? nullptr : ev;
    if (every) (void)hipEventRecord(every[0], st);
    if ((e = launch_projection(a, &ranges, st)) != hipSuccess) return e;
    if (every) (void)hipEventRecord(every[1], st);
    if ((e = launch_fresh(a, ranges, st)) != hipSuccess) return e;
    if (ev) (void)hipEventRecord(ev[2], st);
    if ((e = launch_split(a, st)) != hipSuccess) return e;
    if (ev) (void)hipEventRecord(ev[3], st);
    if ((e = launch_combine(a, st)) != hipSuccess) return e;
    if (every) (void)hipEventRecord(every[4], st);
    return hipSuccess;
}

}  // namespace dkv

extern "C" {

const char *dkv_last_error(void) { return g_last_error.c_str(); }

int64_t kv_page_bytes(const dkv_shape *shape) {
    return shape_ok(shape) ? page_bytes_of(shape) : 0;
}

int64_t kv_page_offset(const dkv_shape *shape, int32_t t, int32_t g, int32_t c, int32_t i) {
    if (!shape_ok(shape)) return -1;
    if (t < 0 || t >= DKV_PAGE_TOKENS || g < 0 || g >= shape->n_kv_heads || c < 0 || c > 1 || i < 0 ||
        i >= shape->head_dim)
        return -1;
    return row_offset(shape, t, g, c) + (int64_t)i * 2;
}

dkv_status kv_placement(int32_t capacity_tokens, int32_t hbm_tail_tokens, int32_t *n_pages,
                        int32_t *first_hbm_page) {
    if (capacity_tokens <= 0 || hbm_tail_tokens < 0 || !n_pages || !first_hbm_page)
        return fail(DKV_E_INVALID_ARG, "kv_placement: capacity must be > 0, tail >= 0, outputs non-null");
    const int32_t P = (int32_t)(((int64_t)capacity_tokens + DKV_PAGE_TOKENS - 1) / DKV_PAGE_TOKENS);
    const int32_t w = (int32_t)std::min<int64_t>(P, ((int64_t)hbm_tail_tokens + DKV_PAGE_TOKENS - 1) /
                                                        DKV_PAGE_TOKENS);
    *n_pages = P;
    *first_hbm_page = P - w;
    return DKV_OK;
}

dkv_status kv_alloc_host(const dkv_shape *shape, int64_t n_pages, uint32_t flags, dkv_pool **out) {
    if (!out || !shape_ok(shape) || n_pages <= 0 || flags > DKV_HOST_NONCOHERENT)
        return fail(DKV_E_INVALID_ARG, "kv_alloc_host: bad shape, n_pages, flags or null output");
    if (pool_too_large(shape, n_pages))
        return fail(DKV_E_OUT_OF_MEMORY, "kv_alloc_host: %lld pages exceed the 1 PiB pool limit", (long long)n_pages);
    return guarded("kv_alloc_host", [&]() -> dkv_status {
        std::unique_ptr<dkv_pool> p = new_pool(shape, n_pages, 0);
        const size_t bytes = (size_t)p->page_bytes * (size_t)n_pages;
        track(p.get());
        void *h = nullptr;
        const unsigned hflags = hipHostMallocMapped | hipHostMallocPortable |
                                (flags == DKV_HOST_NONCOHERENT ? hipHostMallocNonCoherent : hipHostMallocCoherent);
        hipError_t e = hipHostMalloc(&h, bytes, hflags);
        if (e != hipSuccess || !h) {
            (void)hipGetLastError();
            untrack(p.get());
            return fail(DKV_E_OUT_OF_MEMORY, "kv_alloc_host: hipHostMalloc of %zu bytes failed: %s", bytes,
                        hipGetErrorString(e));
        }
        void *d = nullptr;
        e = hipHostGetDevicePointer(&d, h, 0);
        if (e != hipSuccess || !d) {
            (void)hipHostFree(h);
            untrack(p.get());
            return hip_fail(e, "kv_alloc_host: hipHostGetDevicePointer");
        }
        p->host_base = static_cast<char *>(h);
        p->dev_base = static_cast<char *>(d);
        *out = p.release();
        return DKV_OK;
    });
}

dkv_status kv_alloc_hbm(const dkv_shape *shape, int64_t n_pages, dkv_pool **out) {
    if (!out || !shape_ok(shape) || n_pages <= 0)
        return fail(DKV_E_INVALID_ARG, "kv_alloc_hbm: bad shape, n_pages or null output");
    if (pool_too_large(shape, n_pages))
        return fail(DKV_E_OUT_OF_MEMORY, "kv_alloc_hbm: %lld pages exceed the 1 PiB pool limit", (long long)n_pages);
    return guarded("kv_alloc_hbm", [&]() -> dkv_status {
        std::unique_ptr<dkv_pool> p = new_pool(shape, n_pages, 1);
        const size_t bytes = (size_t)p->page_bytes * (size_t)n_pages;
        track(p.get());
        void *d = nullptr;
        hipError_t e = hipMalloc(&d, bytes);
        if (e != hipSuccess || !d) {
            (void)hipGetLastError();
            untrack(p.get());
            return fail(DKV_E_OUT_OF_MEMORY, "kv_alloc_hbm: hipMalloc of %zu bytes failed: %s", bytes,
                        hipGetErrorString(e));
        }
        p->dev_base = static_cast<char *>(d);
        *out = p.release();
        return DKV_OK;
    });
}

dkv_status kv_pool_free_pages(const dkv_pool *pool, int64_t *n_free) {
    if (!pool || !n_free || !live(pool)) return fail(DKV_E_INVALID_ARG, "kv_pool_free_pages: null or freed pool");
    *n_free = pool->n_free;
    return DKV_OK;
}

dkv_status kv_pool_info(const dkv_pool *pool, void **device_base, int64_t *bytes, int32_t *tier) {
    if (!pool || !live(pool)) return fail(DKV_E_INVALID_ARG, "kv_pool_info: null or freed pool");
    if (device_base) *device_base = pool->dev_base;
    if (bytes) *bytes = pool->n_pages * pool->page_bytes;
    if (tier) *tier = pool->tier;
    return DKV_OK;
}

dkv_status kv_pool_free(dkv_pool *pool) {
    if (!pool) return DKV_OK;
    if (!live(pool)) return fail(DKV_E_INVALID_ARG, "kv_pool_free: not a live pool (freed twice?)");
    if (pool->n_layouts > 0)
        return fail(DKV_E_INVALID_ARG, "kv_pool_free: %lld layout(s) still use this pool",
                    (long long)pool->n_layouts);
    untrack(pool);
    hipError_t e = pool->tier == 0 ? hipHostFree(pool->host_base) : hipFree(pool->dev_base);
    delete pool;
    if (e != hipSuccess) return hip_fail(e, "kv_pool_free");
    return DKV_OK;
}

static dkv_status check_pools(const dkv_shape *shape, int32_t batch, const int32_t *capacity_tokens,
                              dkv_pool *host_pool, dkv_pool *hbm_pool, dkv_layout **out, const char *who) {
    if (!out || !shape_ok(shape) || batch <= 0 || !capacity_tokens)
        return fail(DKV_E_INVALID_ARG, "%s: bad shape, batch or null argument", who);
    if (!shape_supported(shape))
        return fail(DKV_E_UNSUPPORTED, "%s: head_dim must be 64/128, group 1/2/4/8, hidden a multiple of 512", who);
    if (batch > 65535) return fail(DKV_E_INVALID_ARG, "%s: batch > 65535", who);
    for (dkv_pool *p : {host_pool, hbm_pool}) {
        if (p && !live(p)) return fail(DKV_E_INVALID_ARG, "%s: a pool argument is not a live pool", who);
        if (p && (p->shape.n_kv_heads != shape->n_kv_heads || p->shape.head_dim != shape->head_dim))
            return fail(DKV_E_INVALID_ARG, "%s: pool page shape differs from the layout's", who);
    }
    if (host_pool && host_pool->tier != 0) return fail(DKV_E_INVALID_ARG, "%s: host_pool is HBM", who);
    if (hbm_pool && hbm_pool->tier != 1) return fail(DKV_E_INVALID_ARG, "%s: hbm_pool is host", who);
    for (int b = 0; b < batch; ++b)
        if (capacity_tokens[b] <= 0)
            return fail(DKV_E_INVALID_ARG, "%s: capacity of sequence %d is not positive", who, b);
    return DKV_OK;
}

// Allocates the layout's device tables and scratch, uploads the page table
// (and the window tables), and hands the layout out; frees everything on
// failure.
// Debug knobs of the LDS producer/consumer split kernels, the race detector
// of their handoff: DKV_LDS_RING=2|3|4 ring slots (default 4 for the VALU
// consumers, 2 for the matrix-core consumer: measured fastest, see
// attn_split.hip), DKV_POISON=1 fills every slot with NaN before it is refilled, so a
// consumer that read a slot before its loads landed would produce NaN
// instead of a silently stale result. Neither changes the arithmetic.
static void choose_lds_ring(dkv_layout *L) {
    L->lds_ring = 0;                   // each ring kernel's own default
    if (const char *env = getenv("DKV_LDS_RING")) {
        const int v = atoi(env);
        if (v >= 2 && v <= 4) L->lds_ring = v;
    }
    const char *poison = getenv("DKV_POISON");
    L->lds_poison = poison && strcmp(poison, "1") == 0;
}

// The projection form of the layout's steps (dkv::projection_form reads only
// the batch, the shape and the thresholds, all fixed at creation).
static int projection_form_of(const dkv_layout *L) {
    dkv::StepArgs a{};
    a.batch = L->batch;
    a.hidden = L->shape.hidden;
    a.n_qkv = (L->shape.n_q_heads + 2 * L->shape.n_kv_heads) * L->shape.head_dim;
    a.proj_mfma_min_batch = L->proj_mfma_min_batch;
    a.proj_splitk_min_batch = L->proj_splitk_min_batch;
    a.proj_ranges = L->proj_ranges;
    return dkv::projection_form(a);
}

// DKV_LOG=1: one line per layout on stderr with the launch plan its decode
// steps will use (measurement and debugging aid; nothing else changes).
static void log_plan(const dkv_layout *L, int64_t n_host, int64_t n_hbm) {
    const char *env = getenv("DKV_LOG");
    if (!env || strcmp(env, "1") != 0) return;
    static const char *const kSplitNames[] = {"regs", "lds", "naive", "mfma", "ldsmfma"};
    const dkv_shape *s = &L->shape;
    const int B = L->batch;
    static const char *const kProjNames[] = {"gemv", "mfma one-tile streamed", "mfma split-k (x staged in LDS)",
                                             "mfma tiled (x and W staged in LDS)"};
    const char *proj = kProjNames[projection_form_of(L)];
    fprintf(stderr,
            "[dkv] layout: batch %d, hidden %d, heads %d/%d, head_dim %d, layers %d; pages per layer: "
            "%lld host, %lld HBM%s; split %d tokens (%d per sequence at most), split kernel %s on %s; "
            "projection %s\n",
            B, s->hidden, s->n_q_heads, s->n_kv_heads, s->head_dim, s->n_layers, (long long)n_host,
            (long long)n_hbm, L->windowed ? " (sliding window)" : "", L->split_tokens, L->max_splits,
            kSplitNames[L->split_variant],
            L->split_waves > 0 ? (std::to_string(L->split_waves) + " looping wavefronts").c_str()
                               : "one wavefront per item",
            proj);
}

static dkv_status finish_layout(dkv_layout *L, const std::vector<uint64_t> &table,
                                const std::vector<uint64_t> *host_pages, const std::vector<uint64_t> *ring,
                                dkv_layout **out) {
    const dkv_shape *shape = &L->shape;
    const int batch = L->batch;
    int32_t max_cap = 0;
    for (int b = 0; b < batch; ++b) max_cap = std::max(max_cap, L->capacity[b]);
    L->split_tokens = choose_split_tokens(batch, shape->n_kv_heads, L->capacity.data());
    L->max_splits = std::max(1, (std::max(1, max_cap - 1) + L->split_tokens - 1) / L->split_tokens);
    int64_t item_slots = 0;
    for (int b = 0; b < batch; ++b) item_slots += (L->capacity[b] - 1 + L->split_tokens - 1) / L->split_tokens;
    L->item_slots = (int32_t)std::max<int64_t>(1, std::min<int64_t>(item_slots, INT32_MAX));
    L->scratch = dkv::scratch_plan(batch, shape->n_q_heads, shape->n_kv_heads, shape->head_dim, L->max_splits + 1);
    L->split_variant = choose_split_variant(shape->n_q_heads / shape->n_kv_heads, shape->head_dim);
    int64_t n_host = 0, n_hbm = 0;
    for (int b = 0; b < batch; ++b) {
        const int hot = L->windowed ? L->window[b] : L->n_pages[b] - L->first_hbm[b];
        n_host += L->n_pages[b] - hot;
        n_hbm += hot;
    }
    L->split_waves = choose_split_waves(n_host, n_hbm);
    L->proj_mfma_min_batch = choose_proj_mfma_min_batch();
    L->proj_splitk_min_batch = choose_proj_splitk_min_batch();
    L->proj_ranges = choose_proj_ranges();
    choose_lds_ring(L);
    log_plan(L, n_host, n_hbm);
    track(L);                          // the last step that can throw
    if (L->host_pool) ++L->host_pool->n_layouts;
    if (L->hbm_pool) ++L->hbm_pool->n_layouts;

    auto cleanup = [&](dkv_status st) {
        untrack(L);
        free_device(L);
        release_pages(L);
        if (L->host_pool) --L->host_pool->n_layouts;
        if (L->hbm_pool) --L->hbm_pool->n_layouts;
        delete L;
        return st;
    };
    // The one-wavefront-per-item launches put the splits of a sequence in
    // grid dimension y (at most 65535); the step's item list packs a split
    // index into 16 bits and indexes its batch * max_splits entries with int.
    if (L->max_splits > 65535) {
        fail(DKV_E_UNSUPPORTED, "kv_layout_create: %d splits per sequence (capacity / split size) exceed 65535",
             L->max_splits);
        return cleanup(DKV_E_UNSUPPORTED);
    }
    if ((int64_t)batch * L->max_splits >= (int64_t)INT32_MAX) {
        fail(DKV_E_UNSUPPORTED, "kv_layout_create: batch x splits per sequence (%lld) exceeds 2^31 - 1",
             (long long)batch * L->max_splits);
        return cleanup(DKV_E_UNSUPPORTED);
    }
    const size_t n_entries = table.size();
    struct {
        void **ptr;
        size_t bytes;
    } allocs[] = {{(void **)&L->d_page_table, n_entries * sizeof(uint64_t)},
                  {(void **)&L->d_capacity, (size_t)batch * sizeof(int32_t)},
                  {(void **)&L->d_scratch, L->scratch.total},
                  {(void **)&L->d_status, 256},
                  {(void **)&L->d_host_pages, host_pages ? host_pages->size() * sizeof(uint64_t) : 0},
                  {(void **)&L->d_ring, ring ? ring->size() * sizeof(uint64_t) : 0},
                  {(void **)&L->d_window, L->windowed ? (size_t)batch * sizeof(int32_t) : 0}};
    for (auto &a : allocs) {
        if (a.bytes == 0) continue;
        if (hipMalloc(a.ptr, a.bytes) != hipSuccess) {
            (void)hipGetLastError();
            *a.ptr = nullptr;
            fail(DKV_E_OUT_OF_MEMORY, "kv_layout_create: hipMalloc of %zu bytes failed", a.bytes);
            return cleanup(DKV_E_OUT_OF_MEMORY);
        }
    }
    hipError_t e = hipMemcpy(L->d_page_table, table.data(), n_entries * sizeof(uint64_t), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(L->d_capacity, L->capacity.data(), (size_t)batch * sizeof(int32_t), hipMemcpyHostToDevice);
    if (e == hipSuccess && host_pages)
        e = hipMemcpy(L->d_host_pages, host_pages->data(), host_pages->size() * sizeof(uint64_t),
                      hipMemcpyHostToDevice);
    if (e == hipSuccess && ring)
        e = hipMemcpy(L->d_ring, ring->data(), ring->size() * sizeof(uint64_t), hipMemcpyHostToDevice);
    if (e == hipSuccess && L->windowed) {
        e = hipMemcpy(L->d_window, L->window.data(), (size_t)batch * sizeof(int32_t), hipMemcpyHostToDevice);
    }
    if (e == hipSuccess) e = hipMemset(L->d_status, 0, 256);
    if (e == hipSuccess) e = hipMemset(L->d_scratch, 0, L->scratch.total);
    if (e != hipSuccess) {
        hip_fail(e, "kv_layout_create: initialising device tables");
        return cleanup(DKV_E_HIP);
    }
    *out = L;
    return DKV_OK;
}

// A layout under construction that an exception interrupted: its pages go
// back to their pools (it was neither tracked nor counted by them yet).
static void abandon_layout(dkv_layout *L) {
    if (!L) return;
    release_pages(L);
    delete L;
}

static dkv_status layout_create_static(const dkv_shape *shape, int32_t batch, const int32_t *capacity_tokens,
                                       const int32_t *hbm_tail_tokens, dkv_pool *host_pool, dkv_pool *hbm_pool,
                                       dkv_layout **out, dkv_layout *&L) {
    L = new dkv_layout();
    L->shape = *shape;
    L->batch = batch;
    L->capacity.assign(capacity_tokens, capacity_tokens + batch);
    L->n_pages.resize(batch);
    L->first_hbm.resize(batch);
    L->host_pool = host_pool;
    L->hbm_pool = hbm_pool;
    int64_t need_host = 0, need_hbm = 0;
    int32_t max_pages = 0;
    for (int b = 0; b < batch; ++b) {
        const int32_t tail = hbm_tail_tokens ? hbm_tail_tokens[b] : 0;
        if (kv_placement(capacity_tokens[b], tail, &L->n_pages[b], &L->first_hbm[b]) != DKV_OK) {
            delete L;
            return fail(DKV_E_INVALID_ARG, "kv_layout_create: sequence %d: capacity %d / hbm tail %d invalid",
                        b, capacity_tokens[b], tail);
        }
        need_host += L->first_hbm[b];
        need_hbm += L->n_pages[b] - L->first_hbm[b];
        max_pages = std::max(max_pages, L->n_pages[b]);
    }
    need_host *= shape->n_layers;
    need_hbm *= shape->n_layers;
    if ((need_host > 0 && !host_pool) || (need_hbm > 0 && !hbm_pool)) {
        delete L;
        return fail(DKV_E_INVALID_ARG,
                    "kv_layout_create: placement needs %lld host and %lld HBM pages but a pool is missing",
                    (long long)need_host, (long long)need_hbm);
    }
    if ((host_pool && host_pool->n_free < need_host) || (hbm_pool && hbm_pool->n_free < need_hbm)) {
        delete L;
        return fail(DKV_E_CAPACITY, "kv_layout_create: needs %lld host / %lld HBM pages, pools have %lld / %lld free",
                    (long long)need_host, (long long)need_hbm, (long long)(host_pool ? host_pool->n_free : 0),
                    (long long)(hbm_pool ? hbm_pool->n_free : 0));
    }
    L->max_pages = max_pages;
    L->owned.reserve((size_t)(need_host + need_hbm));   // so that recording a taken page cannot throw

    // Pages are taken in (layer, sequence, page) order, so each sequence's
    // pages of a tier are consecutive in their pool when it is fresh.
    std::vector<uint64_t> table((size_t)shape->n_layers * batch * max_pages, 0);
    std::vector<int64_t> got;
    for (int layer = 0; layer < shape->n_layers; ++layer) {
        for (int b = 0; b < batch; ++b) {
            for (int tier = 0; tier < 2; ++tier) {
                const int p_lo = tier == 0 ? 0 : L->first_hbm[b];
                const int p_hi = tier == 0 ? L->first_hbm[b] : L->n_pages[b];
                if (p_hi <= p_lo) continue;
                dkv_pool *pool = tier == 0 ? host_pool : hbm_pool;
                take_pages(pool, p_hi - p_lo, got);   // counts were checked above
                for (int p = p_lo; p < p_hi; ++p) {
                    const int64_t idx = got[p - p_lo];
                    L->owned.emplace_back(pool, idx);
                    table[pt_index(L, layer, b, p)] = page_addr(pool, idx);
                }
            }
        }
    }
    return finish_layout(L, table, nullptr, nullptr, out);
}

dkv_status kv_layout_create(const dkv_shape *shape, int32_t batch, const int32_t *capacity_tokens,
                            const int32_t *hbm_tail_tokens, dkv_pool *host_pool, dkv_pool *hbm_pool,
                            dkv_layout **out) {
    dkv_status st = check_pools(shape, batch, capacity_tokens, host_pool, hbm_pool, out, "kv_layout_create");
    if (st != DKV_OK) return st;
    dkv_layout *L = nullptr;
    try {
        return layout_create_static(shape, batch, capacity_tokens, hbm_tail_tokens, host_pool, hbm_pool, out, L);
    } catch (const std::exception &ex) {
        abandon_layout(L);
        return fail(DKV_E_OUT_OF_MEMORY, "kv_layout_create: host memory exhausted (%s)", ex.what());
    }
}

static dkv_status layout_create_windowed(const dkv_shape *shape, int32_t batch, const int32_t *capacity_tokens,
                                         const int32_t *window_tokens, const int32_t *ctx_lens, dkv_pool *host_pool,
                                         dkv_pool *hbm_pool, dkv_layout **out, dkv_layout *&L) {
    const char *who = "kv_layout_create_windowed";
    L = new dkv_layout();
    L->shape = *shape;
    L->batch = batch;
    L->windowed = 1;
    L->capacity.assign(capacity_tokens, capacity_tokens + batch);
    L->n_pages.resize(batch);
    L->first_hbm.resize(batch);
    L->window.resize(batch);
    L->host_pool = host_pool;
    L->hbm_pool = hbm_pool;
    int64_t need_host = 0, need_hbm = 0;
    int32_t max_pages = 0, max_window = 0;
    for (int b = 0; b < batch; ++b) {
        if (window_tokens[b] <= 0 || ctx_lens[b] < 0 || ctx_lens[b] >= capacity_tokens[b]) {
            delete L;
            return fail(DKV_E_INVALID_ARG, "%s: sequence %d: window %d must be > 0 and ctx_lens %d in [0, capacity %d)",
                        who, b, window_tokens[b], ctx_lens[b], capacity_tokens[b]);
        }
        L->n_pages[b] = (int32_t)(((int64_t)capacity_tokens[b] + DKV_PAGE_TOKENS - 1) / DKV_PAGE_TOKENS);
        L->window[b] = (int32_t)std::min<int64_t>(L->n_pages[b],
                                                  ((int64_t)window_tokens[b] + DKV_PAGE_TOKENS - 1) / DKV_PAGE_TOKENS);
        L->first_hbm[b] = L->n_pages[b];
        need_host += L->n_pages[b];
        need_hbm += L->window[b];
        max_pages = std::max(max_pages, L->n_pages[b]);
        max_window = std::max(max_window, L->window[b]);
    }
    need_host *= shape->n_layers;
    need_hbm *= shape->n_layers;
    if (host_pool->n_free < need_host || hbm_pool->n_free < need_hbm) {
        delete L;
        return fail(DKV_E_CAPACITY, "%s: needs %lld host / %lld HBM pages, pools have %lld / %lld free", who,
                    (long long)need_host, (long long)need_hbm, (long long)host_pool->n_free,
                    (long long)hbm_pool->n_free);
    }
    L->max_pages = max_pages;
    L->max_window = max_window;
    L->owned.reserve((size_t)(need_host + need_hbm));   // so that recording a taken page cannot throw

    // Every page has a host page; page p of the window uses HBM ring slot
    // p % W. The pages [P - W + 1, P] up to the one holding slot ctx_lens[b]
    // start in HBM.
    const size_t n_entries = (size_t)shape->n_layers * batch * max_pages;
    std::vector<uint64_t> table(n_entries, 0), host_pages(n_entries, 0);
    std::vector<uint64_t> ring((size_t)shape->n_layers * batch * max_window, 0);
    std::vector<int64_t> got;
    for (int layer = 0; layer < shape->n_layers; ++layer) {
        for (int b = 0; b < batch; ++b) {
            const int W = L->window[b];
            take_pages(host_pool, L->n_pages[b], got);
            for (int p = 0; p < L->n_pages[b]; ++p) {
                L->owned.emplace_back(host_pool, got[p]);
                host_pages[pt_index(L, layer, b, p)] = table[pt_index(L, layer, b, p)] = page_addr(host_pool, got[p]);
            }
            take_pages(hbm_pool, W, got);
            for (int k = 0; k < W; ++k) {
                L->owned.emplace_back(hbm_pool, got[k]);
                ring[((size_t)layer * batch + b) * max_window + k] = page_addr(hbm_pool, got[k]);
            }
            const int P = ctx_lens[b] / DKV_PAGE_TOKENS;
            for (int p = std::max(0, P - W + 1); p <= P; ++p)
                table[pt_index(L, layer, b, p)] = ring[((size_t)layer * batch + b) * max_window + p % W];
        }
    }
    return finish_layout(L, table, &host_pages, &ring, out);
}

dkv_status kv_layout_create_windowed(const dkv_shape *shape, int32_t batch, const int32_t *capacity_tokens,
                                     const int32_t *window_tokens, const int32_t *ctx_lens, dkv_pool *host_pool,
                                     dkv_pool *hbm_pool, dkv_layout **out) {
    const char *who = "kv_layout_create_windowed";
    dkv_status st = check_pools(shape, batch, capacity_tokens, host_pool, hbm_pool, out, who);
    if (st != DKV_OK) return st;
    if (!window_tokens || !ctx_lens || !host_pool || !hbm_pool)
        return fail(DKV_E_INVALID_ARG, "%s: window_tokens, ctx_lens and both pools are required", who);
    dkv_layout *L = nullptr;
    try {
        return layout_create_windowed(shape, batch, capacity_tokens, window_tokens, ctx_lens, host_pool, hbm_pool,
                                      out, L);
    } catch (const std::exception &ex) {
        abandon_layout(L);
        return fail(DKV_E_OUT_OF_MEMORY, "%s: host memory exhausted (%s)", who, ex.what());
    }
}

static dkv_status kv_layout_timing_enable_body(dkv_layout *L, int32_t enable, int32_t max_steps) {
    if (!L || !live(L) || enable < 0 || enable > 2 || (enable && max_steps <= 0))
        return fail(DKV_E_INVALID_ARG,
                    "kv_layout_timing_enable: null or freed layout, enable not 0, 1 or 2, or max_steps <= 0");
    HIP_TRY(hipDeviceSynchronize());
    for (hipEvent_t e : L->timing_events) (void)hipEventDestroy(e);
    L->timing_events.clear();
    L->timing_recorded = 0;
    L->timing_mode = enable;
    if (!enable) return DKV_OK;
    L->timing_events.resize((size_t)max_steps * kTimingEvents);
    for (auto &e : L->timing_events) HIP_TRY(hipEventCreate(&e));
    return DKV_OK;
}

dkv_status kv_layout_timing_enable(dkv_layout *L, int32_t enable, int32_t max_steps) {
    return guarded("kv_layout_timing_enable",
                   [&] { return kv_layout_timing_enable_body(L, enable, max_steps); });
}

dkv_status kv_layout_timing_read(dkv_layout *L, double *ms_proj, double *ms_fresh, double *ms_split,
                                 double *ms_combine, int32_t *n_steps) {
    if (!L || !live(L)) return fail(DKV_E_INVALID_ARG, "kv_layout_timing_read: null or freed layout");
    HIP_TRY(hipDeviceSynchronize());
    double sum[kTimingEvents - 1] = {};
    for (int32_t i = 0; i < L->timing_recorded; ++i) {
        hipEvent_t *ev = &L->timing_events[(size_t)i * kTimingEvents];
        for (int k = 0; k + 1 < kTimingEvents; ++k) {
            if (L->timing_mode == 2 && k != 2) continue;   // only the split kernel's pair was recorded
            float ms = 0.0f;
            HIP_TRY(hipEventElapsedTime(&ms, ev[k], ev[k + 1]));
            sum[k] += ms;
        }
    }
    if (ms_proj) *ms_proj = sum[0];
    if (ms_fresh) *ms_fresh = sum[1];
    if (ms_split) *ms_split = sum[2];
    if (ms_combine) *ms_combine = sum[3];
    if (n_steps) *n_steps = L->timing_recorded;
    L->timing_recorded = 0;
    return DKV_OK;
}

dkv_status kv_layout_free(dkv_layout *L) {
    if (!L) return DKV_OK;
    if (!untrack(L)) return fail(DKV_E_INVALID_ARG, "kv_layout_free: not a live layout (freed twice?)");
    (void)hipDeviceSynchronize();
    for (hipEvent_t e : L->timing_events) (void)hipEventDestroy(e);
    free_device(L);
    release_pages(L);
    if (L->host_pool) --L->host_pool->n_layouts;
    if (L->hbm_pool) --L->hbm_pool->n_layouts;
    delete L;
    return DKV_OK;
}

static dkv_status kv_layout_page_tier_body(const dkv_layout *L, int32_t seq, int32_t page, int32_t *tier) {
    if (!L || !tier || !live(L)) return fail(DKV_E_INVALID_ARG, "kv_layout_page_tier: null or freed layout");
    if (seq < 0 || seq >= L->batch || page < 0 || page >= L->n_pages[seq])
        return fail(DKV_E_INVALID_ARG, "kv_layout_page_tier: index out of range");
    std::vector<uint64_t> row;
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(table_row(L, 0, seq, page, page, row));
    *tier = host_view(L, row[0]) ? 0 : 1;
    return DKV_OK;
}

dkv_status kv_layout_page_tier(const dkv_layout *L, int32_t seq, int32_t page, int32_t *tier) {
    return guarded("kv_layout_page_tier", [&] { return kv_layout_page_tier_body(L, seq, page, tier); });
}

int32_t kv_layout_split_tokens(const dkv_layout *L) { return L && live(L) ? L->split_tokens : 0; }

int32_t kv_layout_split_kernel(const dkv_layout *L) { return L && live(L) ? L->split_variant : -1; }

int32_t kv_layout_split_waves(const dkv_layout *L) { return L && live(L) ? L->split_waves : -1; }

int32_t kv_layout_projection_kernel(const dkv_layout *L) { return L && live(L) ? projection_form_of(L) : -1; }

dkv_status kv_layout_set_split_kernel(dkv_layout *L, int32_t kernel) {
    if (!L || !live(L)) return fail(DKV_E_INVALID_ARG, "kv_layout_set_split_kernel: null or freed layout");
    const int32_t group = L->shape.n_q_heads / L->shape.n_kv_heads;
    const bool ok = kernel == dkv::kSplitRegisters || kernel == dkv::kSplitLds || kernel == dkv::kSplitNaive ||
                    (kernel == dkv::kSplitMfma && group >= dkv::kMfmaMinGroup) ||
                    (kernel == dkv::kSplitLdsMfma && lds_mfma_supported(group, L->shape.head_dim));
    if (!ok)
        return fail(DKV_E_INVALID_ARG, "kv_layout_set_split_kernel: unknown kernel %d, or not for this shape", kernel);
    L->split_variant = kernel;
    return DKV_OK;
}

static dkv_status check_range(const dkv_layout *L, int32_t layer, int32_t seq, int32_t start, int32_t n,
                              const char *who) {
    if (!L || !live(L)) return fail(DKV_E_INVALID_ARG, "%s: null or freed layout", who);
    if (layer < 0 || layer >= L->shape.n_layers || seq < 0 || seq >= L->batch || start < 0 || n < 0)
        return fail(DKV_E_INVALID_ARG, "%s: layer/seq/start/n out of range", who);
    if ((int64_t)start + n > L->capacity[seq])
        return fail(DKV_E_CAPACITY, "%s: slots [%d, %lld) exceed capacity %d", who, start,
                    (long long)start + n, L->capacity[seq]);
    return DKV_OK;
}

// Memory a kernel can read in place: HBM (hipMalloc) or managed memory.
// Pinned host memory and ordinary CPU memory (which the runtime does not
// know, an error it reports and that is cleared here) are host memory.
static bool device_resident(const void *p) {
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

static dkv_status kv_append_body(dkv_layout *L, int32_t layer, int32_t seq, int32_t start, int32_t n,
                                 const uint16_t *k, const uint16_t *v, dkv_stream_t stream) {
    dkv_status st = check_range(L, layer, seq, start, n, "kv_append");
    if (st != DKV_OK) return st;
    if (n == 0) return DKV_OK;
    if (!k || !v) return fail(DKV_E_INVALID_ARG, "kv_append: null k or v");
    const bool on_device = device_resident(k);
    if (on_device != device_resident(v))
        return fail(DKV_E_INVALID_ARG, "kv_append: k and v must both be device or both be host buffers");
    if (on_device) {
        // Device buffers: one kernel scatters the rows into the pages on
        // `stream` (after any earlier work there that moves pages), then waits.
        if (((uintptr_t)k | (uintptr_t)v) & 15u)
            return fail(DKV_E_INVALID_ARG, "kv_append: device k and v must be 16-byte aligned");
        dkv::AppendArgs a{};
        a.n_kv_heads = L->shape.n_kv_heads;
        a.head_dim = L->shape.head_dim;
        a.start = start;
        a.page_table = L->d_page_table + pt_index(L, layer, seq, 0);
        a.k = k;
        a.v = v;
        hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
        hipError_t e = dkv::launch_append(a, n, hs);
        if (e == hipSuccess) e = hipStreamSynchronize(hs);
        if (e != hipSuccess) return hip_fail(e, "kv_append");
        return DKV_OK;
    }
    const dkv_shape *s = &L->shape;
    const int D = s->head_dim, Hkv = s->n_kv_heads;
    const size_t row = (size_t)D * 2;
    const size_t tok_elems = (size_t)Hkv * D;
    const int p_first = start / DKV_PAGE_TOKENS, p_last = (start + n - 1) / DKV_PAGE_TOKENS;
    hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
    HIP_TRY(hipStreamSynchronize(hs));            // earlier work may still move or write pages
    std::vector<uint64_t> addr;
    HIP_TRY(table_row(L, layer, seq, p_first, p_last, addr));

    auto fill = [&](char *page, int p) {
        const int t_lo = std::max(start, p * DKV_PAGE_TOKENS);
        const int t_hi = std::min(start + n, (p + 1) * DKV_PAGE_TOKENS);
        for (int t = t_lo; t < t_hi; ++t)
            for (int g = 0; g < Hkv; ++g) {
                const size_t src = (size_t)(t - start) * tok_elems + (size_t)g * D;
                memcpy(page + row_offset(s, t % DKV_PAGE_TOKENS, g, 0), k + src, row);
                memcpy(page + row_offset(s, t % DKV_PAGE_TOKENS, g, 1), v + src, row);
            }
    };

    // Host pages: the CPU writes them in place, page by page, in parallel.
    parallel_for(p_last - p_first + 1, [&](int64_t i0, int64_t i1) {
        for (int64_t i = i0; i < i1; ++i)
            if (char *page = host_view(L, addr[i])) fill(page, p_first + (int)i);
    });

    // HBM pages: assemble each touched page on the host (reading it back
    // first when only part of it is written) and copy it in.
    const size_t pb = (size_t)page_bytes_of(s);
    std::vector<char> img(pb);
    for (int p = p_first; p <= p_last; ++p) {
        const uint64_t a = addr[p - p_first];
        if (host_view(L, a)) continue;
        void *dpage = reinterpret_cast<void *>((uintptr_t)a);
        const int t_lo = std::max(start, p * DKV_PAGE_TOKENS);
        const int t_hi = std::min(start + n, (p + 1) * DKV_PAGE_TOKENS);
        if (t_hi - t_lo < DKV_PAGE_TOKENS) {
            HIP_TRY(hipMemcpyAsync(img.data(), dpage, pb, hipMemcpyDeviceToHost, hs));
            HIP_TRY(hipStreamSynchronize(hs));
        }
        fill(img.data(), p);
        HIP_TRY(hipMemcpyAsync(dpage, img.data(), pb, hipMemcpyHostToDevice, hs));
        HIP_TRY(hipStreamSynchronize(hs));
    }
    return DKV_OK;
}

dkv_status kv_append(dkv_layout *L, int32_t layer, int32_t seq, int32_t start, int32_t n, const uint16_t *k,
                     const uint16_t *v, dkv_stream_t stream) {
    return guarded("kv_append", [&] { return kv_append_body(L, layer, seq, start, n, k, v, stream); });
}

static dkv_status kv_read_body(const dkv_layout *L, int32_t layer, int32_t seq, int32_t start, int32_t n,
                               uint16_t *k_out, uint16_t *v_out) {
    dkv_status st = check_range(L, layer, seq, start, n, "kv_read");
    if (st != DKV_OK) return st;
    if (n == 0) return DKV_OK;
    if (!k_out || !v_out) return fail(DKV_E_INVALID_ARG, "kv_read: null output");
    HIP_TRY(hipDeviceSynchronize());
    const dkv_shape *s = &L->shape;
    const int D = s->head_dim, Hkv = s->n_kv_heads;
    const size_t row = (size_t)D * 2;
    const size_t tok_elems = (size_t)Hkv * D;
    const int p_first = start / DKV_PAGE_TOKENS, p_last = (start + n - 1) / DKV_PAGE_TOKENS;
    std::vector<uint64_t> addr;
    HIP_TRY(table_row(L, layer, seq, p_first, p_last, addr));
    std::vector<char> img((size_t)page_bytes_of(s));
    for (int p = p_first; p <= p_last; ++p) {
        const char *page = host_view(L, addr[p - p_first]);
        if (!page) {
            HIP_TRY(hipMemcpy(img.data(), reinterpret_cast<const void *>((uintptr_t)addr[p - p_first]), img.size(),
                              hipMemcpyDeviceToHost));
            page = img.data();
        }
        const int t_lo = std::max(start, p * DKV_PAGE_TOKENS);
        const int t_hi = std::min(start + n, (p + 1) * DKV_PAGE_TOKENS);
        for (int t = t_lo; t < t_hi; ++t)
            for (int g = 0; g < Hkv; ++g) {
                const size_t dst = (size_t)(t - start) * tok_elems + (size_t)g * D;
                memcpy(k_out + dst, page + row_offset(s, t % DKV_PAGE_TOKENS, g, 0), row);
                memcpy(v_out + dst, page + row_offset(s, t % DKV_PAGE_TOKENS, g, 1), row);
            }
    }
    return DKV_OK;
}

dkv_status kv_read(const dkv_layout *L, int32_t layer, int32_t seq, int32_t start, int32_t n, uint16_t *k_out,
                   uint16_t *v_out) {
    return guarded("kv_read", [&] { return kv_read_body(L, layer, seq, start, n, k_out, v_out); });
}

static dkv_status dkv_cpu_attention_body(const dkv_layout *L, int32_t layer, const float *q, const uint16_t *k_new,
                                         const uint16_t *v_new, const int32_t *ctx_lens, float *out,
                                         int32_t n_threads, int32_t *threads_used) {
    if (!L || !live(L)) return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention: null or freed layout");
    if (layer < 0 || layer >= L->shape.n_layers)
        return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention: layer %d out of range", layer);
    if (!q || !k_new || !v_new || !ctx_lens || !out)
        return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention: null pointer argument");
    if (n_threads < 1 || n_threads > 1024)
        return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention: n_threads %d outside [1, 1024]", n_threads);
    const int B = L->batch;
    for (int b = 0; b < B; ++b)
        if (ctx_lens[b] < 0 || ctx_lens[b] > L->capacity[b] - 1)
            return fail(DKV_E_CAPACITY, "dkv_cpu_attention: ctx_lens[%d] = %d outside [0, %d]", b, ctx_lens[b],
                        L->capacity[b] - 1);
    HIP_TRY(hipDeviceSynchronize());              // pages written by earlier steps are complete
    std::vector<const char *> pages((size_t)B * L->max_pages, nullptr);
    std::vector<uint64_t> addr;
    for (int b = 0; b < B; ++b) {
        const int n = (ctx_lens[b] + DKV_PAGE_TOKENS - 1) / DKV_PAGE_TOKENS;
        if (n == 0) continue;
        HIP_TRY(table_row(L, layer, b, 0, n - 1, addr));
        for (int p = 0; p < n; ++p) {
            const char *page = host_view(L, addr[(size_t)p]);
            if (!page)
                return fail(DKV_E_INVALID_ARG,
                            "dkv_cpu_attention: page %d of sequence %d is in HBM; the CPU reads host pages only",
                            p, b);
            pages[(size_t)b * L->max_pages + p] = page;
        }
    }
    return dkv_cpu_attention_pages(reinterpret_cast<const void *const *>(pages.data()), L->max_pages, &L->shape, B,
                                   q, k_new, v_new, ctx_lens, out, n_threads, threads_used);
}

dkv_status dkv_cpu_attention(const dkv_layout *L, int32_t layer, const float *q, const uint16_t *k_new,
                             const uint16_t *v_new, const int32_t *ctx_lens, float *out, int32_t n_threads,
                             int32_t *threads_used) {
    return guarded("dkv_cpu_attention", [&] {
        return dkv_cpu_attention_body(L, layer, q, k_new, v_new, ctx_lens, out, n_threads, threads_used);
    });
}

static dkv_status dkv_cpu_attention_pages_body(const void *const *pages, int32_t max_pages, const dkv_shape *shape,
                                               int32_t batch, const float *q, const uint16_t *k_new,
                                               const uint16_t *v_new, const int32_t *ctx_lens, float *out,
                                               int32_t n_threads, int32_t *threads_used) {
    if (!shape_ok(shape) || !shape_supported(shape))
        return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention_pages: invalid or unsupported shape");
    if (!pages || !q || !k_new || !v_new || !ctx_lens || !out || batch < 1 || max_pages < 1)
        return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention_pages: null pointer, batch or max_pages");
    if (n_threads < 1 || n_threads > 1024)
        return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention_pages: n_threads %d outside [1, 1024]", n_threads);
    for (int b = 0; b < batch; ++b) {
        const int64_t n = ((int64_t)ctx_lens[b] + DKV_PAGE_TOKENS - 1) / DKV_PAGE_TOKENS;
        if (ctx_lens[b] < 0 || n > max_pages)
            return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention_pages: ctx_lens[%d] = %d does not fit %d pages", b,
                        ctx_lens[b], max_pages);
        for (int p = 0; p < n; ++p)
            if (!pages[(size_t)b * max_pages + p])
                return fail(DKV_E_INVALID_ARG, "dkv_cpu_attention_pages: page %d of sequence %d is missing", p, b);
    }
    dkv::CpuAttentionJob job{};
    job.batch = batch;
    job.n_q_heads = shape->n_q_heads;
    job.n_kv_heads = shape->n_kv_heads;
    job.head_dim = shape->head_dim;
    job.max_pages = max_pages;
    job.pages = reinterpret_cast<const char *const *>(pages);
    job.ctx_lens = ctx_lens;
    job.q = q;
    job.k_new = k_new;
    job.v_new = v_new;
    job.out = out;
    job.n_threads = n_threads;
    const int used = dkv::cpu_attention_run(job);
    if (threads_used) *threads_used = used;
    return DKV_OK;
}

dkv_status dkv_cpu_attention_pages(const void *const *pages, int32_t max_pages, const dkv_shape *shape,
                                   int32_t batch, const float *q, const uint16_t *k_new, const uint16_t *v_new,
                                   const int32_t *ctx_lens, float *out, int32_t n_threads, int32_t *threads_used) {
    return guarded("dkv_cpu_attention_pages", [&] {
        return dkv_cpu_attention_pages_body(pages, max_pages, shape, batch, q, k_new, v_new, ctx_lens, out,
                                            n_threads, threads_used);
    });
}

static dkv_status dkv_cpu_stream_read_body(const void *host_ptr, uint64_t bytes, int32_t n_threads,
                                           uint64_t *checksum) {
    if (!host_ptr || bytes % 64 || n_threads < 1 || n_threads > 1024)
        return fail(DKV_E_INVALID_ARG, "dkv_cpu_stream_read: null pointer, bytes not a multiple of 64, or "
                                       "n_threads outside [1, 1024]");
    const uint64_t sum = dkv::cpu_stream_read(host_ptr, bytes, n_threads);
    if (checksum) *checksum = sum;
    return DKV_OK;
}

dkv_status dkv_cpu_stream_read(const void *host_ptr, uint64_t bytes, int32_t n_threads, uint64_t *checksum) {
    return guarded("dkv_cpu_stream_read",
                   [&] { return dkv_cpu_stream_read_body(host_ptr, bytes, n_threads, checksum); });
}

static dkv_status step_impl(dkv_layout *L, int32_t layer, const uint16_t *q_in, const uint16_t *W,
                            const int32_t *ctx_lens, void *out, int out_f32, dkv_stream_t stream,
                            const char *who, char *scratch = nullptr, size_t scratch_capacity = 0) {
    if (!L || !live(L)) return fail(DKV_E_INVALID_ARG, "%s: null or freed layout", who);
    if (layer < 0 || layer >= L->shape.n_layers)
        return fail(DKV_E_INVALID_ARG, "%s: layer %d out of range", who, layer);
    if (!q_in || !W || !ctx_lens || !out) return fail(DKV_E_INVALID_ARG, "%s: null pointer argument", who);
    if (((uintptr_t)q_in | (uintptr_t)W) & 15u)
        return fail(DKV_E_INVALID_ARG, "%s: q_in and W_qkv must be 16-byte aligned", who);
    if (((uintptr_t)ctx_lens & 3u) || ((uintptr_t)out & (out_f32 ? 3u : 1u)))
        return fail(DKV_E_INVALID_ARG, "%s: misaligned ctx_lens or attn_out", who);
    const dkv_shape *s = &L->shape;
    dkv::StepArgs a{};
    a.batch = L->batch;
    a.hidden = s->hidden;
    a.n_q_heads = s->n_q_heads;
    a.n_kv_heads = s->n_kv_heads;
    a.head_dim = s->head_dim;
    a.n_qkv = (s->n_q_heads + 2 * s->n_kv_heads) * s->head_dim;
    a.max_pages = L->max_pages;
    a.split_tokens = L->split_tokens;
    a.split_variant = L->split_variant;
    a.split_waves = L->split_waves;
    a.lds_ring = L->lds_ring;
    a.lds_poison = L->lds_poison;
    a.proj_mfma_min_batch = L->proj_mfma_min_batch;
    a.proj_splitk_min_batch = L->proj_splitk_min_batch;
    a.proj_ranges = L->proj_ranges;
    a.max_splits = L->max_splits;
    a.part_slots = L->max_splits + 1;
    a.item_slots = L->item_slots;
    a.qscale = (float)(1.4426950408889634074 / std::sqrt((double)s->head_dim));
    a.page_table = L->d_page_table + (size_t)layer * L->batch * L->max_pages;
    a.capacity = L->d_capacity;
    a.x = q_in;
    a.w = W;
    a.ctx_lens = ctx_lens;
    a.out = out;
    a.out_f32 = out_f32;
    if (scratch && L->scratch.total > scratch_capacity)
        return fail(DKV_E_CAPACITY, "%s: this layout's step needs %zu bytes of scratch, more than the %zu available",
                    who, L->scratch.total, scratch_capacity);
    dkv::carve_scratch(a, scratch ? scratch : L->d_scratch, L->scratch);
    a.status = L->d_status;
    hipEvent_t *ev = nullptr;
    if (!L->timing_events.empty() && (size_t)(L->timing_recorded + 1) * kTimingEvents <= L->timing_events.size())
        ev = &L->timing_events[(size_t)L->timing_recorded++ * kTimingEvents];
    hipError_t e = dkv::launch_decode_step(a, reinterpret_cast<hipStream_t>(stream), ev, L->timing_mode == 2);
    if (e != hipSuccess) return hip_fail(e, who);
    return DKV_OK;
}

dkv_status decode_step(dkv_layout *L, int32_t layer, const uint16_t *q_in, const uint16_t *W_qkv,
                       const int32_t *ctx_lens, uint16_t *attn_out, dkv_stream_t stream) {
    return step_impl(L, layer, q_in, W_qkv, ctx_lens, attn_out, 0, stream, "decode_step");
}

}  // extern "C"

dkv_status dkv::report_hip_error(hipError_t e, const char *what) { return hip_fail(e, what); }

dkv_status dkv::decode_step_on_scratch(dkv_layout *L, int32_t layer, const uint16_t *q_in, const uint16_t *W,
                                       const int32_t *ctx_lens, uint16_t *attn_out, dkv_stream_t stream,
                                       char *scratch, size_t capacity, const char *who) {
    if (!scratch) return fail(DKV_E_INVALID_ARG, "%s: no scratch", who);
    return step_impl(L, layer, q_in, W, ctx_lens, attn_out, 0, stream, who, scratch, capacity);
}

extern "C" {

dkv_status decode_step_f32(dkv_layout *L, int32_t layer, const uint16_t *q_in, const uint16_t *W_qkv,
                           const int32_t *ctx_lens, float *attn_out, dkv_stream_t stream) {
    return step_impl(L, layer, q_in, W_qkv, ctx_lens, attn_out, 1, stream, "decode_step_f32");
}

dkv_status kv_advance(dkv_layout *L, int32_t *ctx_lens, dkv_stream_t stream) {
    if (!L || !ctx_lens || !live(L)) return fail(DKV_E_INVALID_ARG, "kv_advance: null argument or freed layout");
    if ((uintptr_t)ctx_lens & 3u) return fail(DKV_E_INVALID_ARG, "kv_advance: misaligned ctx_lens");
    dkv::AdvanceArgs a{};
    a.batch = L->batch;
    a.n_layers = L->shape.n_layers;
    a.max_pages = L->max_pages;
    a.max_window = L->max_window;
    a.page_bytes = page_bytes_of(&L->shape);
    a.windowed = L->windowed;
    a.page_table = L->d_page_table;
    a.host_pages = L->d_host_pages;
    a.ring = L->d_ring;
    a.window = L->d_window;
    a.capacity = L->d_capacity;
    a.ctx_lens = ctx_lens;
    a.status = L->d_status;
    hipError_t e = dkv::launch_advance(a, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "kv_advance");
    return DKV_OK;
}

dkv_status kv_layout_check_status(dkv_layout *L) {
    if (!L || !live(L)) return fail(DKV_E_INVALID_ARG, "kv_layout_check_status: null or freed layout");
    HIP_TRY(hipDeviceSynchronize());
    uint32_t flag = 0;
    HIP_TRY(hipMemcpy(&flag, L->d_status, sizeof flag, hipMemcpyDeviceToHost));
    HIP_TRY(hipMemset(L->d_status, 0, sizeof flag));
    if (flag & 1u)
        return fail(DKV_E_CAPACITY, "decode_step: a ctx_lens entry was outside [0, capacity - 1]");
    return DKV_OK;
}

dkv_status kv_pool_copy(dkv_pool *dst, const dkv_pool *src, int64_t bytes, dkv_stream_t stream) {
    if (!dst || !src || !live(dst) || !live(src) || bytes < 0 || dst->page_bytes != src->page_bytes ||
        bytes > dst->n_pages * dst->page_bytes || bytes > src->n_pages * src->page_bytes)
        return fail(DKV_E_INVALID_ARG, "kv_pool_copy: null pool, page sizes differ or bytes out of range");
    if (bytes == 0) return DKV_OK;
    const void *from = src->tier == 0 ? (const void *)src->host_base : (const void *)src->dev_base;
    void *to = dst->tier == 0 ? (void *)dst->host_base : (void *)dst->dev_base;
    HIP_TRY(hipMemcpyAsync(to, from, (size_t)bytes, hipMemcpyDefault, reinterpret_cast<hipStream_t>(stream)));
    return DKV_OK;
}

dkv_status dkv_host_buffer_alloc(uint64_t bytes, uint32_t flags, void **host_ptr, void **device_ptr) {
    if (!bytes || !host_ptr || !device_ptr || flags > DKV_HOST_NONCOHERENT)
        return fail(DKV_E_INVALID_ARG, "dkv_host_buffer_alloc: bad size, flags or null output");
    void *h = nullptr, *d = nullptr;
    const unsigned hflags = hipHostMallocMapped | hipHostMallocPortable |
                            (flags == DKV_HOST_NONCOHERENT ? hipHostMallocNonCoherent : hipHostMallocCoherent);
    hipError_t e = hipHostMalloc(&h, (size_t)bytes, hflags);
    if (e != hipSuccess || !h) {
        (void)hipGetLastError();
        return fail(DKV_E_OUT_OF_MEMORY, "dkv_host_buffer_alloc: hipHostMalloc of %llu bytes failed: %s",
                    (unsigned long long)bytes, hipGetErrorString(e));
    }
    e = hipHostGetDevicePointer(&d, h, 0);
    if (e != hipSuccess || !d) {
        (void)hipHostFree(h);
        return hip_fail(e, "dkv_host_buffer_alloc: hipHostGetDevicePointer");
    }
    *host_ptr = h;
    *device_ptr = d;
    return DKV_OK;
}

dkv_status dkv_host_buffer_free(void *host_ptr) {
    if (!host_ptr) return DKV_OK;
    HIP_TRY(hipHostFree(host_ptr));
    return DKV_OK;
}

dkv_status dkv_copy(void *dst, const void *src, uint64_t bytes, dkv_stream_t stream) {
    if (!dst || !src) return fail(DKV_E_INVALID_ARG, "dkv_copy: null pointer");
    if (!bytes) return DKV_OK;
    HIP_TRY(hipMemcpyAsync(dst, src, (size_t)bytes, hipMemcpyDefault, reinterpret_cast<hipStream_t>(stream)));
    return DKV_OK;
}

dkv_status dkv_gemm_bf16_nt(const uint16_t *A, const uint16_t *B, float *C, int32_t M, int32_t N, int32_t K,
                            int32_t tile_order, dkv_stream_t stream) {
    if (!A || !B || !C || M <= 0 || N <= 0 || K <= 0 || M % 128 || N % 128 || K % 64 ||
        (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C) & 15u) || (tile_order != 0 && tile_order != 1) ||
        (tile_order == 1 && (N / 128) % 8 != 0))
        return fail(DKV_E_INVALID_ARG,
                    "dkv_gemm_bf16_nt: need M, N multiples of 128, K of 64, aligned pointers, tile_order 0/1 "
                    "(1: N/128 a multiple of 8)");
    hipError_t e = dkv::launch_gemm_nt(A, B, C, M, N, K, tile_order == 1, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dkv_gemm_bf16_nt");
    return DKV_OK;
}

uint64_t dkv_gemm_bstationary_workspace_bytes(int32_t M, int32_t N, int32_t K) {
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    return dkv::gemm_bstationary_workspace_bytes(M, N, K);
}

dkv_status dkv_gemm_bf16_nt_bstationary(const uint16_t *A, const uint16_t *B, float *C, int32_t M, int32_t N,
                                        int32_t K, float *workspace, uint64_t workspace_bytes,
                                        dkv_stream_t stream) {
    if (!A || !B || !C || !workspace || M <= 0 || N <= 0 || K <= 0 || M % 64 || N % 128 || K % 512 ||
        (((uintptr_t)A | (uintptr_t)B | (uintptr_t)C | (uintptr_t)workspace) & 15u))
        return fail(DKV_E_INVALID_ARG,
                    "dkv_gemm_bf16_nt_bstationary: need M a multiple of 64, N of 128, K of 512, aligned pointers");
    if (workspace_bytes < dkv::gemm_bstationary_workspace_bytes(M, N, K))
        return fail(DKV_E_CAPACITY, "dkv_gemm_bf16_nt_bstationary: workspace of %llu bytes, %llu needed",
                    (unsigned long long)workspace_bytes,
                    (unsigned long long)dkv::gemm_bstationary_workspace_bytes(M, N, K));
    hipError_t e = dkv::launch_gemm_nt_bstationary(A, B, C, M, N, K, workspace, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "dkv_gemm_bf16_nt_bstationary");
    return DKV_OK;
}

static dkv_status dkv_probe_stream_read_body(const void *ptr, uint64_t bytes, int32_t n_regions, int32_t grid,
                                             int32_t unroll, int32_t reps, float *ms_median) {
    // unroll < 0 selects nontemporal loads with |unroll| in flight
    const bool nt = unroll < 0;
    if (nt) unroll = -unroll;
    if (!ptr || !ms_median || bytes == 0 || bytes % 16 || ((uintptr_t)ptr & 15u) || grid <= 0 || reps <= 0 ||
        n_regions <= 0 || !(unroll == 1 || unroll == 2 || unroll == 4 || unroll == 8))
        return fail(DKV_E_INVALID_ARG, "dkv_probe_stream_read: bad argument");
    auto region = [&](int r) { return static_cast<const char *>(ptr) + (size_t)(r % n_regions) * bytes; };
    hipStream_t st;
    HIP_TRY(hipStreamCreate(&st));
    uint32_t *sink = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    std::vector<float> ts;
    hipError_t e = hipMalloc(&sink, 64);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = dkv::launch_stream_read(region(n_regions - 1), bytes, grid, unroll, nt, sink, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    for (int r = 0; r < reps && e == hipSuccess; ++r) {
        e = hipEventRecord(e0, st);
        if (e == hipSuccess) e = dkv::launch_stream_read(region(r), bytes, grid, unroll, nt, sink, st);
        if (e == hipSuccess) e = hipEventRecord(e1, st);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        ts.push_back(ms);
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipFree(sink);
    (void)hipStreamDestroy(st);
    if (e != hipSuccess) return hip_fail(e, "dkv_probe_stream_read");
    std::sort(ts.begin(), ts.end());
    *ms_median = ts[ts.size() / 2];
    return DKV_OK;
}

dkv_status dkv_probe_stream_read(const void *ptr, uint64_t bytes, int32_t grid, int32_t unroll, int32_t reps,
                                 float *ms_median) {
    return guarded("dkv_probe_stream_read",
                   [&] { return dkv_probe_stream_read_body(ptr, bytes, 1, grid, unroll, reps, ms_median); });
}

static dkv_status dkv_probe_page_read_body(const void *ptr, uint64_t bytes, int32_t page_bytes, int32_t runs,
                                          int32_t waves, int32_t skew, int32_t reps, float *ms_median) {
    if (!ptr || !ms_median || ((uintptr_t)ptr & 15u) || page_bytes <= 0 || runs <= 0 || waves <= 0 ||
        reps <= 0 || waves % runs || page_bytes % (runs * 1024) || bytes % (uint64_t)page_bytes)
        return fail(DKV_E_INVALID_ARG, "dkv_probe_page_read: bad argument");
    const int run16 = page_bytes / runs / 1024;
    const uint64_t pages = bytes / (uint64_t)page_bytes;
    const int items = waves / runs;
    if ((run16 != 4 && run16 != 8) || pages % (uint64_t)items || pages / (uint64_t)items > (uint64_t)INT32_MAX)
        return fail(DKV_E_INVALID_ARG, "dkv_probe_page_read: runs must be 4 or 8 KiB and the pages divide evenly");
    const int ppi = (int)(pages / (uint64_t)items);
    hipStream_t st;
    HIP_TRY(hipStreamCreate(&st));
    uint32_t *sink = nullptr;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    std::vector<float> ts;
    hipError_t e = hipMalloc(&sink, 64);
    if (e == hipSuccess) e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) e = dkv::launch_page_read(ptr, ppi, page_bytes, runs, waves, skew, sink, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    for (int r = 0; r < reps && e == hipSuccess; ++r) {
        e = hipEventRecord(e0, st);
        if (e == hipSuccess) e = dkv::launch_page_read(ptr, ppi, page_bytes, runs, waves, skew, sink, st);
        if (e == hipSuccess) e = hipEventRecord(e1, st);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        ts.push_back(ms);
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    (void)hipFree(sink);
    (void)hipStreamDestroy(st);
    if (e != hipSuccess) return hip_fail(e, "dkv_probe_page_read");
    std::sort(ts.begin(), ts.end());
    *ms_median = ts[ts.size() / 2];
    return DKV_OK;
}

dkv_status dkv_probe_page_read(const void *ptr, uint64_t bytes, int32_t page_bytes, int32_t runs, int32_t waves,
                               int32_t skew, int32_t reps, float *ms_median) {
    return guarded("dkv_probe_page_read", [&] {
        return dkv_probe_page_read_body(ptr, bytes, page_bytes, runs, waves, skew, reps, ms_median);
    });
}

dkv_status dkv_probe_stream_read_cycled(const void *ptr, uint64_t bytes, int32_t n_regions, int32_t grid,
                                        int32_t unroll, int32_t reps, float *ms_median) {
    return guarded("dkv_probe_stream_read_cycled", [&] {
        return dkv_probe_stream_read_body(ptr, bytes, n_regions, grid, unroll, reps, ms_median);
    });
}

}  // extern "C"
