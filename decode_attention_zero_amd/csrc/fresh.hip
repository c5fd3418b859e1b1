// The new token of one decode step on gfx950: its query, key and value are
// formed from the projection's fp32 sums, the key and value are consumed on
// chip and written back once.
//
// One workgroup of four wavefronts per (sequence b, KV head g):
//  * adds the projection slabs of the group's rows (G query heads, then the
//    K and V head) in range order; the queries are scaled by log2(e)/sqrt(d)
//    (scores in log2 units) and stored in fp32 for the split kernel; k_new
//    and v_new are rounded once to bf16 (nearest even) and kept in LDS;
//  * scores the fresh token against each of the G query heads from LDS and
//    writes its one-token softmax state (s_new, 1, v_new) into the partial
//    slot after the sequence's splits, where the combine merges it like any
//    split;
//  * writes the bf16 K and V rows once into slot ctx_lens[b] of the
//    sequence's pages, host or HBM (the "storer" role).
// The new K/V thus exist only in this kernel's registers and LDS before the
// single write-back: the fusion of the projection that generates them with
// the attention that consumes them, in the core-method section of the
// DirectKV digest ("长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）") and in
// "KV Cache 内存层级" overview, 2.1 去搬运：DirectKV (fresh K/V consumed from
// shared memory instead of written out and read back). The projection itself
// stays a separate launch spread over hundreds of workgroups, which is what
// reading W at HBM speed takes; what crosses between the two launches is fp32
// partial sums, not K/V.
//
// The step's other bookkeeping happens here too: the range check of
// ctx_lens, the list of the split kernel's work items (built by one extra
// workgroup, the launch's first) and the reset of its work queue.
#include "device_common.h"

namespace dkv {
namespace {

constexpr int kFreshWaves = 4;
constexpr int kFreshThreads = 64 * kFreshWaves;

// The step's item list: (sequence, split) for every split that holds tokens,
// sequence-major, then the count in entry 0. One workgroup walks the batch
// in chunks of kFreshThreads sequences: each thread takes one sequence's
// split count (the next chunk's is loaded while this chunk is scanned), an
// exclusive scan over the workgroup places each sequence's run of entries,
// and the chunk's entries are then written by all threads together,
// contiguously (an entry finds its sequence by a binary search over the
// chunk's run ends in LDS), so that a sequence with many splits does not
// serialise them on one thread. The batch is read once: linear in its size.
__device__ void build_item_list(const StepArgs &a) {
    __shared__ int s_wave[kFreshWaves];
    __shared__ int s_end[kFreshThreads];     // end of each sequence's run within the chunk
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int base = 0;
    int next = tid < a.batch ? splits_of(a, tid) : 0;
    for (int c0 = 0; c0 < a.batch; c0 += kFreshThreads) {
        const int mine = next;
        next = c0 + kFreshThreads + tid < a.batch ? splits_of(a, c0 + kFreshThreads + tid) : 0;
        int incl = mine;                      // inclusive prefix within the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off);
            if (lane >= off) incl += t;
        }
        const int wave_total = wave_sum_int(mine);
        if (lane == 0) s_wave[wave] = wave_total;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kFreshWaves; ++w) {
            before += w < wave ? s_wave[w] : 0;
            total += s_wave[w];
        }
        s_end[tid] = before + incl;
        __syncthreads();
        for (int e = tid; e < total; e += kFreshThreads) {
            int lo = 0, hi = kFreshThreads - 1;   // the first run whose end is past e
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_end[mid] > e) hi = mid;
                else lo = mid + 1;
            }
            const int s = e - (lo ? s_end[lo - 1] : 0);
            a.item_list[1 + base + e] = ((uint32_t)(c0 + lo) << 16) | (uint32_t)s;
        }
        base += total;
        __syncthreads();                      // s_wave and s_end are rewritten by the next chunk
    }
    if (tid == 0) a.item_list[0] = (uint32_t)base;
}

// KS slabs (1, 2, 4 or 8). Each thread owns up to RPT of the group's rows and
// issues all RPT x KS loads of its slabs before it adds them, each row in
// range order (the same sums, in the same order, as a plain loop).
template <int D, int G, int KS>
__global__ __launch_bounds__(kFreshThreads) void fresh_token_kernel(StepArgs a) {
    constexpr int DPL = D / 64;        // dims per lane
    constexpr int NR = (G + 2) * D;    // the group's rows: G query heads, K, V
    constexpr int RPT = (NR + kFreshThreads - 1) / kFreshThreads;
    reset_items(a);
    if (blockIdx.x == 0) {                    // the extra workgroup: the item list
        build_item_list(a);
        return;
    }
    const int b = (blockIdx.x - 1) / a.n_kv_heads;
    const int g = (blockIdx.x - 1) - b * a.n_kv_heads;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    __shared__ float s_q[G][D];
    __shared__ float s_kv[2][D];               // rounded K and V, as fp32 (exact)
    __shared__ __attribute__((aligned(16))) uint16_t s_kvb[2][D];   // their bf16 bits

    const int L = a.ctx_lens[b];
    const bool in_range = L >= 0 && L < a.capacity[b];
    if (g == 0 && tid == 0) check_context_range(a, b);

    const size_t slab = (size_t)a.batch * a.n_qkv;
    const float *yb = a.proj_part + (size_t)b * a.n_qkv;
    const int krow = a.n_q_heads * D + g * D;
    const int vrow = krow + a.n_kv_heads * D;
    float *qout = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * D;
    float part[RPT][KS];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = tid + j * kFreshThreads;
        if (r < NR) {
            const int n = r < G * D ? g * G * D + r : r < (G + 1) * D ? krow + (r - G * D) : vrow + (r - (G + 1) * D);
#pragma unroll
            for (int k = 0; k < KS; ++k) part[j][k] = yb[(size_t)k * slab + n];
        }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int r = tid + j * kFreshThreads;
        if (r >= NR) break;
        float y = part[j][0];
#pragma unroll
        for (int k = 1; k < KS; ++k) y += part[j][k];
        if (r < G * D) {
            const float qv = y * a.qscale;
            s_q[r / D][r % D] = qv;
            qout[r] = qv;
        } else {
            const int c = (r - G * D) / D, i = (r - G * D) % D;
            const uint16_t h = f32_to_bf16(y);
            s_kvb[c][i] = h;
            s_kv[c][i] = __uint_as_float((uint32_t)h << 16);
        }
    }
    __syncthreads();
    if (!in_range) return;

    // One-token state of each query head: m = s_new, l = 1, o = v_new.
    const int slot_s = (L + a.split_tokens - 1) / a.split_tokens;
    for (int h = wave; h < G; h += kFreshWaves) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) part = fmaf(s_q[h][lane * DPL + e], s_kv[0][lane * DPL + e], part);
        const float s_new = wave_sum(part);
        const size_t slot = ((size_t)b * a.n_q_heads + (size_t)g * G + h) * a.part_slots + slot_s;
        float *po = a.part_o + slot * D + lane * DPL;
#pragma unroll
        for (int e = 0; e < DPL; ++e) po[e] = s_kv[1][lane * DPL + e];
        if (lane == 0) a.part_ml[slot] = make_float2(s_new, 1.0f);
    }

    // The single write-back: lanes 0-31 of the last wave store the K row,
    // lanes 32-63 the V row.
    if (wave == kFreshWaves - 1) {
        const int c = lane >> 5;
        const int li = lane & 31;
        char *page = reinterpret_cast<char *>(a.page_table[(size_t)b * a.max_pages + L / kPageTokens]);
        char *dst = page + ((size_t)((g * 2 + c) * kPageTokens + (L % kPageTokens)) * D) * 2;
        const char *src = reinterpret_cast<const char *>(s_kvb[c]);
        constexpr int BPL = D * 2 / 32;    // bytes per lane
        if constexpr (BPL == 8) {
            *reinterpret_cast<uint2 *>(dst + li * 8) = *reinterpret_cast<const uint2 *>(src + li * 8);
        } else {
            *reinterpret_cast<uint32_t *>(dst + li * 4) = *reinterpret_cast<const uint32_t *>(src + li * 4);
        }
    }
}

template <int D, int G>
void launch(const StepArgs &a, int ranges, hipStream_t st) {
    const dim3 grid(1 + a.batch * a.n_kv_heads);     // workgroup 0 builds the item list
    switch (ranges) {
        case 1: fresh_token_kernel<D, G, 1><<<grid, kFreshThreads, 0, st>>>(a); break;
        case 2: fresh_token_kernel<D, G, 2><<<grid, kFreshThreads, 0, st>>>(a); break;
        case 4: fresh_token_kernel<D, G, 4><<<grid, kFreshThreads, 0, st>>>(a); break;
        default: fresh_token_kernel<D, G, 8><<<grid, kFreshThreads, 0, st>>>(a); break;
    }
}

}  // namespace

hipError_t launch_fresh(const StepArgs &a, int ranges, hipStream_t st) {
    const int G = a.n_q_heads / a.n_kv_heads;
    if (ranges != 1 && ranges != 2 && ranges != 4 && ranges != 8) return hipErrorInvalidValue;
    if (a.head_dim == 128) {
        switch (G) {
            case 1: launch<128, 1>(a, ranges, st); break;
            case 2: launch<128, 2>(a, ranges, st); break;
            case 4: launch<128, 4>(a, ranges, st); break;
            case 8: launch<128, 8>(a, ranges, st); break;
            default: return hipErrorInvalidValue;
        }
    } else if (a.head_dim == 64) {
        switch (G) {
            case 1: launch<64, 1>(a, ranges, st); break;
            case 2: launch<64, 2>(a, ranges, st); break;
            case 4: launch<64, 4>(a, ranges, st); break;
            case 8: launch<64, 8>(a, ranges, st); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dkv
