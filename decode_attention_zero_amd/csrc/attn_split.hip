// Split attention of one zero-copy decode step on gfx950 (MI355X): one
// wavefront per work item (sequence b, KV head g, token split s) streams the
// split's KV pages in place -- host pages over the host link, HBM pages from
// HBM, chosen only by the page's address -- and keeps an online-softmax state
// for the G query heads that share the KV head, so each remote byte is read
// once for all of them. Writes an unnormalised partial (m, l, o) per query
// head and split. Two arithmetic forms share the page streaming: VALU with
// DPP row sums (SplitState; groups of 1 and 2, and on request) and the
// matrix cores (MfmaState; the default from groups of 4).
//
// Method (pages): "长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）" (DirectKV
// digest), 核心方法: the attention kernel reads CPU-resident KV directly, with a
// layout arranged for coalesced remote reads. The split/merge of the softmax
// state is the standard flash-decoding decomposition (not on the pages); the
// split boundaries depend only on token indices, never on where a page lives,
// so host and HBM placements give bit-identical results.
#include <algorithm>

#include "device_common.h"

namespace dkv {
namespace {

// VALU split attention. Work item (KV head g, split s, sequence b): in the
// one-wavefront-per-item launches g = blockIdx.x and (b, s) is entry
// blockIdx.y + gridDim.y * blockIdx.z of the step's item list (XCD-aware
// order, see launch).
//
// Lane mapping inside a page run (K tile then V tile, each [16 tok][D] bf16):
// wave load j reads bytes [j*1024, (j+1)*1024) of a tile, lane l the 16 bytes
// at l*16, i.e. token j*TPL + l/LPT, dims 8*(l%LPT) .. +7. Every wave load is
// one fully used, contiguous 1 KiB -- the coalesced remote access the layout is
// arranged for. A token's score is summed over its LPT lanes with DPP; each
// group of lanes holding the same token slot across loads (a "row") keeps its
// own online-softmax state, merged across rows at the end of the item.
//
// Pages are double-buffered in registers (ping-pong, so no copies): the next
// page's loads are in flight while the current one is computed. Full pages
// take a mask-free path; only the split's last page can be partial.
//
// WPI wavefronts share a work item by splitting each tile's wave loads (WPI
// = 2: wave 0 takes tokens 0-7 of every page, wave 1 tokens 8-15), so every
// byte is still read once; their softmax states are merged through LDS at
// the end of the item, in a fixed order. Used for groups of 8 query heads,
// whose single-wave state would need 367 registers (one wave per SIMD); even
// so that form spills, which is why groups of 8 run on the matrix cores.
template <int D, int G, int WPI = 1>
struct SplitState {
    static constexpr int LPT = D / 8;               // lanes per token
    static constexpr int TPL = 64 / LPT;            // tokens per wave load
    static constexpr int NLD = kPageTokens / TPL;   // wave loads per 16-token tile
    static constexpr int NLDW = NLD / WPI;          // of those, loads per wavefront
    static constexpr int TILE = kPageTokens * D * 2;
    static constexpr int RUN = 2 * TILE;
    static_assert(NLD % WPI == 0, "tile loads must split evenly over the wavefronts");

    float q[G][8];
    float m[G], l[G], acc[G][8];
    int sub;                       // page token of this lane in the wave's first load

    // `run` points at this lane's 16 bytes of the wave's first load of the run.
    __device__ __forceinline__ void load(const char *run, uint4 (&kr)[NLDW], uint4 (&vr)[NLDW]) const {
#pragma unroll
        for (int j = 0; j < NLDW; ++j) kr[j] = load_stream(run + j * 1024);
#pragma unroll
        for (int j = 0; j < NLDW; ++j) vr[j] = load_stream(run + TILE + j * 1024);
    }

    // One page. PARTIAL: only the first n_valid tokens of the page count;
    // `sub` is the page token this lane holds in the wave's first load.
    template <bool PARTIAL>
    __device__ __forceinline__ void page(const uint4 (&kr)[NLDW], const uint4 (&vr)[NLDW], int sub,
                                         int n_valid) {
        constexpr int NLD = NLDW;
        float sc[NLD][G];
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            float kf[8];
            unpack8(kr[j], kf);
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float d0 = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) d0 = fmaf(q[h][e], kf[e], d0);
                sc[j][h] = token_sum<LPT>(d0);
            }
        }
        bool valid[NLD];
#pragma unroll
        for (int j = 0; j < NLD; ++j) valid[j] = !PARTIAL || (j * TPL + sub < n_valid);

        // New running max per head; the rescale runs only when some row's max
        // grew (otherwise its factor would be exactly 1).
        float mx[G];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            mx[h] = m[h];
#pragma unroll
            for (int j = 0; j < NLD; ++j)
                if (valid[j]) mx[h] = fmaxf(mx[h], sc[j][h]);
            grow |= mx[h] > m[h];
        }
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float alpha = (mx[h] == m[h]) ? 1.0f : rescale(m[h], mx[h]);
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
                m[h] = mx[h];
            }
        }

#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            float vf[8];
            unpack8(vr[j], vf);
            if (PARTIAL && !valid[j]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) vf[e] = 0.0f;   // stale slots may hold any bits
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float p = fast_exp2(sc[j][h] - m[h]);
                if (PARTIAL && !valid[j]) p = 0.0f;
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
            }
        }
    }

    template <bool PARTIAL>
    __device__ __forceinline__ void page(const uint4 (&kr)[NLDW], const uint4 (&vr)[NLDW], int n_valid) {
        page<PARTIAL>(kr, vr, sub, n_valid);
    }

    // Query rows of heads h0 .. h0 + G - 1 (this lane's 8 dims) and an empty
    // softmax state.
    __device__ __forceinline__ void init(const StepArgs &a, int b, int h0, int dl) {
        const float *qb = a.q + ((size_t)b * a.n_q_heads + (size_t)h0) * D + dl * 8;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float4 lo = *reinterpret_cast<const float4 *>(qb + h * D);
            const float4 hi = *reinterpret_cast<const float4 *>(qb + h * D + 4);
            q[h][0] = lo.x; q[h][1] = lo.y; q[h][2] = lo.z; q[h][3] = lo.w;
            q[h][4] = hi.x; q[h][5] = hi.y; q[h][6] = hi.z; q[h][7] = hi.w;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            m[h] = kNegInf;
            l[h] = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;
        }
    }

    // Merges the row states (lanes l and l ^ off, off >= LPT) in a fixed order
    // and writes the partial (m, l, o) of heads h0 .. h0 + G - 1 for split s.
    __device__ __forceinline__ void finish(const StepArgs &a, int b, int h0, int s, int dl) {
        const bool row0 = (threadIdx.x & 63) < LPT;     // lanes of the wave's first row
#pragma unroll
        for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float mo = __shfl_xor(m[h], off);
                const float lo = __shfl_xor(l[h], off);
                const float M = fmaxf(m[h], mo);
                const float c1 = rescale(m[h], M);
                const float c2 = rescale(mo, M);
                l[h] = fmaf(l[h], c1, lo * c2);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ao = __shfl_xor(acc[h][e], off);
                    acc[h][e] = fmaf(acc[h][e], c1, ao * c2);
                }
                m[h] = M;
            }
        }
        if constexpr (WPI == 2) {
            // Wave 1 hands its merged state to wave 0 through LDS.
            __shared__ float xw[G][2 + LPT * 8];
            const int w = threadIdx.x >> 6;
            if (w == 1 && row0) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    if (dl == 0) {
                        xw[h][0] = m[h];
                        xw[h][1] = l[h];
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) xw[h][2 + dl * 8 + e] = acc[h][e];
                }
            }
            __syncthreads();
            if (w == 0) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float mo = xw[h][0];
                    const float lo = xw[h][1];
                    const float M = fmaxf(m[h], mo);
                    const float c1 = rescale(m[h], M);
                    const float c2 = rescale(mo, M);
                    l[h] = fmaf(l[h], c1, lo * c2);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(acc[h][e], c1, xw[h][2 + dl * 8 + e] * c2);
                    m[h] = M;
                }
            }
            __syncthreads();     // the buffer is free again before the next item
            if (w != 0) return;
        }
        if (row0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const size_t slot = ((size_t)b * a.n_q_heads + (size_t)h0 + h) * a.part_slots + s;
                float *po = a.part_o + slot * D + dl * 8;
                *reinterpret_cast<float4 *>(po) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
                *reinterpret_cast<float4 *>(po + 4) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
                if (dl == 0) a.part_ml[slot] = make_float2(m[h], l[h]);
            }
        }
    }
};

// Streams the pages holding tokens [t0, t1) of one sequence through state
// `st`: page runs at pt[p] + run_off are double-buffered in registers
// (ping-pong, so no copies), the next page's loads in flight while the
// current one is computed. Full pages take a mask-free path; only the last
// page can be partial. (Reading the item's page addresses once, one per
// lane, and broadcasting them with readlane avoids the page-table load
// between page loads, but measured slower on MI355X: 1 GiB in HBM at group
// 4, 0.176 vs 0.169 ms; on the host link it needs fewer looping wavefronts
// to stay at the ceiling.)
template <class S>
__device__ __forceinline__ void stream_pages(S &st, const uint64_t *pt, size_t run_off, int t0, int t1) {
    constexpr int NLD = S::NLDW;
    const int p0 = t0 / kPageTokens;
    const int p1 = (t1 + kPageTokens - 1) / kPageTokens;   // pages [p0, p1)
    const int pf = t1 / kPageTokens;                        // pages [p0, pf) are full
    auto run_of = [&](int p) { return reinterpret_cast<const char *>(pt[p]) + run_off; };
    uint4 ka[NLD], va[NLD], kb[NLD], vb[NLD];
    int p = p0;
    st.load(run_of(p), ka, va);
    while (p + 1 < pf) {                 // pages p (in a) and p + 1 are full
        st.load(run_of(p + 1), kb, vb);
        st.template page<false>(ka, va, kPageTokens);
        if (p + 2 < p1) st.load(run_of(p + 2), ka, va);
        st.template page<false>(kb, vb, kPageTokens);
        p += 2;
    }
    if (p < pf) {                        // one last full page (in a), maybe a partial one after
        if (p + 1 < p1) st.load(run_of(p + 1), kb, vb);
        st.template page<false>(ka, va, kPageTokens);
        if (p + 1 < p1) st.template page<true>(kb, vb, t1 - (p + 1) * kPageTokens);
    } else if (p < p1) {                 // the partial page (in a)
        st.template page<true>(ka, va, t1 - p * kPageTokens);
    }
}

// One work item: split s of sequence b, KV head g, query heads h0 .. h0 + G - 1,
// on the WPI wavefronts of the workgroup.
template <int D, int G, int WPI>
__device__ __forceinline__ void split_item(const StepArgs &a, int s, int g, int h0, int b) {
    using S = SplitState<D, G, WPI>;
    constexpr int LPT = S::LPT;

    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) return;
    const int t0 = s * a.split_tokens;
    if (t0 >= L) return;
    const int t1 = min(t0 + a.split_tokens, L);

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int dl = lane % LPT;

    S st;
    st.init(a, b, h0, dl);
    st.sub = lane / LPT + w * S::NLDW * S::TPL;
    const size_t run_off = (size_t)g * S::RUN + (size_t)w * S::NLDW * 1024 + (size_t)lane * 16;
    stream_pages(st, a.page_table + (size_t)b * a.max_pages, run_off, t0, t1);
    st.finish(a, b, h0, s, dl);
}

// ------------------------------------------------------------------------------
// Matrix-core arithmetic for a group of query heads. Per page, the group's
// scores are one dense product S = K Q^T ([16 tokens] x [d] x [G heads]) and
// its output update one product O^T += V^T P^T, so they run on
// v_mfma_f32_16x16x32_bf16 and v_mfma_f32_16x16x16_bf16; on VALU the same
// work costs ~500 instructions per 8 KiB page run at G = 4 and ~830 at G = 8,
// more than a CU issues in the time HBM delivers the run. The page loads are
// the same contiguous 1 KiB wave loads as above; each run is then staged in
// the wavefront's own LDS buffer to reach the MFMA operand layouts. Staged
// token rows are padded by 16 bytes: that keeps the row-wise K reads, the
// column-wise V reads and the staging writes free of bank conflicts, and
// every lane's LDS addresses a single base plus constant offsets.
//
// Precision: the matrix cores take bf16 operands. K and V are bf16 already;
// the fp32 queries and probabilities are each split into two bf16 terms, hi =
// bf16(x) and lo = bf16(x - hi), which represent x to ~2^-17 relative, and
// both terms go through the same product: the 16 MFMA columns hold the hi
// terms of heads 0 .. G-1 in columns 0 .. G-1 and their lo terms mirrored in
// columns 15 .. 16-G, and a row-mirror DPP add forms hi + lo. Products of
// bf16 terms are exact in fp32 and accumulate in fp32.
//
// Lane l (column j = l % 16, row group q = l / 16) owns, for head min(j,
// 15-j): the scores of page tokens 4q .. 4q+3, the output dims 16n + 4q ..
// +3 of every 16-dim block n, and a running max and partial sum. The running
// max is common to the four row groups (the PV product sums over all 16
// tokens), so each page's max is reduced across them. Every column's
// arithmetic depends only on its own head, so the per-query-head comparator
// (one head per item) gives the same bits as the grouped kernel.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));   // round to nearest even
}

// s_waitcnt lgkmcnt(0) only (vmcnt and expcnt left unconstrained).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

template <int D, int G>
struct MfmaState {
    static constexpr int LPT = D / 8;               // 16-byte chunks per token row
    static constexpr int TPL = 64 / LPT;            // tokens per wave load
    static constexpr int NLDW = kPageTokens / TPL;  // wave loads per 16-token tile
    static constexpr int TILE = kPageTokens * D * 2;
    static constexpr int RUN = 2 * TILE;
    static constexpr int ROW = D * 2 + 16;          // staged token row (padded)
    static constexpr int STILE = kPageTokens * ROW; // staged K or V tile
    static constexpr int STAGE = 2 * STILE;         // LDS bytes per wavefront
    static constexpr int NKB = D / 32;              // 32-dim blocks of the score product
    static constexpr int NDB = D / 16;              // 16-dim blocks of the output
    static_assert(G >= 1 && G <= 8, "hi and lo terms of the group fill at most 16 columns");

    char *lds;            // this wavefront's staging buffer
    int lane, col, kq;
    int x16, x32;         // ds_bpermute byte addresses of lanes lane ^ 16 and lane ^ 32
    bf16x8 qop[NKB];      // B operand of the score product: this lane's column, dims 32c + 8kq ..
    f32x4 o[NDB];         // O^T[16n + 4kq + r][col]
    float m, l;


    __device__ __forceinline__ void load(const char *run, uint4 (&kr)[NLDW], uint4 (&vr)[NLDW]) const {
#pragma unroll
        for (int j = 0; j < NLDW; ++j) kr[j] = load_stream(run + j * 1024);
#pragma unroll
        for (int j = 0; j < NLDW; ++j) vr[j] = load_stream(run + TILE + j * 1024);
    }

    __device__ __forceinline__ void init(const StepArgs &a, int b, int h0) {
        lane = threadIdx.x & 63;
        col = lane & 15;
        kq = lane >> 4;
        x16 = (lane ^ 16) << 2;
        x32 = (lane ^ 32) << 2;
        const int head = col < G ? col : (col >= 16 - G ? 15 - col : -1);
#pragma unroll
        for (int c = 0; c < NKB; ++c) {
            uint32_t w[4] = {0u, 0u, 0u, 0u};
            if (head >= 0) {
                const float *qp = a.q + ((size_t)b * a.n_q_heads + (size_t)(h0 + head)) * D + 32 * c + 8 * kq;
                const float4 f0 = *reinterpret_cast<const float4 *>(qp);
                const float4 f1 = *reinterpret_cast<const float4 *>(qp + 4);
                const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint16_t t = bf16_bits(f[e]);
                    if (col >= 8) t = bf16_bits(f[e] - __uint_as_float((uint32_t)t << 16));
                    w[e >> 1] |= (uint32_t)t << (16 * (e & 1));
                }
            }
            qop[c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
        m = kNegInf;
        l = 0.0f;
#pragma unroll
        for (int n = 0; n < NDB; ++n) o[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }

    template <bool PARTIAL>
    __device__ __forceinline__ void page(const uint4 (&kr)[NLDW], const uint4 (&vr)[NLDW], int n_valid) {
        // Stage the run: lane l of wave load j holds token j*TPL + l/LPT, chunk l%LPT.
        char *wr = lds + (lane / LPT) * ROW + (lane % LPT) * 16;
#pragma unroll
        for (int j = 0; j < NLDW; ++j) {
            *reinterpret_cast<uint4 *>(wr + j * TPL * ROW) = kr[j];
            *reinterpret_cast<uint4 *>(wr + STILE + j * TPL * ROW) = vr[j];
        }
        wait_lds();
        asm volatile("" ::: "memory");
        compute<PARTIAL, false>(lds, lds + STILE, n_valid);
    }

    // Byte address of 16-byte chunk `chunk` of token row t of a tile in LDS:
    // padded rows of ROW bytes (the staging above), or with SWZ unpadded rows
    // of D * 2 bytes whose chunk c sits at chunk position c ^ (t & 15) (the
    // LDS ring's image, D = 128), which keeps 16 tokens' reads of the same
    // chunk on 16 different bank groups without padding.
    template <bool SWZ>
    __device__ __forceinline__ const char *chunk_at(const char *tile, int t, int chunk) const {
        if constexpr (SWZ) return tile + t * (D * 2) + ((chunk ^ (t & 15)) << 4);
        else return tile + t * ROW + (chunk << 4);
    }

    // One page from its K and V tiles in LDS.
    template <bool PARTIAL, bool SWZ>
    __device__ __forceinline__ void compute(const char *ktile, const char *vtile, int n_valid) {
        // S = K Q^T: A = K rows (token = col), B = the query terms.
        f32x4 sc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < NKB; ++c) {
            const uint4 kv = *reinterpret_cast<const uint4 *>(chunk_at<SWZ>(ktile, col, kq + 4 * c));
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kv), qop[c], sc, 0, 0, 0);
        }
        float sv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sv[r] = sc[r] + dpp<0x140>(sc[r]);                   // hi + lo (row mirror)
            if (PARTIAL && 4 * kq + r >= n_valid) sv[r] = kNegInf;
        }
        float pm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        pm = fmaxf(pm, __int_as_float(__builtin_amdgcn_ds_bpermute(x16, __float_as_int(pm))));
        pm = fmaxf(pm, __int_as_float(__builtin_amdgcn_ds_bpermute(x32, __float_as_int(pm))));
        const float mn = fmaxf(m, pm);
        if (__builtin_amdgcn_ballot_w64(mn > m) != 0) {
            const float alpha = (mn == m) ? 1.0f : rescale(m, mn);
            l *= alpha;
#pragma unroll
            for (int n = 0; n < NDB; ++n) o[n] *= alpha;
            m = mn;
        }
        uint16_t pb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(sv[r] - m);
            l += p;
            const uint16_t hi = bf16_bits(p);
            pb[r] = col < 8 ? hi : bf16_bits(p - __uint_as_float((uint32_t)hi << 16));
        }
        const s16x4 pop = {(short)pb[0], (short)pb[1], (short)pb[2], (short)pb[3]};

        // O^T += V^T P^T: A = V^T (dim = col, tokens 4kq .. 4kq+3), B = P^T; in
        // groups of four 16-dim blocks, so that only one group's V reads are
        // held in registers at a time. The A operand comes from one transposing
        // LDS read (ds_read_b64_tr_b16) per block: within each 16-lane group,
        // lane i receives element i % 4 of the 8-byte pieces addressed by lanes
        // i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 (measured on gfx950), so
        // lane j of row group kq addresses dims 16n + 4 (j % 4) .. +3 of token
        // 4kq + j / 4, and lane col gets dim 16n + col of tokens 4kq .. 4kq+3.
        // Lane col's 8-byte piece of block n: token 4kq + col/4, bytes
        // 32n + 8 (col % 4), i.e. chunk 2n + (col / 2) % 2, half col % 2.
        const int vt = 4 * kq + (col >> 2);
#pragma unroll
        for (int n0 = 0; n0 < NDB; n0 += 4) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int n = n0; n < n0 + 4; ++n) {
                const char *vp = chunk_at<SWZ>(vtile, vt, 2 * n + ((col >> 1) & 1)) + (col & 1) * 8;
                s16x4 vop = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)vp);
                if (PARTIAL) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        // Slots past the valid tokens may hold any bits (NaN times a
                        // zero weight would still be NaN).
                        if (4 * kq + r >= n_valid) vop[r] = 0;
                }
                o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pop, o[n], 0, 0, 0);
            }
        }
        asm volatile("" ::: "memory");   // the next run's staging stays behind these reads
    }

    // Sums the partial sums over the row groups and the hi/lo output columns,
    // and writes the partial (m, l, o) of heads h0 .. h0 + G - 1 for split s.
    __device__ __forceinline__ void finish(const StepArgs &a, int b, int h0, int s) {
        float lt = l + __shfl_xor(l, 16);
        lt = lt + __shfl_xor(lt, 32);
#pragma unroll
        for (int n = 0; n < NDB; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[n][r] += dpp<0x140>(o[n][r]);
        if (col < G) {
            const size_t slot = ((size_t)b * a.n_q_heads + (size_t)(h0 + col)) * a.part_slots + s;
            float *po = a.part_o + slot * D + 4 * kq;
#pragma unroll
            for (int n = 0; n < NDB; ++n)
                *reinterpret_cast<float4 *>(po + 16 * n) = make_float4(o[n][0], o[n][1], o[n][2], o[n][3]);
            if (kq == 0) a.part_ml[slot] = make_float2(m, lt);
        }
    }
};

template <int D, int G>
__device__ __forceinline__ void split_item_mfma(const StepArgs &a, char *stage, int s, int g, int h0, int b) {
    using S = MfmaState<D, G>;
    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) return;
    const int t0 = s * a.split_tokens;
    if (t0 >= L) return;
    const int t1 = min(t0 + a.split_tokens, L);
    S st;
    st.lds = stage;
    st.init(a, b, h0);
    const size_t run_off = (size_t)g * S::RUN + (size_t)(threadIdx.x & 63) * 16;
    stream_pages(st, a.page_table + (size_t)b * a.max_pages, run_off, t0, t1);
    st.finish(a, b, h0, s);
}

// Matrix-core split kernels: one wavefront per work item (KV head blockIdx.x,
// item list entry blockIdx.y + gridDim.y * blockIdx.z), or (PER_QUERY_HEAD,
// G = 1) the naive comparator with one item per query head, (s, h, b) =
// blockIdx (x, y, z) over every split slot; and the looping form for
// host-dominated layouts.
constexpr int kMfmaWavesPerSimd = 3;   // register budget: 168 per lane

template <int D, int G, bool PER_QUERY_HEAD = false>
__global__ __launch_bounds__(64, kMfmaWavesPerSimd) void attn_split_mfma_kernel(StepArgs a) {
    __shared__ __attribute__((aligned(16))) char stage[MfmaState<D, G>::STAGE];
    if constexpr (PER_QUERY_HEAD) {
        // The naive comparator keeps a plain (split, query head, sequence) order.
        const int h = blockIdx.y;
        split_item_mfma<D, G>(a, stage, blockIdx.x, h / (a.n_q_heads / a.n_kv_heads), h, blockIdx.z);
    } else {
        int b, s;
        if (!listed_item(a, blockIdx.y + gridDim.y * blockIdx.z, b, s)) return;
        split_item_mfma<D, G>(a, stage, s, blockIdx.x, blockIdx.x * G, b);
    }
}

// The looping form runs a few hundred wavefronts in all (one or two per CU),
// so it may use the registers of a whole SIMD; it takes its items from the
// same queue as attn_split_persistent_kernel below.
template <int D, int G>
__global__ __launch_bounds__(64, 1) void attn_split_mfma_persistent_kernel(StepArgs a) {
    __shared__ __attribute__((aligned(16))) char stage[MfmaState<D, G>::STAGE];
    __shared__ int item;
    const int n_items = a.n_kv_heads * (int)a.item_list[0];
    for (;;) {
        const int i = take_item(a, &item);
        if (i >= n_items) break;
        const int g = i % a.n_kv_heads;
        int b, s;
        listed_item(a, i / a.n_kv_heads, b, s);
        split_item_mfma<D, G>(a, stage, s, g, g * G, b);
    }
}

// One wavefront per work item (KV head blockIdx.x, item list entry
// blockIdx.y + gridDim.y * blockIdx.z).
// PER_QUERY_HEAD (with G = 1) is the naive zero-copy comparator, not the
// method: one work item per query head (s, h, b) = blockIdx (x, y, z), so each KV head's pages
// cross the link once per query head of its group (G times per step) instead
// of once. Each head's arithmetic is the same as in the grouped kernel.
template <int D, int G, int WPI, bool PER_QUERY_HEAD = false>
__global__ __launch_bounds__(64 * WPI, WPI) void attn_split_kernel(StepArgs a) {
    if constexpr (PER_QUERY_HEAD) {
        const int h = blockIdx.y;
        split_item<D, G, WPI>(a, blockIdx.x, h / (a.n_q_heads / a.n_kv_heads), h, blockIdx.z);
    } else {
        int b, s;
        if (!listed_item(a, blockIdx.y + gridDim.y * blockIdx.z, b, s)) return;
        split_item<D, G, WPI>(a, s, blockIdx.x, blockIdx.x * G, b);
    }
}

// The same work items on a fixed number of workgroups (gridDim.x), each
// taking the next item from a shared queue (take_item) in the order (KV head
// fastest, then the item list's (sequence, split) pairs), so the waves in flight read the runs
// of the same pages together. Bounding the waves in flight bounds the
// requests queued on the host link, where too many outstanding reads lower
// its bandwidth (the streaming-read probe drops from 57.5 to 56.0 GB/s when
// it keeps 8 MiB in flight instead of 1 MiB). Taking items as waves free up,
// rather than every gridDim.x-th item, keeps ragged contexts balanced: with
// 8192-token items of sequences of 8192 to 131072 tokens the fixed stride
// left the link 1.3 % idle at the end of a step. Each item is computed
// exactly as above, whichever wave takes it.
template <int D, int G, int WPI>
__global__ __launch_bounds__(64 * WPI, WPI) void attn_split_persistent_kernel(StepArgs a) {
    __shared__ int item;
    const int n_items = a.n_kv_heads * (int)a.item_list[0];
    for (;;) {
        const int i = take_item(a, &item);
        if (i >= n_items) break;
        const int g = i % a.n_kv_heads;
        int b, s;
        listed_item(a, i / a.n_kv_heads, b, s);
        split_item<D, G, WPI>(a, s, g, g * G, b);
    }
}

// ------------------------------------------------------------------------------
// Producer/consumer variant. One workgroup per work item: wavefront 0 is the
// producer and streams the item's page runs with LDS DMA
// (global_load_lds_dwordx4: 16 bytes per lane straight into LDS, no
// registers) into an NS-slot ring, keeping NS - 1 runs in flight;
// wavefronts 1 .. NC are consumers, each owning G / NC of the group's query
// heads, reading every run from LDS once it has landed. The run is fetched
// from host memory or HBM once for all NC consumers. Per page the workgroup
// meets at one barrier: the producer has waited for that run's loads
// (s_waitcnt vmcnt, so the ring slot is complete) and the consumers have
// finished the previous run (so its slot may be refilled). Every head's
// arithmetic is the same as in attn_split_kernel, in the same order, so both
// variants give identical bits.

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every outstanding DMA load); the compiler may not move memory
// accesses across it.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_barrier" ::: "memory"); }

constexpr int kAuxNontemporal = 2;   // cache-policy bits of the DMA load: nt

template <int D, int G, int NC, int NS>
__global__ __launch_bounds__(64 * (NC + 1)) void attn_split_lds_kernel(StepArgs a) {
    static_assert(G % NC == 0 && NS >= 2, "bad variant");
    constexpr int HW = G / NC;                 // query heads per consumer
    using S = SplitState<D, HW>;
    constexpr int NLD = S::NLD;
    constexpr int LPT = S::LPT;
    constexpr int LPP = 2 * NLD;               // DMA loads per page run
    __shared__ __attribute__((aligned(16))) char ring[NS][S::RUN];

    const int g = blockIdx.x;
    int b, s;
    if (!listed_item(a, blockIdx.y + gridDim.y * blockIdx.z, b, s)) return;
    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) return;
    const int t0 = s * a.split_tokens;
    if (t0 >= L) return;
    const int t1 = min(t0 + a.split_tokens, L);
    const int p0 = t0 / kPageTokens;
    const int np = (t1 + kPageTokens - 1) / kPageTokens - p0;   // pages p0 .. p0 + np - 1
    const int pf = t1 / kPageTokens;                              // pages below pf are full

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;

    if (wave == 0) {
        // Producer. Page addresses come 64 at a time into one VGPR pair per
        // lane and are broadcast with readlane, so no vector load of the page
        // table sits between the DMA loads (its wait would drain them).
        const uint64_t *pt = a.page_table + (size_t)b * a.max_pages + p0;
        const size_t run_off = (size_t)g * S::RUN + (size_t)lane * 16;
        uint64_t window = 0;
        auto issue = [&](int i) {
            if ((i & 63) == 0) window = (i + lane < np) ? pt[i + lane] : 0;
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)window, i & 63);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(window >> 32), i & 63);
            const char *src = reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo) + run_off;
            char *dst = ring[i % NS];
#pragma unroll
            for (int j = 0; j < LPP; ++j)
                __builtin_amdgcn_global_load_lds(src + j * 1024, (__attribute__((address_space(3))) void *)(dst + j * 1024),
                                                 16, 0, kAuxNontemporal);
        };
        for (int i = 0; i < NS - 1 && i < np; ++i) issue(i);
        for (int i = 0; i < np; ++i) {
            if (i + NS - 2 < np) wait_vmcnt<LPP * (NS - 2)>();   // runs i + 1 .. i + NS - 2 may still fly
            else wait_vmcnt<0>();
            ring_barrier();
            if (i + NS - 1 < np) {                                // refills the slot of run i - 1
                if (a.lds_poison) {
                    // Debug: NaN over the freed slot, landed before its refill is issued.
                    char *dst = ring[(i + NS - 1) % NS] + lane * 16;
#pragma unroll
                    for (int j = 0; j < LPP; ++j)
                        *reinterpret_cast<uint4 *>(dst + j * 1024) = make_uint4(0x7FC07FC0u, 0x7FC07FC0u,
                                                                               0x7FC07FC0u, 0x7FC07FC0u);
                    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
                }
                issue(i + NS - 1);
            }
        }
        return;
    }

    // Consumer wave c = wave - 1: query heads h0 .. h0 + HW - 1.
    const int sub = lane / LPT;
    const int dl = lane % LPT;
    const int h0 = g * G + (wave - 1) * HW;
    S st;
    st.init(a, b, h0, dl);
    for (int i = 0; i < np; ++i) {
        ring_barrier();
        const char *slot = ring[i % NS] + lane * 16;
        uint4 kr[NLD], vr[NLD];
#pragma unroll
        for (int j = 0; j < NLD; ++j) kr[j] = *reinterpret_cast<const uint4 *>(slot + j * 1024);
#pragma unroll
        for (int j = 0; j < NLD; ++j) vr[j] = *reinterpret_cast<const uint4 *>(slot + S::TILE + j * 1024);
        if (p0 + i < pf) st.template page<false>(kr, vr, sub, kPageTokens);
        else st.template page<true>(kr, vr, sub, t1 - (p0 + i) * kPageTokens);
    }
    st.finish(a, b, h0, s, dl);
}

// Producer/consumer form with a matrix-core consumer (groups of 4 and 8,
// head_dim 128): the producer/consumer pipeline of the pages (DirectKV
// digest, 核心方法; "KV Cache 内存层级" overview, 2.1: producer, consumer and
// storer warp groups) with the register kernel's arithmetic, so that the
// two streaming schemes compare with the same consumer. One workgroup of two
// wavefronts per work item: wavefront 0 streams the item's page runs into an
// NS-slot LDS ring with LDS DMA (global_load_lds_dwordx4), NS - 1 runs in
// flight; wavefront 1 runs MfmaState::compute on each run straight from its
// ring slot, so a run is never copied from registers into LDS. The DMA writes
// lane l's 16 bytes to slot byte 16 l of its 1 KiB load, but each lane picks
// which 16 bytes of the run it fetches: load j covers token rows 4j .. 4j + 3
// of the K tile (j < 4) or the V tile, and lane l fetches chunk (l % 16) ^ t
// of row t = 4 (j % 4) + l / 16, so the slot holds each row's chunk c at
// position c ^ t, the layout MfmaState::compute<SWZ = true> reads without
// bank conflicts. Every load still covers one contiguous 1 KiB of the run.
// Same handoff as attn_split_lds_kernel: one barrier per page. Two ring
// slots (one run in flight per producer) with four wavefronts per SIMD (123
// VGPRs, 16 KiB of LDS: eight workgroups per CU) measured fastest, within a
// few percent of the register kernel with every page in HBM (MI355X, split
// kernel, all-HBM: config-2 shape 0.165 vs 0.161 ms, config-4 shape 0.62-0.64
// vs 0.65 ms, 70B layer 1.31 vs 1.30 ms); three or four slots leave the
// compiler at 176 VGPRs (two wavefronts per SIMD) and run 15-20 % slower.
template <int G, int NS>
__global__ __launch_bounds__(128, 4) void attn_split_lds_mfma_kernel(StepArgs a) {
    constexpr int D = 128;
    using S = MfmaState<D, G>;
    constexpr int LPP = S::RUN / 1024;                          // DMA loads per page run
    static_assert(S::TILE == 4096 && LPP == 8, "the swizzle assumes 16-chunk rows, 4 rows per load");
    __shared__ __attribute__((aligned(16))) char ring[NS][S::RUN];

    const int g = blockIdx.x;
    int b, s;
    if (!listed_item(a, blockIdx.y + gridDim.y * blockIdx.z, b, s)) return;
    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) return;
    const int t0 = s * a.split_tokens;
    if (t0 >= L) return;
    const int t1 = min(t0 + a.split_tokens, L);
    const int p0 = t0 / kPageTokens;
    const int np = (t1 + kPageTokens - 1) / kPageTokens - p0;   // pages p0 .. p0 + np - 1
    const int pf = t1 / kPageTokens;                              // pages below pf are full
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;

    if (wave == 0) {
        const uint64_t *pt = a.page_table + (size_t)b * a.max_pages + p0;
        const size_t run_off = (size_t)g * S::RUN;
        uint64_t window = 0;
        auto issue = [&](int i) {
            if ((i & 63) == 0) window = (i + lane < np) ? pt[i + lane] : 0;
            const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)window, i & 63);
            const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(window >> 32), i & 63);
            const char *run = reinterpret_cast<const char *>(((uint64_t)hi << 32) | lo) + run_off;
            char *dst = ring[i % NS];
#pragma unroll
            for (int j = 0; j < LPP; ++j) {
                // Row t of the tile, chunk position lane % 16: the row's chunk (lane % 16) ^ t.
                // (Computed here: an array of these offsets captured by the lambda made hipcc
                // drop the kernel's host-side launch stub.)
                const int t = 4 * (j % 4) + lane / 16;
                const char *src = run + (j / 4) * S::TILE + t * (D * 2) + (((lane % 16) ^ t) << 4);
                __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(dst + j * 1024), 16, 0,
                                                 kAuxNontemporal);
            }
        };
        for (int i = 0; i < NS - 1 && i < np; ++i) issue(i);
        for (int i = 0; i < np; ++i) {
            if (i + NS - 2 < np) wait_vmcnt<LPP * (NS - 2)>();   // runs i + 1 .. i + NS - 2 may still fly
            else wait_vmcnt<0>();
            ring_barrier();
            if (i + NS - 1 < np) {                                // refills the slot of run i - 1
                if (a.lds_poison) {
                    char *dst = ring[(i + NS - 1) % NS] + lane * 16;
#pragma unroll
                    for (int j = 0; j < LPP; ++j)
                        *reinterpret_cast<uint4 *>(dst + j * 1024) = make_uint4(0x7FC07FC0u, 0x7FC07FC0u,
                                                                               0x7FC07FC0u, 0x7FC07FC0u);
                    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
                }
                issue(i + NS - 1);
            }
        }
        return;
    }

    S st;
    st.init(a, b, g * G);
    for (int i = 0; i < np; ++i) {
        ring_barrier();
        const char *slot = ring[i % NS];
        if (p0 + i < pf) st.template compute<false, true>(slot, slot + S::TILE, kPageTokens);
        else st.template compute<true, true>(slot, slot + S::TILE, t1 - (p0 + i) * kPageTokens);
    }
    st.finish(a, b, g * G, s);
}

// XCD-aware item order of the one-wavefront-per-item launches: the KV head is
// the fastest grid dimension. Workgroups go to the GPU's 8 XCDs round-robin
// in linear order, so with 8 KV heads each XCD (its own L2 and a fixed share
// of the fabric bandwidth) serves one KV head, and every KV head carries the
// same bytes whatever the sequences' lengths. With the split index fastest,
// XCD k got splits s = k (mod 8): with ragged contexts every sequence has a
// split 0 but only the long ones a split 7 or 15, so one XCD streamed 2.3x
// the bytes of another (MI355X, batch 32, contexts U[8192, 131072], all in
// HBM, 8192-token splits: 1.87 ms, the busiest XCD's bytes at 1/8 of the
// chip's bandwidth). The host does not know ctx_lens, so the grid has a
// workgroup for every split the capacities allow (item_slots per KV head),
// and the y/z index walks the step's item list: the workgroups with work are
// dispatched first, those past the list's end return at once. Sizing the grid
// by the capacities rather than by batch x max_splits matters: 2048 trailing
// empty workgroups behind 2048 items still cost 5 % (MI355X, batch 32,
// 65536-token contexts in HBM, 8192-token splits: 1.236 ms vs 1.298 ms).
dim3 item_grid(const StepArgs &a) {
    const int ny = std::min(a.item_slots, 65535);
    return dim3(a.n_kv_heads, ny, (a.item_slots + ny - 1) / ny);
}

template <int D, int G>
void launch(const StepArgs &a, hipStream_t st) {
    // Groups of 8 query heads share each work item between two wavefronts.
    constexpr int WPI = G >= 8 ? 2 : 1;
    const dim3 grid = item_grid(a);
    if (a.split_variant == kSplitNaive) {
        // Per query head, with the arithmetic of the layout's grouped kernel.
        const dim3 heads(a.max_splits, a.n_q_heads, a.batch);
        if (G >= kMfmaMinGroup) attn_split_mfma_kernel<D, 1, true><<<heads, 64, 0, st>>>(a);
        else attn_split_kernel<D, 1, WPI, true><<<heads, 64 * WPI, 0, st>>>(a);
    } else if (a.split_variant == kSplitMfma) {
        if (a.split_waves > 0) attn_split_mfma_persistent_kernel<D, G><<<a.split_waves, 64, 0, st>>>(a);
        else attn_split_mfma_kernel<D, G><<<grid, 64, 0, st>>>(a);
    } else if (a.split_variant == kSplitLds) {
        // Consumers own at most 4 query heads each; 4 ring slots (3 runs in
        // flight) unless a debug knob asks for 2 or 3.
        constexpr int NC = G > 4 ? G / 4 : 1;
        if (a.lds_ring == 2) attn_split_lds_kernel<D, G, NC, 2><<<grid, 64 * (NC + 1), 0, st>>>(a);
        else if (a.lds_ring == 3) attn_split_lds_kernel<D, G, NC, 3><<<grid, 64 * (NC + 1), 0, st>>>(a);
        else attn_split_lds_kernel<D, G, NC, 4><<<grid, 64 * (NC + 1), 0, st>>>(a);
    } else if (a.split_waves > 0) {
        attn_split_persistent_kernel<D, G, WPI><<<a.split_waves, 64 * WPI, 0, st>>>(a);
    } else {
        attn_split_kernel<D, G, WPI><<<grid, 64 * WPI, 0, st>>>(a);
    }
}

// The LDS ring with a matrix-core consumer (head_dim 128, one workgroup per
// item in the same XCD-aware order).
template <int G>
void launch_lds_mfma(const StepArgs &a, hipStream_t st) {
    const dim3 grid = item_grid(a);
    if (a.lds_ring == 3) attn_split_lds_mfma_kernel<G, 3><<<grid, 128, 0, st>>>(a);
    else if (a.lds_ring == 4) attn_split_lds_mfma_kernel<G, 4><<<grid, 128, 0, st>>>(a);
    else attn_split_lds_mfma_kernel<G, 2><<<grid, 128, 0, st>>>(a);
}

}  // namespace

hipError_t launch_split(const StepArgs &a, hipStream_t st) {
    const int G = a.n_q_heads / a.n_kv_heads;
    if (a.split_variant == kSplitLdsMfma) {
        if (a.head_dim == 128 && G == 4) launch_lds_mfma<4>(a, st);
        else if (a.head_dim == 128 && G == 8) launch_lds_mfma<8>(a, st);
        else return hipErrorInvalidValue;
        return hipGetLastError();
    }
    if (a.head_dim == 128) {
        switch (G) {
            case 1: launch<128, 1>(a, st); break;
            case 2: launch<128, 2>(a, st); break;
            case 4: launch<128, 4>(a, st); break;
            case 8: launch<128, 8>(a, st); break;
            default: return hipErrorInvalidValue;
        }
    } else if (a.head_dim == 64) {
        switch (G) {
            case 1: launch<64, 1>(a, st); break;
            case 2: launch<64, 2>(a, st); break;
            case 4: launch<64, 4>(a, st); break;
            case 8: launch<64, 8>(a, st); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dkv
