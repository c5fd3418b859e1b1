// Kernels of one zero-copy decode step on gfx950 (MI355X).
//
// Three stream-ordered launches per layer:
//   1. qkv_proj_kernel     y = W x for the batch (HBM-bound on W): q kept in
//                          fp32 scratch (pre-scaled for exp2), fresh K/V
//                          rounded once to bf16 into a small HBM scratch.
//   2. attn_split_kernel   one wavefront per work item (sequence b, KV head g,
//                          token split s): streams the split's KV pages in
//                          place -- host pages over the host link, HBM pages
//                          from HBM, chosen only by the page's address -- and
//                          keeps an online-softmax state for the G query heads
//                          that share the KV head, so each remote byte is read
//                          once for all of them. Writes an unnormalised
//                          partial (m, l, o).
//   3. attn_combine_kernel one wavefront per (b, query head): scores the fresh
//                          token from the scratch (it never travels to host
//                          memory and back), merges the partials and the fresh
//                          token in a fixed order, writes attn_out, and writes
//                          the fresh K/V once into slot ctx_lens[b] of the
//                          sequence's last page.
//
// Method (pages): "长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）" (DirectKV
// digest), 核心方法: the kernel reads CPU-resident KV directly with a layout
// arranged for coalesced remote reads, and the fresh K/V stay on chip instead
// of being written to CPU memory and read back. The split/merge of the
// softmax state is the standard flash-decoding decomposition (not on the
// pages); the split boundaries depend only on token indices, never on where a
// page lives, so host and HBM placements give bit-identical results.
#include "dkv_internal.h"

namespace dkv {
namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// From this batch size on, y = W x has enough columns (sequences) to be a
// real contraction and runs on MFMA; below it W is read by a VALU GEMV.
constexpr int kMfmaMinBatch = 32;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// KV pages are streamed once per step: nontemporal 16-byte loads keep them
// from displacing reusable lines and measured ~13 % more HBM read bandwidth
// on gfx950 than plain loads for the same page-run pattern.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void unpack8(const uint4 &v, float f[8]) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Cross-lane move inside a 16-lane row (DPP). CTRL: 0xB1 = quad_perm
// [1,0,3,2] (lane ^ 1), 0x4E = quad_perm [2,3,0,1] (lane ^ 2),
// 0x141 = row_half_mirror (i <-> 7 - i in each 8-lane half), 0x140 =
// row_mirror (i <-> 15 - i).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the LPT consecutive lanes that hold one token (LPT = 8 or 16);
// every lane of the group gets the total.
template <int LPT>
__device__ __forceinline__ float token_sum(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    if constexpr (LPT == 16) v += dpp<0x140>(v);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// 2^x with the hardware instruction (v_exp_f32). Softmax exponents here are
// <= 0; results below 2^-126 may flush to 0, which is below the weight of
// any token that matters at fp32 resolution.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(x - M) weight of a softmax state whose max is x, under a common max M;
// a state that has seen no token (x = -inf) weighs 0.
__device__ __forceinline__ float rescale(float x, float M) {
    return x == kNegInf ? 0.0f : fast_exp2(x - M);
}

// ------------------------------------------------------------------------------
// 1. QKV projection: y_b = W x_b with fp32 accumulation. Rows < Hq*d are q
// (kept fp32, pre-scaled for exp2); the rest are the fresh K then V heads,
// rounded once to bf16.
__device__ __forceinline__ void store_projection(const StepArgs &a, int n, int b, float y) {
    const int D = a.head_dim;
    const int nq = a.n_q_heads * D;
    if (n < nq) {
        a.q[(size_t)b * nq + n] = y * a.qscale;
    } else {
        const int n2 = n - nq;
        const int c = n2 / (a.n_kv_heads * D);
        const int rem = n2 - c * (a.n_kv_heads * D);
        const int g = rem / D, i = rem - g * D;
        a.kv_new[(((size_t)b * a.n_kv_heads + g) * 2 + c) * D + i] = f32_to_bf16(y);
    }
}

// Sequences whose ctx_lens entry is out of range raise the layout's flag.
__device__ __forceinline__ void check_context_range(const StepArgs &a, int b) {
    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) atomicOr(a.status, 1u);
}

// 1a. Small batches (B < 32): a GEMV on VALU. One wavefront computes 4 output
// rows for BT sequences; lanes split the hidden dimension in 16-byte
// (8 x bf16) chunks, so each W row is read as contiguous 1 KiB wave loads.
template <int BT>
__global__ __launch_bounds__(256) void qkv_proj_kernel(StepArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * 4 + wave) * 4;
    const int b0 = blockIdx.y * BT;
    const int nb = min(BT, a.batch - b0);

    if (blockIdx.x == 0 && threadIdx.x < nb) check_context_range(a, b0 + threadIdx.x);
    if (row0 >= a.n_qkv) return;

    float acc[4][BT];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) acc[r][bb] = 0.0f;

    for (int k = lane * 8; k < a.hidden; k += 512) {
        float wf[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const uint4 w = *reinterpret_cast<const uint4 *>(a.w + (size_t)(row0 + r) * a.hidden + k);
            unpack8(w, wf[r]);
        }
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) {
            if (bb < nb) {
                float xf[8];
                unpack8(*reinterpret_cast<const uint4 *>(a.x + (size_t)(b0 + bb) * a.hidden + k), xf);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r][bb] = fmaf(wf[r][e], xf[e], acc[r][bb]);
            }
        }
    }

    float y = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) {
            const float v = wave_sum(acc[r][bb]);
            if (lane == r * BT + bb) y = v;
        }

    if (lane < 4 * BT) {
        const int r = lane / BT, bb = lane % BT;
        if (bb < nb) store_projection(a, row0 + r, b0 + bb, y);
    }
}

// 1b. Batches of 32 or more: the projection is a dense [N_qkv x hidden] x
// [hidden x B] contraction, done on the matrix cores with
// v_mfma_f32_16x16x32_bf16 (bf16 in, fp32 accumulate). One wavefront owns 16
// W rows and 16*NB sequences, so every W byte is read once per step.
// Operand layout of the 16x16x32 MFMA: lane l supplies A[i = l%16][k = 8*(l/16)
// .. +7] and B[k = 8*(l/16) .. +7][j = l%16], and receives
// D[i = 4*(l/16) + r][j = l%16], r < 4. A is the W tile (rows of W are
// contiguous in k), B is x^T (rows of x are contiguous in k), so both operands
// are plain 16-byte loads from row-major memory.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NB>
struct MfmaChunk {
    static constexpr int UK = 4;   // 32-wide k steps per chunk (128 k)
    uint4 w[UK];
    uint4 x[UK][NB];
};

template <int NB>
__device__ __forceinline__ void mfma_load(MfmaChunk<NB> &c, const uint16_t *wrow,
                                          const uint16_t *const (&xrow)[NB], int k0) {
#pragma unroll
    for (int u = 0; u < MfmaChunk<NB>::UK; ++u) {
        c.w[u] = *reinterpret_cast<const uint4 *>(wrow + k0 + 32 * u);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) c.x[u][nb] = *reinterpret_cast<const uint4 *>(xrow[nb] + k0 + 32 * u);
    }
}

template <int NB>
__device__ __forceinline__ void mfma_step(const MfmaChunk<NB> &c, f32x4 (&acc)[NB]) {
#pragma unroll
    for (int u = 0; u < MfmaChunk<NB>::UK; ++u) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, c.w[u]);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, c.x[u][nb]),
                                                              acc[nb], 0, 0, 0);
    }
}

// Split-k: the workgroup's KS wavefronts (blockDim.x / 64, 2 or 4) take equal
// k ranges of the same 16-row x 16*NB-sequence tile; their partial tiles are
// added through LDS in wave order, so the result does not depend on timing.
template <int NB>
__global__ __launch_bounds__(256) void qkv_proj_mfma_kernel(StepArgs a) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int ks = blockDim.x >> 6;
    const int row0 = blockIdx.x * 16;
    const int b0 = blockIdx.y * 16 * NB;
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int krange = a.hidden / ks;      // a multiple of 256 (checked at launch)
    const int kbeg = wave * krange;

    if (blockIdx.x == 0 && wave == 0) {
        for (int b = b0 + lane; b < min(a.batch, b0 + 16 * NB); b += 64) check_context_range(a, b);
    }

    // Columns past the batch read a valid row (the last sequence's) and are
    // never stored, so the k loop has no per-lane branches.
    const uint16_t *wrow = a.w + (size_t)(row0 + i) * a.hidden + kbeg + kq;
    const uint16_t *xrow[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        xrow[nb] = a.x + (size_t)min(b0 + nb * 16 + i, a.batch - 1) * a.hidden + kbeg + kq;
    f32x4 acc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // The 128-wide chunks of a wave's k range come in pairs: ping-pong between
    // two register sets, the next chunk's loads in flight while the current
    // one feeds the matrix cores.
    constexpr int KC = 32 * MfmaChunk<NB>::UK;
    MfmaChunk<NB> c0, c1;
    mfma_load(c0, wrow, xrow, 0);
    for (int k0 = 0; k0 < krange; k0 += 2 * KC) {
        mfma_load(c1, wrow, xrow, k0 + KC);
        mfma_step(c0, acc);
        if (k0 + 2 * KC < krange) mfma_load(c0, wrow, xrow, k0 + 2 * KC);
        mfma_step(c1, acc);
    }

    __shared__ f32x4 partial[3][NB][64];
    if (wave > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) partial[wave - 1][nb][lane] = acc[nb];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < ks; ++w) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] += partial[w - 1][nb][lane];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int b = b0 + nb * 16 + i;
        if (b < a.batch) {
#pragma unroll
            for (int r = 0; r < 4; ++r) store_projection(a, row0 + 4 * (lane >> 4) + r, b, acc[nb][r]);
        }
    }
}

// ------------------------------------------------------------------------------
// 2. Split attention. Work item (s, g, b) = blockIdx (x, y, z); one wavefront.
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
template <int D, int G>
struct SplitState {
    static constexpr int LPT = D / 8;               // lanes per token
    static constexpr int TPL = 64 / LPT;            // tokens per wave load
    static constexpr int NLD = kPageTokens / TPL;   // wave loads per 16-token tile
    static constexpr int TILE = kPageTokens * D * 2;
    static constexpr int RUN = 2 * TILE;

    float q[G][8];
    float m[G], l[G], acc[G][8];

    __device__ __forceinline__ void load(const char *run, uint4 (&kr)[NLD], uint4 (&vr)[NLD]) const {
#pragma unroll
        for (int j = 0; j < NLD; ++j) kr[j] = load_stream(run + j * 1024);
#pragma unroll
        for (int j = 0; j < NLD; ++j) vr[j] = load_stream(run + TILE + j * 1024);
    }

    // One page. PARTIAL: only the first n_valid tokens of the page count.
    template <bool PARTIAL>
    __device__ __forceinline__ void page(const uint4 (&kr)[NLD], const uint4 (&vr)[NLD], int sub,
                                         int n_valid) {
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
};

template <int D, int G>
__global__ __launch_bounds__(64) void attn_split_kernel(StepArgs a) {
    using S = SplitState<D, G>;
    constexpr int NLD = S::NLD;
    constexpr int LPT = S::LPT;

    const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) return;
    const int t0 = s * a.split_tokens;
    if (t0 >= L) return;
    const int t1 = min(t0 + a.split_tokens, L);

    const int lane = threadIdx.x;
    const int sub = lane / LPT;
    const int dl = lane % LPT;

    S st;
    {
        const float *qb = a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * D + dl * 8;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float4 lo = *reinterpret_cast<const float4 *>(qb + h * D);
            const float4 hi = *reinterpret_cast<const float4 *>(qb + h * D + 4);
            st.q[h][0] = lo.x; st.q[h][1] = lo.y; st.q[h][2] = lo.z; st.q[h][3] = lo.w;
            st.q[h][4] = hi.x; st.q[h][5] = hi.y; st.q[h][6] = hi.z; st.q[h][7] = hi.w;
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
        st.m[h] = kNegInf;
        st.l[h] = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.0f;
    }

    const uint64_t *pt = a.page_table + (size_t)b * a.max_pages;
    const size_t run_off = (size_t)g * S::RUN + (size_t)lane * 16;
    auto run_of = [&](int p) { return reinterpret_cast<const char *>(pt[p]) + run_off; };

    const int p0 = t0 / kPageTokens;
    const int p1 = (t1 + kPageTokens - 1) / kPageTokens;   // pages [p0, p1)
    const int pf = t1 / kPageTokens;                        // pages [p0, pf) are full
    uint4 ka[NLD], va[NLD], kb[NLD], vb[NLD];
    int p = p0;
    st.load(run_of(p), ka, va);
    while (p + 1 < pf) {                 // pages p (in a) and p + 1 are full
        st.load(run_of(p + 1), kb, vb);
        st.template page<false>(ka, va, sub, kPageTokens);
        if (p + 2 < p1) st.load(run_of(p + 2), ka, va);
        st.template page<false>(kb, vb, sub, kPageTokens);
        p += 2;
    }
    if (p < pf) {                        // one last full page (in a), maybe a partial one after
        if (p + 1 < p1) st.load(run_of(p + 1), kb, vb);
        st.template page<false>(ka, va, sub, kPageTokens);
        if (p + 1 < p1) st.template page<true>(kb, vb, sub, t1 - (p + 1) * kPageTokens);
    } else if (p < p1) {                 // the partial page (in a)
        st.template page<true>(ka, va, sub, t1 - p * kPageTokens);
    }

    // Merge the row states (lanes l and l ^ off, off >= LPT) in a fixed order.
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(st.m[h], off);
            const float lo = __shfl_xor(st.l[h], off);
            const float M = fmaxf(st.m[h], mo);
            const float c1 = rescale(st.m[h], M);
            const float c2 = rescale(mo, M);
            st.l[h] = fmaf(st.l[h], c1, lo * c2);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float ao = __shfl_xor(st.acc[h][e], off);
                st.acc[h][e] = fmaf(st.acc[h][e], c1, ao * c2);
            }
            st.m[h] = M;
        }
    }

    if (sub == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const size_t slot = ((size_t)b * a.n_q_heads + (size_t)g * G + h) * a.max_splits + s;
            float *po = a.part_o + slot * D + dl * 8;
            *reinterpret_cast<float4 *>(po) =
                make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
            *reinterpret_cast<float4 *>(po + 4) =
                make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
            if (dl == 0) a.part_ml[slot] = make_float2(st.m[h], st.l[h]);
        }
    }
}

// ------------------------------------------------------------------------------
// 3. Combine + fresh token + write-back. One wavefront per (b, query head).
template <int D, int G>
__global__ __launch_bounds__(64) void attn_combine_kernel(StepArgs a) {
    constexpr int DPL = D / 64;    // dims per lane
    const int b = blockIdx.x / a.n_q_heads;
    const int h = blockIdx.x - b * a.n_q_heads;
    const int g = h / G;
    const int lane = threadIdx.x;
    const int L = a.ctx_lens[b];
    const size_t obase = ((size_t)b * a.n_q_heads + h) * D + (size_t)lane * DPL;

    float o[DPL];
    if (L < 0 || L >= a.capacity[b]) {
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = __builtin_nanf("");
    } else {
        const float *qh = a.q + ((size_t)b * a.n_q_heads + h) * D;
        const uint16_t *kn = a.kv_new + ((size_t)b * a.n_kv_heads + g) * 2 * D;
        const uint16_t *vn = kn + D;
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            part = fmaf(qh[lane * DPL + e], __uint_as_float((uint32_t)kn[lane * DPL + e] << 16), part);
        const float s_new = wave_sum(part);

        const int S = (L + a.split_tokens - 1) / a.split_tokens;
        const size_t slot0 = ((size_t)b * a.n_q_heads + h) * a.max_splits;
        const float2 *ml = a.part_ml + slot0;
        const float *po = a.part_o + slot0 * D + (size_t)lane * DPL;

        float M = s_new;
        for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s].x);
        float den = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
        for (int s = 0; s < S; ++s) {
            const float2 st = ml[s];
            const float c = fast_exp2(st.x - M);
            den = fmaf(c, st.y, den);
#pragma unroll
            for (int e = 0; e < DPL; ++e) o[e] = fmaf(c, po[(size_t)s * D + e], o[e]);
        }
        const float cn = fast_exp2(s_new - M);
        den += cn;
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            o[e] = fmaf(cn, __uint_as_float((uint32_t)vn[lane * DPL + e] << 16), o[e]) / den;

        // The fresh K and V rows go to slot L once: lanes 0-31 the K row,
        // lanes 32-63 the V row (one query head per KV group does it).
        if (h % G == 0) {
            const int c = lane >> 5;
            char *page = reinterpret_cast<char *>(a.page_table[(size_t)b * a.max_pages + L / kPageTokens]);
            char *dst = page + ((size_t)((g * 2 + c) * kPageTokens + (L % kPageTokens)) * D) * 2;
            const char *src = reinterpret_cast<const char *>(kn + c * D);
            constexpr int BPL = D * 2 / 32;    // bytes per lane
            const int li = lane & 31;
            if constexpr (BPL == 8) {
                *reinterpret_cast<uint2 *>(dst + li * 8) = *reinterpret_cast<const uint2 *>(src + li * 8);
            } else {
                *reinterpret_cast<uint32_t *>(dst + li * 4) = *reinterpret_cast<const uint32_t *>(src + li * 4);
            }
        }
    }

    if (a.out_f32) {
        float *out = reinterpret_cast<float *>(a.out) + obase;
#pragma unroll
        for (int e = 0; e < DPL; ++e) out[e] = o[e];
    } else {
        uint16_t *out = reinterpret_cast<uint16_t *>(a.out) + obase;
#pragma unroll
        for (int e = 0; e < DPL; ++e) out[e] = f32_to_bf16(o[e]);
    }
}

template <int D, int G>
void launch_attention(const StepArgs &a, hipStream_t st, hipEvent_t *ev) {
    dim3 grid_split(a.max_splits, a.n_kv_heads, a.batch);
    attn_split_kernel<D, G><<<grid_split, 64, 0, st>>>(a);
    if (ev) (void)hipEventRecord(ev[2], st);
    attn_combine_kernel<D, G><<<a.batch * a.n_q_heads, 64, 0, st>>>(a);
    if (ev) (void)hipEventRecord(ev[3], st);
}

template <int D>
void dispatch_group(const StepArgs &a, int G, hipStream_t st, hipEvent_t *ev) {
    switch (G) {
        case 1: launch_attention<D, 1>(a, st, ev); break;
        case 2: launch_attention<D, 2>(a, st, ev); break;
        case 4: launch_attention<D, 4>(a, st, ev); break;
        default: launch_attention<D, 8>(a, st, ev); break;
    }
}

// ------------------------------------------------------------------------------
// Streaming-read probe: grid-stride 16-byte loads, U in flight per lane.
template <int U, bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4 *__restrict__ p, uint64_t nvec,
                                                          uint32_t *sink) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    uint32_t x = 0;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride * U) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t j = i + (uint64_t)u * stride;
            v[u] = j < nvec ? (NT ? load_stream(p + j) : p[j]) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (x == 0x9E3779B9u) sink[0] = x;   // keeps the loads alive
}

}  // namespace

hipError_t launch_decode_step(const StepArgs &a, hipStream_t st, hipEvent_t *ev) {
    constexpr int BT = 8;
    const int G = a.n_q_heads / a.n_kv_heads;
    if (!((a.head_dim == 128 || a.head_dim == 64) && (G == 1 || G == 2 || G == 4 || G == 8)))
        return hipErrorInvalidValue;
    if (ev) (void)hipEventRecord(ev[0], st);
    if (a.batch >= kMfmaMinBatch) {
        // 16 W rows x 64 sequences per workgroup (32 for batches up to 32),
        // k split over 4 wavefronts (2 when hidden is not a multiple of 1024)
        const int threads = (a.hidden % 1024 == 0) ? 256 : 128;
        if (a.batch <= 32) {
            qkv_proj_mfma_kernel<2><<<dim3(a.n_qkv / 16, (a.batch + 31) / 32), threads, 0, st>>>(a);
        } else {
            qkv_proj_mfma_kernel<4><<<dim3(a.n_qkv / 16, (a.batch + 63) / 64), threads, 0, st>>>(a);
        }
    } else {
        dim3 grid_proj((a.n_qkv + 15) / 16, (a.batch + BT - 1) / BT);
        qkv_proj_kernel<BT><<<grid_proj, 256, 0, st>>>(a);
    }
    if (ev) (void)hipEventRecord(ev[1], st);
    if (a.head_dim == 128) dispatch_group<128>(a, G, st, ev);
    else dispatch_group<64>(a, G, st, ev);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void *ptr, uint64_t bytes, int grid, int unroll, bool nontemporal,
                              uint32_t *sink, hipStream_t st) {
    const uint4 *p = reinterpret_cast<const uint4 *>(ptr);
    const uint64_t nvec = bytes / 16;
    if (nontemporal) {
        switch (unroll) {
            case 1: stream_read_kernel<1, true><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            case 2: stream_read_kernel<2, true><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            case 4: stream_read_kernel<4, true><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            case 8: stream_read_kernel<8, true><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (unroll) {
            case 1: stream_read_kernel<1, false><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            case 2: stream_read_kernel<2, false><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            case 4: stream_read_kernel<4, false><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            case 8: stream_read_kernel<8, false><<<grid, 256, 0, st>>>(p, nvec, sink); break;
            default: return hipErrorInvalidValue;
        }
    }
    return hipGetLastError();
}

}  // namespace dkv
