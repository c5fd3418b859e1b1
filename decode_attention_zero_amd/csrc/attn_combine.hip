// Split combine of one decode step on gfx950.
//
// One workgroup of four wavefronts per (sequence b, query head h) merges the
// partial softmax states (m_s, l_s, o_s) of the sequence's splits and, in the
// slot after them, the fresh token's one-token state (s_new, 1, v_new) that
// the fresh-token kernel wrote:
//     M = max_s m_s,   o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// every sum taken in a fixed order (slots strided over the waves, then the
// waves' sums in wave order), so the result does not depend on timing, and
// writes attn_out (bf16, round to nearest even, or fp32). The split/merge of
// the softmax state is the standard flash-decoding decomposition; the pages
// ("长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）", 核心方法) fix only that
// the attention reads the KV in place, not how it is partitioned.
#include "device_common.h"

namespace dkv {
namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 64 * kWaves;   // slots weighed per pass
constexpr int kPrefetch = 8;          // slots per wave held in registers on the short path

template <int D>
__global__ __launch_bounds__(64 * kWaves) void attn_combine_kernel(StepArgs a) {
    constexpr int DPL = D / 64;    // output dims per lane
    const int b = blockIdx.x / a.n_q_heads;
    const int h = blockIdx.x - b * a.n_q_heads;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int L = a.ctx_lens[b];
    const size_t obase = ((size_t)b * a.n_q_heads + h) * D + (size_t)lane * DPL;

    __shared__ float s_red[kWaves];
    __shared__ float s_c[kChunk];
    __shared__ float s_o[kWaves][D];
    __shared__ float s_den[kWaves];

    float o[DPL];
    if (L < 0 || L >= a.capacity[b]) {
        if (wave != 0) return;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = __builtin_nanf("");
    } else {
        // The sequence's splits, then the fresh token.
        const int S = (L + a.split_tokens - 1) / a.split_tokens + 1;
        const size_t slot0 = ((size_t)b * a.n_q_heads + h) * a.part_slots;
        const float2 *ml = a.part_ml + slot0;
        const float *po = a.part_o + slot0 * D + (size_t)lane * DPL;

        float den = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
        if (S <= kWaves * kPrefetch) {
            // Short path (every split count up to 31): each thread's state and
            // each wave's output vectors are loaded at once, so the merge waits
            // for memory once. Same sums, in the same order, as the loop below.
            const float2 st = tid < S ? ml[tid] : make_float2(kNegInf, 0.0f);
            float ov[kPrefetch][DPL];
#pragma unroll
            for (int i = 0; i < kPrefetch; ++i) {
                const int j = wave + kWaves * i;
                if constexpr (DPL == 2) {
                    const float2 v = j < S ? *reinterpret_cast<const float2 *>(po + (size_t)j * D)
                                           : make_float2(0.0f, 0.0f);
                    ov[i][0] = v.x;
                    ov[i][1] = v.y;
                } else {
                    for (int e = 0; e < DPL; ++e) ov[i][e] = j < S ? po[(size_t)j * D + e] : 0.0f;
                }
            }
            float mx = wave_max(st.x);
            if (lane == 0) s_red[wave] = mx;
            __syncthreads();
            float M = s_red[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_red[w]);
            float c = 0.0f;
            if (tid < S) {
                c = fast_exp2(st.x - M);
                den = fmaf(c, st.y, den);
            }
            s_c[tid] = c;
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kPrefetch; ++i) {
                const int j = wave + kWaves * i;
                if (j < S) {
                    const float cj = s_c[j];
#pragma unroll
                    for (int e = 0; e < DPL; ++e) o[e] = fmaf(cj, ov[i][e], o[e]);
                }
            }
        } else {
            // Pass 1: the common max.
            float mx = kNegInf;
            for (int s = tid; s < S; s += kChunk) mx = fmaxf(mx, ml[s].x);
            mx = wave_max(mx);
            if (lane == 0) s_red[wave] = mx;
            __syncthreads();
            float M = s_red[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_red[w]);

            // Pass 2: weights of a chunk of slots into LDS, then each wave adds
            // the weighted outputs of the chunk's slots w, w + 4, ...
            for (int c0 = 0; c0 < S; c0 += kChunk) {
                const int s = c0 + tid;
                float c = 0.0f;
                if (s < S) {
                    const float2 st = ml[s];
                    c = fast_exp2(st.x - M);
                    den = fmaf(c, st.y, den);
                }
                __syncthreads();                  // the previous chunk's weights are consumed
                s_c[tid] = c;
                __syncthreads();
                const int n = min(kChunk, S - c0);
#pragma unroll 4
                for (int j = wave; j < n; j += kWaves) {
                    const float cj = s_c[j];
                    const float *p = po + (size_t)(c0 + j) * D;
                    if constexpr (DPL == 2) {
                        const float2 v = *reinterpret_cast<const float2 *>(p);
                        o[0] = fmaf(cj, v.x, o[0]);
                        o[1] = fmaf(cj, v.y, o[1]);
                    } else {
#pragma unroll
                        for (int e = 0; e < DPL; ++e) o[e] = fmaf(cj, p[e], o[e]);
                    }
                }
            }
        }
        den = wave_sum(den);
        if (lane == 0) s_den[wave] = den;
#pragma unroll
        for (int e = 0; e < DPL; ++e) s_o[wave][lane * DPL + e] = o[e];
        __syncthreads();
        if (wave != 0) return;

        float dsum = s_den[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) dsum += s_den[w];
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            float acc = s_o[0][lane * DPL + e];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) acc += s_o[w][lane * DPL + e];
            o[e] = acc / dsum;
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

}  // namespace

hipError_t launch_combine(const StepArgs &a, hipStream_t st) {
    if (a.head_dim == 128) {
        attn_combine_kernel<128><<<a.batch * a.n_q_heads, 64 * kWaves, 0, st>>>(a);
    } else if (a.head_dim == 64) {
        attn_combine_kernel<64><<<a.batch * a.n_q_heads, 64 * kWaves, 0, st>>>(a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace dkv
