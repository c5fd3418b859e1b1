// Split combine, fresh token and write-back of one decode step on gfx950.
//
// One workgroup of four wavefronts per (sequence b, query head h):
//  * scores the fresh token from the projection's scratch (the new K/V never
//    travel to host memory and back before they are used),
//  * merges the split partials (m_s, l_s, o_s) and the fresh token:
//      M = max(s_new, max_s m_s),  o = (sum_s 2^(m_s - M) o_s + 2^(s_new - M) v_new)
//                                      / (sum_s 2^(m_s - M) l_s + 2^(s_new - M)),
//    every sum taken in a fixed order (splits strided over the waves, then the
//    waves' sums in wave order), so the result does not depend on timing,
//  * writes attn_out (bf16, round to nearest even, or fp32), and
//  * for the first query head of each KV group, writes the fresh K and V rows
//    once into slot ctx_lens[b] of the sequence's pages (host or HBM): the
//    single write-back of the new token ("storer" role in the core-method
//    section of the DirectKV digest, "长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）").
#include "device_common.h"

namespace dkv {
namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 64 * kWaves;   // splits weighed per pass

template <int D, int G>
__global__ __launch_bounds__(64 * kWaves) void attn_combine_kernel(StepArgs a) {
    constexpr int DPL = D / 64;    // output dims per lane
    const int b = blockIdx.x / a.n_q_heads;
    const int h = blockIdx.x - b * a.n_q_heads;
    const int g = h / G;
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
        const float *qh = a.q + ((size_t)b * a.n_q_heads + h) * D;
        const uint16_t *kn = a.kv_new + ((size_t)b * a.n_kv_heads + g) * 2 * D;
        const uint16_t *vn = kn + D;
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            part = fmaf(qh[lane * DPL + e], __uint_as_float((uint32_t)kn[lane * DPL + e] << 16), part);
        const float s_new = wave_sum(part);    // every wave computes it (no barrier)

        const int S = (L + a.split_tokens - 1) / a.split_tokens;
        const size_t slot0 = ((size_t)b * a.n_q_heads + h) * a.max_splits;
        const float2 *ml = a.part_ml + slot0;
        const float *po = a.part_o + slot0 * D + (size_t)lane * DPL;

        // Pass 1: the common max.
        float mx = s_new;
        for (int s = tid; s < S; s += kChunk) mx = fmaxf(mx, ml[s].x);
        mx = wave_max(mx);
        if (lane == 0) s_red[wave] = mx;
        __syncthreads();
        float M = s_red[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_red[w]);

        // Pass 2: weights of a chunk of splits into LDS, then each wave adds
        // the weighted outputs of the chunk's splits w, w + 4, ...
        float den = 0.0f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = 0.0f;
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
        den = wave_sum(den);
        if (lane == 0) s_den[wave] = den;
#pragma unroll
        for (int e = 0; e < DPL; ++e) s_o[wave][lane * DPL + e] = o[e];
        __syncthreads();

        if (wave == 0) {
            float dsum = s_den[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) dsum += s_den[w];
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                float acc = s_o[0][lane * DPL + e];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) acc += s_o[w][lane * DPL + e];
                o[e] = acc;
            }
            const float cn = fast_exp2(s_new - M);
            dsum += cn;
#pragma unroll
            for (int e = 0; e < DPL; ++e)
                o[e] = fmaf(cn, __uint_as_float((uint32_t)vn[lane * DPL + e] << 16), o[e]) / dsum;
        } else if (wave == 1 && h % G == 0) {
            // The fresh K and V rows go to slot L once: lanes 0-31 the K row,
            // lanes 32-63 the V row (one query head per KV group does it).
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
            return;
        } else {
            return;
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
void launch(const StepArgs &a, hipStream_t st) {
    attn_combine_kernel<D, G><<<a.batch * a.n_q_heads, 64 * kWaves, 0, st>>>(a);
}

}  // namespace

hipError_t launch_combine(const StepArgs &a, hipStream_t st) {
    const int G = a.n_q_heads / a.n_kv_heads;
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
