// Fused QKV projection of one decode step on gfx950: y_b = W_qkv x_b for
// every sequence b, fp32 accumulation of exact bf16 products. Rows below
// Hq*d are the query (kept in fp32, pre-scaled by log2(e)/sqrt(d) so that
// scores come out in log2 units); the rest are the fresh K then V heads,
// rounded once to bf16. The projection that produces the new token's K/V is
// part of the decode step, as in the core-method section of the DirectKV
// digest ("长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）"); the step is bound
// by reading W from HBM at every batch size here, so both variants are built
// to stream W once at full bandwidth.
#include "device_common.h"

namespace dkv {
namespace {


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

// Sums each of the N values (N a power of two <= 64) over the 64 lanes of
// the wave, leaving the total of value i in the lanes whose top log2(N)
// lane-id bits equal i. One butterfly halves the value count per step
// (N - 1 shuffles in all instead of 6 N), then plain butterflies finish the
// lanes that still share an index. The order of additions is fixed.
template <int N, int TOTAL>
__device__ __forceinline__ void halve(float (&v)[TOTAL], int lane) {
    if constexpr (N > 1) {
        constexpr int off = 32 * N / TOTAL;    // 32 on the first step, then 16, 8, ...
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int i = 0; i < N / 2; ++i) {
            const float send = upper ? v[i] : v[i + N / 2];
            const float keep = upper ? v[i + N / 2] : v[i];
            v[i] = keep + __shfl_xor(send, off);
        }
        halve<N / 2, TOTAL>(v, lane);
    }
}

template <int N>
__device__ __forceinline__ float reduce_scatter(float (&v)[N], int lane) {
    static_assert(N >= 2 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
    halve<N, N>(v, lane);
    float r = v[0];
#pragma unroll
    for (int off = 32 / N; off >= 1; off >>= 1) r += __shfl_xor(r, off);
    return r;
}

// 1a. Small batches: a GEMV on VALU. A workgroup owns 4 W rows and BT
// sequences; its KS wavefronts split the hidden dimension into equal ranges,
// and each lane reads 16-byte (8 x bf16) chunks, so every W row is read as
// contiguous 1 KiB wave loads, all of a wave's loads issued before its
// FMAs (short k ranges, unrolled). The wave's 4*BT partial sums are reduced
// with a reduce-scatter butterfly and the KS waves' sums added through LDS in
// wave order, so the result does not depend on timing.
template <int BT, int KS>
__global__ __launch_bounds__(64 * KS) void qkv_proj_gemv_kernel(StepArgs a) {
    constexpr int NV = 4 * BT;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * 4;
    const int b0 = blockIdx.y * BT;
    const int nb = min(BT, a.batch - b0);
    const int krange = a.hidden / KS;     // a multiple of 512 (checked at launch)
    const int kbeg = wave * krange;

    if (blockIdx.x == 0 && threadIdx.x < nb) check_context_range(a, b0 + threadIdx.x);

    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;

    const uint16_t *w0 = a.w + (size_t)row0 * a.hidden;
#pragma unroll 2
    for (int k = kbeg + lane * 8; k < kbeg + krange; k += 512) {
        float wf[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) unpack8(*reinterpret_cast<const uint4 *>(w0 + (size_t)r * a.hidden + k), wf[r]);
#pragma unroll
        for (int bb = 0; bb < BT; ++bb) {
            if (bb < nb) {
                float xf[8];
                unpack8(*reinterpret_cast<const uint4 *>(a.x + (size_t)(b0 + bb) * a.hidden + k), xf);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[r * BT + bb] = fmaf(wf[r][e], xf[e], acc[r * BT + bb]);
            }
        }
    }

    const float y = reduce_scatter<NV>(acc, lane);
    constexpr int SHIFT = NV == 64 ? 0 : NV == 32 ? 1 : NV == 16 ? 2 : 3;
    const int idx = lane >> SHIFT;            // value index this lane holds
    const bool owner = (lane & ((1 << SHIFT) - 1)) == 0;

    float total = y;
    if constexpr (KS > 1) {
        __shared__ float part[KS][NV];
        if (owner) part[wave][idx] = y;
        __syncthreads();
        if (wave != 0) return;
        total = part[0][idx];
#pragma unroll
        for (int w = 1; w < KS; ++w) total += part[w][idx];
    }
    if (owner) {
        const int r = idx / BT, bb = idx % BT;
        if (bb < nb) store_projection(a, row0 + r, b0 + bb, total);
    }
}

// 1b. Larger batches: the projection is a dense [N_qkv x hidden] x [hidden x B]
// contraction, done on the matrix cores with v_mfma_f32_16x16x32_bf16 (bf16
// in, fp32 accumulate). Operand layout of the 16x16x32 MFMA: lane l supplies
// A[i = l%16][k = 8*(l/16) .. +7] and B[k = 8*(l/16) .. +7][j = l%16], and
// receives D[i = 4*(l/16) + r][j = l%16], r < 4. A is a W tile (W rows are
// contiguous in k), B is x^T (x rows are contiguous in k), so both operands
// are plain 16-byte loads from row-major memory.
//
// One wavefront owns 16 W rows x a 512-wide slice of k x up to 64 sequences
// (NBT tiles of 16): it loads its W slice once (16 KiB, issued together with
// the first sequence tile's x slice, all before the first MFMA) and keeps it
// in registers while it walks the sequence tiles, the next tile's x slice
// in flight during the current tile's 16 MFMAs. x is small and shared by
// every workgroup, so it comes from L2; W crosses HBM once. The KS
// wavefronts of a workgroup cover the hidden dimension (CH slices each) and
// add their partial tiles through LDS in wave order, so the result does not
// depend on timing. Batches above 64 take more workgroup columns.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NK>
__device__ __forceinline__ void load_slice(uint4 (&v)[NK], const uint16_t *row, int k0) {
#pragma unroll
    for (int u = 0; u < NK; ++u) v[u] = *reinterpret_cast<const uint4 *>(row + k0 + 32 * u);
}

template <int NK>
__device__ __forceinline__ void mfma_slice(f32x4 &acc, const uint4 (&w)[NK], const uint4 (&x)[NK]) {
#pragma unroll
    for (int u = 0; u < NK; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w[u]),
                                                      __builtin_bit_cast(bf16x8, x[u]), acc, 0, 0, 0);
}

template <int KS, int NBT>
__global__ __launch_bounds__(64 * KS) void qkv_proj_mfma_kernel(StepArgs a, int ch) {
    constexpr int KSL = 512;            // k per slice
    constexpr int NK = KSL / 32;        // MFMA k steps per slice
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int row0 = blockIdx.x * 16;
    const int b0 = blockIdx.y * 16 * NBT;

    if (blockIdx.x == 0 && wave == 0)
        for (int b = b0 + lane; b < min(a.batch, b0 + 16 * NBT); b += 64) check_context_range(a, b);

    // Sequences past the batch read a valid row (the last one) and are never stored.
    const uint16_t *wrow = a.w + (size_t)(row0 + i) * a.hidden + kq;
    const uint16_t *xrow[NBT];
#pragma unroll
    for (int t = 0; t < NBT; ++t) xrow[t] = a.x + (size_t)min(b0 + 16 * t + i, a.batch - 1) * a.hidden + kq;

    f32x4 acc[NBT];
#pragma unroll
    for (int t = 0; t < NBT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int c = 0; c < ch; ++c) {
        const int k0 = (wave * ch + c) * KSL;
        uint4 wv[NK], xa[NK], xb[NK];
        load_slice(wv, wrow, k0);
        load_slice(xa, xrow[0], k0);
        __builtin_amdgcn_sched_barrier(0);     // the slice's loads go out before the first MFMA
#pragma unroll
        for (int t = 0; t < NBT; t += 2) {
            if (t + 1 < NBT) load_slice(xb, xrow[t + 1], k0);
            mfma_slice(acc[t], wv, xa);
            if (t + 1 < NBT) {
                if (t + 2 < NBT) load_slice(xa, xrow[t + 2], k0);
                mfma_slice(acc[t + 1], wv, xb);
            }
        }
    }

    if constexpr (KS > 1) {
        __shared__ f32x4 partial[KS - 1][NBT][64];
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < NBT; ++t) partial[wave - 1][t][lane] = acc[t];
        }
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < KS; ++w)
#pragma unroll
            for (int t = 0; t < NBT; ++t) acc[t] += partial[w - 1][t][lane];
    }
#pragma unroll
    for (int t = 0; t < NBT; ++t) {
        const int b = b0 + 16 * t + i;
        if (b < a.batch) {
#pragma unroll
            for (int r = 0; r < 4; ++r) store_projection(a, row0 + 4 * (lane >> 4) + r, b, acc[t][r]);
        }
    }
}

// 1c. One tile of up to 16 sequences: the same 16x16x32 MFMA tiles, but each
// wavefront streams its 16 W rows over a k range of hidden / KSPLIT in
// 256-wide chunks, the next chunk's W and x loads in flight while the
// current chunk's 8 MFMAs run (register double buffer), so a few thousand
// wavefronts keep W streaming from HBM for the whole launch instead of
// issuing one burst each. The KSPLIT wavefronts of a workgroup share the 16
// rows and add their partial tiles through LDS in wave order.
template <int KSPLIT>
__global__ __launch_bounds__(64 * KSPLIT) void qkv_proj_stream_kernel(StepArgs a) {
    constexpr int KC = 256;             // k per chunk
    constexpr int NK = KC / 32;         // MFMA k steps per chunk
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int row0 = blockIdx.x * 16;
    const int krange = a.hidden / KSPLIT;      // a multiple of 256 (checked at launch)
    const int nch = krange / KC;

    if (blockIdx.x == 0 && wave == 0 && lane < a.batch) check_context_range(a, lane);

    // Lanes of sequences past the batch load nothing and feed zeros; their
    // columns are never stored.
    const bool live = i < a.batch;
    const uint16_t *wrow = a.w + (size_t)(row0 + i) * a.hidden + wave * krange + kq;
    const uint16_t *xrow = a.x + (size_t)min(i, a.batch - 1) * a.hidden + wave * krange + kq;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    uint4 wa[NK], xa[NK], wb[NK], xb[NK];
    auto load_x = [&](uint4 (&v)[NK], int k0) {
        if (live) load_slice(v, xrow, k0);
        else {
#pragma unroll
            for (int u = 0; u < NK; ++u) v[u] = make_uint4(0u, 0u, 0u, 0u);
        }
    };
    load_slice(wa, wrow, 0);
    load_x(xa, 0);
    for (int c = 0; c < nch; c += 2) {
        if (c + 1 < nch) {
            load_slice(wb, wrow, (c + 1) * KC);
            load_x(xb, (c + 1) * KC);
        }
        mfma_slice(acc, wa, xa);
        if (c + 1 < nch) {
            if (c + 2 < nch) {
                load_slice(wa, wrow, (c + 2) * KC);
                load_x(xa, (c + 2) * KC);
            }
            mfma_slice(acc, wb, xb);
        }
    }

    if constexpr (KSPLIT > 1) {
        __shared__ f32x4 partial[KSPLIT - 1][64];
        if (wave > 0) partial[wave - 1][lane] = acc;
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int w = 1; w < KSPLIT; ++w) acc += partial[w - 1][lane];
    }
    if (i < a.batch) {
#pragma unroll
        for (int r = 0; r < 4; ++r) store_projection(a, row0 + 4 * (lane >> 4) + r, i, acc[r]);
    }
}

template <int KS>
void launch_mfma(const StepArgs &a, int ch, hipStream_t st) {
    const int nbt = (a.batch + 15) / 16;
    if (nbt == 1) {
        qkv_proj_mfma_kernel<KS, 1><<<dim3(a.n_qkv / 16, 1), 64 * KS, 0, st>>>(a, ch);
    } else if (nbt == 2) {
        qkv_proj_mfma_kernel<KS, 2><<<dim3(a.n_qkv / 16, 1), 64 * KS, 0, st>>>(a, ch);
    } else {
        qkv_proj_mfma_kernel<KS, 4><<<dim3(a.n_qkv / 16, (nbt + 3) / 4), 64 * KS, 0, st>>>(a, ch);
    }
}

template <int BT>
hipError_t launch_gemv(const StepArgs &a, hipStream_t st) {
    // Largest split of the hidden dimension (up to 8 waves) that leaves each
    // wave a range of at least two 512-wide steps; 1 for short rows.
    int ks = 8;
    while (ks > 1 && (a.hidden % (512 * ks) != 0 || a.hidden / (512 * ks) < 2)) ks >>= 1;
    const dim3 grid(a.n_qkv / 4, (a.batch + BT - 1) / BT);
    switch (ks) {
        case 1: qkv_proj_gemv_kernel<BT, 1><<<grid, 64, 0, st>>>(a); break;
        case 2: qkv_proj_gemv_kernel<BT, 2><<<grid, 128, 0, st>>>(a); break;
        case 4: qkv_proj_gemv_kernel<BT, 4><<<grid, 256, 0, st>>>(a); break;
        default: qkv_proj_gemv_kernel<BT, 8><<<grid, 512, 0, st>>>(a); break;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_projection(const StepArgs &a, hipStream_t st) {
    if (a.hidden % 512 != 0 || a.n_qkv % 16 != 0) return hipErrorInvalidValue;
    if (a.batch >= a.proj_mfma_min_batch && a.batch <= 16) {
        // One sequence tile: streamed over k by up to 4 wavefronts per row block.
        int ksplit = 4;
        while (ksplit > 1 && a.hidden % (256 * ksplit) != 0) ksplit >>= 1;
        const dim3 grid(a.n_qkv / 16);
        switch (ksplit) {
            case 1: qkv_proj_stream_kernel<1><<<grid, 64, 0, st>>>(a); break;
            case 2: qkv_proj_stream_kernel<2><<<grid, 128, 0, st>>>(a); break;
            default: qkv_proj_stream_kernel<4><<<grid, 256, 0, st>>>(a); break;
        }
    } else if (a.batch >= a.proj_mfma_min_batch) {
        // Up to 8 wavefronts per workgroup over the 512-wide k slices.
        const int n_slices = a.hidden / 512;
        int ks = 8;
        while (ks > 1 && n_slices % ks != 0) ks >>= 1;
        const int ch = n_slices / ks;
        switch (ks) {
            case 1: launch_mfma<1>(a, ch, st); break;
            case 2: launch_mfma<2>(a, ch, st); break;
            case 4: launch_mfma<4>(a, ch, st); break;
            default: launch_mfma<8>(a, ch, st); break;
        }
    } else if (a.batch <= 4) {
        (void)launch_gemv<4>(a, st);
    } else if (a.batch <= 8) {
        (void)launch_gemv<8>(a, st);
    } else {
        (void)launch_gemv<16>(a, st);
    }
    return hipGetLastError();
}

}  // namespace dkv
