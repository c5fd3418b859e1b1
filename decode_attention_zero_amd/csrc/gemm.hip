// GEMM with an operand in host memory: the matrix-multiplication experiment
// the pages use to show why zero-copy needs CPU-aware tiling. The DirectKV
// digest ("长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）") and the "KV Cache
// 内存层级" overview (opening section, Fig. 2(a): a 10240-square GEMM, 65 ms
// with a 200 MB swap buffer vs 1122 ms reading CPU memory directly; 2.1: the
// CPU-aware tiling makes the HBM operand the one that is re-read, so each B
// tile crosses the link once) describe it; this is a gfx950 rendition.
//
//   C[M][N] (fp32) = A[M][K] (bf16, HBM) x B[N][K]^T (bf16, host or HBM)
//
// Each workgroup computes a (64*WM) x 128 tile of C with the LDS-staged
// matrix-core tile product of mfma_tile.h (both operands staged per 64-wide
// k step, loads two steps ahead); every element of C is one fp32 sum over k
// in the same order whatever the tile order or where B lives, so all
// variants give identical bits.
//
// Tile orders (the only difference between the zero-copy variants):
//   row-major  (naive): workgroup id -> (m block, n block), n fastest; the
//              workgroups in flight cover many B column blocks, so B's
//              column blocks are fetched over the link again for every m
//              block.
//   CPU-aware: workgroup id % 8 picks the XCD (the dispatcher places
//              workgroups on the 8 XCDs round-robin); XCD x owns the n blocks
//              x, x + 8, ..., and runs all m blocks of one n block back to
//              back, so that block's B rows (128 x K) are fetched over the
//              link into the XCD's L2 and re-read from there, while A (in
//              HBM) is the operand read again -- with nontemporal loads, so it
//              streams past the L2 instead of evicting B (without that, the
//              10240-square product took 135 ms instead of 15.5 ms with the
//              earlier register-only kernel).
#include "mfma_tile.h"

namespace dkv {
namespace {

using tile::bf16x8;
using tile::f32x4;
using tile::kRowBytes;
using tile::kStepK;
constexpr int kTileN = tile::kN;
constexpr int kXcds = 8;

template <int WM, bool CPU_AWARE>
__global__ __launch_bounds__(128 * WM, WM == 4 ? 2 : 1) void gemm_nt_kernel(const uint16_t *__restrict__ A, const uint16_t *B,
                                                           float *__restrict__ C, int M, int N, int K) {
    using T = tile::Shape<WM>;
    __shared__ __attribute__((aligned(16))) char lds[2][T::STAGE];
    const int nmb = M / T::BM, nnb = N / kTileN;
    const int id = blockIdx.x;
    int mb, nb;
    if (CPU_AWARE) {
        const int xcd = id % kXcds, local = id / kXcds;
        mb = local % nmb;
        nb = xcd + kXcds * (local / nmb);
    } else {
        mb = id / nnb;
        nb = id % nnb;
    }
    const int m0 = mb * T::BM, n0 = nb * kTileN;

    f32x4 acc[4][4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // K is a multiple of 64; A is read nontemporally in the CPU-aware order.
    tile::product<WM, CPU_AWARE, false>(acc, lds, A, B, K, m0, M, n0, 0, K / kStepK);

    const tile::Lane ln;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int col = n0 + ln.wn * 64 + tn * 16 + ln.i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + ln.wm * 64 + tm * 16 + ln.kq * 4 + r;
                C[(size_t)row * N + col] = acc[tm][tn][r];
            }
        }
}

template <int WM>
void launch_tiles(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K, bool cpu_aware,
                  hipStream_t st) {
    const int blocks = (M / (64 * WM)) * (N / kTileN);
    if (cpu_aware) gemm_nt_kernel<WM, true><<<blocks, 128 * WM, 0, st>>>(A, B, C, M, N, K);
    else gemm_nt_kernel<WM, false><<<blocks, 128 * WM, 0, st>>>(A, B, C, M, N, K);
}

// ---------------------------------------------------------------------------
// B-stationary form: the CPU-aware tiling of the "KV Cache 内存层级" overview
// (2.1 去搬运：DirectKV: every tile of the remote operand crosses the link once,
// the remote traffic drops from O(n^3) to O(n^2), and partial results of C go
// through HBM instead, which roughly doubles the HBM traffic) taken
// literally. Workgroup (n tile, k tile) keeps the 128 x 512 tile of B in LDS
// (128 KiB: rows of 1 KiB, 16-byte chunk c of row n at chunk position
// c ^ (n % 16), so the MFMA operand reads of 16 rows hit 16 bank groups) and
// sweeps all of M past it in 64-row blocks: the tile is fetched first -- from
// host memory, once -- and A slices are staged in LDS two steps ahead as in
// gemm_nt_kernel. The
// workgroup writes its fp32 partial C[:, n tile] of k tile p to slab p of a
// workspace, and gemm_bstat_reduce_kernel adds the slabs in k order. The
// workgroups of one k tile read the same A columns in the same order, so
// those that share an XCD meet in its L2.
constexpr int kBsN = 128;                       // B tile rows (n)
constexpr int kBsK = 512;                       // B tile k extent
constexpr int kBsM = 64;                        // rows of A per sweep block
constexpr int kBsThreads = 256;                 // 4 wavefronts, each 64 (m) x 32 (n)
constexpr int kBsRow = kBsK * 2;                // bytes of a B row in LDS
constexpr int kBsSteps = kBsK / kStepK;         // 64-wide k steps per tile

__device__ __forceinline__ int bs_offset(int n, int chunk) {
    return n * kBsRow + ((chunk ^ (n & 15)) << 4);
}

// One 64-wide k step's A slice (64 rows x 64 k) of the sweep.
struct BsStep {
    static constexpr int ACH = kBsM * (kStepK / 8) / kBsThreads;   // 2 chunks per thread
    u32x4 a[ACH];   // a native vector type: register-allocated, unlike the uint4 struct here

    __device__ __forceinline__ void load(const uint16_t *A, int K, int k0, int step) {
        const int t = threadIdx.x;
        const int mb = step / kBsSteps, s = step % kBsSteps;
#pragma unroll
        for (int c = 0; c < ACH; ++c) {
            const int ch = t + c * kBsThreads;
            a[c] = *reinterpret_cast<const u32x4 *>(A + (size_t)(mb * kBsM + (ch >> 3)) * K + k0 + s * kStepK +
                                                    (ch & 7) * 8);
        }
    }

    __device__ __forceinline__ void stage(char *abuf) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int c = 0; c < ACH; ++c) {
            const int ch = t + c * kBsThreads;
            *reinterpret_cast<u32x4 *>(abuf + (ch >> 3) * kRowBytes + (ch & 7) * 16) = a[c];
        }
    }
};

// k step s (0 .. kBsSteps-1) of a block of the sweep: the wavefront's 4 x 2
// MFMA tiles over the step's 64 k values.
template <int S>
__device__ __forceinline__ void bs_compute(f32x4 (&acc)[4][2], const char *abuf, const char *bt) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, i = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        uint4 af[4], bf[2];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
            af[tm] = *reinterpret_cast<const uint4 *>(abuf + (tm * 16 + i) * kRowBytes + (h * 4 + kq) * 16);
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
            bf[tn] = *reinterpret_cast<const uint4 *>(bt + bs_offset(wave * 32 + tn * 16 + i, S * 8 + h * 4 + kq));
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 2; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[tm]),
                                                                      __builtin_bit_cast(bf16x8, bf[tn]),
                                                                      acc[tm][tn], 0, 0, 0);
    }
}

// Even and odd k steps of the two-deep pipeline (gemm_nt_kernel's scheme):
// at an even step x holds the next step and y receives the one after; at an
// odd step the roles swap.
template <int S>
__device__ __forceinline__ void bs_step(f32x4 (&acc)[4][2], BsStep &x, BsStep &y, const uint16_t *A, int K, int k0,
                                        int step, int total, char (&as)[2][kBsM * kRowBytes], const char *bt) {
    if constexpr (S % 2 == 0) {
        if (step + 2 < total) y.load(A, K, k0, step + 2);
        bs_compute<S>(acc, as[0], bt);
        if (step + 1 < total) x.stage(as[1]);
    } else {
        if (step + 2 < total) x.load(A, K, k0, step + 2);
        bs_compute<S>(acc, as[1], bt);
        if (step + 1 < total) y.stage(as[0]);
    }
    __syncthreads();
}

__global__ __launch_bounds__(kBsThreads, 1) void gemm_bstat_partial_kernel(const uint16_t *__restrict__ A,
                                                                        const uint16_t *B, float *__restrict__ P,
                                                                        int M, int N, int K) {
    __shared__ __attribute__((aligned(16))) char bt[kBsN * kBsRow];
    __shared__ __attribute__((aligned(16))) char as[2][kBsM * kRowBytes];
    const int n0 = blockIdx.x * kBsN, k0 = blockIdx.y * kBsK;
    float *slab = P + (size_t)blockIdx.y * M * N;
    const int total = (M / kBsM) * kBsSteps;     // (m block, k step) pairs, k step fastest
    const int t = threadIdx.x;
    static_assert(kBsSteps == 8, "the sweep below unrolls 8 k steps per block");

    // The B tile, fetched once: 8192 16-byte chunks, 8 per thread in flight
    // at a time (each 1 KiB row read as 64 contiguous chunks).
    constexpr int BCH = kBsN * (kBsK / 8) / kBsThreads;   // 32
#pragma unroll
    for (int c0 = 0; c0 < BCH; c0 += 8) {
        u32x4 v[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ch = t + (c0 + c) * kBsThreads;
            v[c] = *reinterpret_cast<const u32x4 *>(B + (size_t)(n0 + (ch >> 6)) * K + k0 + (ch & 63) * 8);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ch = t + (c0 + c) * kBsThreads;
            *reinterpret_cast<u32x4 *>(bt + bs_offset(ch >> 6, ch & 63)) = v[c];
        }
    }

    // The sweep over M, one 64-row block at a time, 8 k steps per block.
    const int lane = t & 63, wave = t >> 6, i = lane & 15, kq = lane >> 4;
    BsStep x, y;
    x.load(A, K, k0, 0);
    x.stage(as[0]);
    if (total > 1) x.load(A, K, k0, 1);
    __syncthreads();
    for (int mb = 0; mb < M / kBsM; ++mb) {
        f32x4 acc[4][2];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) acc[tm][tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const int st = mb * kBsSteps;
        bs_step<0>(acc, x, y, A, K, k0, st + 0, total, as, bt);
        bs_step<1>(acc, x, y, A, K, k0, st + 1, total, as, bt);
        bs_step<2>(acc, x, y, A, K, k0, st + 2, total, as, bt);
        bs_step<3>(acc, x, y, A, K, k0, st + 3, total, as, bt);
        bs_step<4>(acc, x, y, A, K, k0, st + 4, total, as, bt);
        bs_step<5>(acc, x, y, A, K, k0, st + 5, total, as, bt);
        bs_step<6>(acc, x, y, A, K, k0, st + 6, total, as, bt);
        bs_step<7>(acc, x, y, A, K, k0, st + 7, total, as, bt);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 2; ++tn) {
                const int col = n0 + wave * 32 + tn * 16 + i;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    slab[(size_t)(mb * kBsM + tm * 16 + kq * 4 + r) * N + col] = acc[tm][tn][r];
            }
    }
}

// C = sum of the KT slabs in k order, four elements per thread.
__global__ __launch_bounds__(256) void gemm_bstat_reduce_kernel(const float4 *__restrict__ P, float4 *__restrict__ C,
                                                               size_t n4, int kt_count) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= n4) return;
    float4 sum = P[e];
#pragma unroll 4
    for (int p = 1; p < kt_count; ++p) {
        const float4 v = P[(size_t)p * n4 + e];
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    C[e] = sum;
}

}  // namespace

uint64_t gemm_bstationary_workspace_bytes(int M, int N, int K) {
    return (uint64_t)(K / kBsK) * (uint64_t)M * (uint64_t)N * sizeof(float);
}

// M a multiple of 64, N of 128, K of 512; workspace of
// gemm_bstationary_workspace_bytes(M, N, K) bytes.
hipError_t launch_gemm_nt_bstationary(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K,
                                      float *workspace, hipStream_t st) {
    const dim3 grid(N / kBsN, K / kBsK);
    gemm_bstat_partial_kernel<<<grid, kBsThreads, 0, st>>>(A, B, workspace, M, N, K);
    const size_t n4 = (size_t)M * N / 4;
    gemm_bstat_reduce_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>(
        reinterpret_cast<const float4 *>(workspace), reinterpret_cast<float4 *>(C), n4, K / kBsK);
    return hipGetLastError();
}

// M a multiple of 128 (256-row tiles when M allows), N of 128, K of 64.
hipError_t launch_gemm_nt(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K,
                          bool cpu_aware, hipStream_t st) {
    if (M % 256 == 0) launch_tiles<4>(A, B, C, M, N, K, cpu_aware, st);
    else launch_tiles<2>(A, B, C, M, N, K, cpu_aware, st);
    return hipGetLastError();
}

}  // namespace dkv
