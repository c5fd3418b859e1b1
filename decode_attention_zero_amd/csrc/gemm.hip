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
// Both operands are k-contiguous rows, so every MFMA operand is a plain
// 16-byte load: lane l of v_mfma_f32_16x16x32_bf16 supplies A[i = l%16][k =
// 8*(l/16) .. +7] and B[j = l%16][same k] and receives C[4*(l/16) + r][l%16].
// A workgroup (4 wavefronts, 2 x 2) computes a 128 x 128 tile of C; each
// wavefront a 64 x 64 block (4 x 4 MFMA tiles), with the next 32-wide k step
// in flight while the current one feeds the matrix cores. Every element of C
// is one fp32 sum over k in the same order whatever the tile order or where
// B lives, so all variants give identical bits.
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
//              10240-square product took 135 ms instead of 15.5 ms).
#include "device_common.h"

namespace dkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 128;
constexpr int kXcds = 8;

struct GemmOperands {
    uint4 a[4];
    uint4 b[4];
};

// STREAM_A: A is loaded nontemporally, so the HBM operand streams past the L2
// instead of evicting the B lines the other workgroups of the XCD will read.
template <bool STREAM_A>
__device__ __forceinline__ void gemm_load(GemmOperands &o, const uint16_t *const (&ar)[4],
                                          const uint16_t *const (&br)[4], int k) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
        o.a[t] = STREAM_A ? load_stream(ar[t] + k) : *reinterpret_cast<const uint4 *>(ar[t] + k);
#pragma unroll
    for (int t = 0; t < 4; ++t) o.b[t] = *reinterpret_cast<const uint4 *>(br[t] + k);
}

__device__ __forceinline__ void gemm_mma(f32x4 (&acc)[4][4], const GemmOperands &o) {
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, o.a[tm]),
                                                                  __builtin_bit_cast(bf16x8, o.b[tn]),
                                                                  acc[tm][tn], 0, 0, 0);
}

template <bool CPU_AWARE>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const uint16_t *__restrict__ A, const uint16_t *B,
                                                      float *__restrict__ C, int M, int N, int K) {
    const int nmb = M / kTile, nnb = N / kTile;
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
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 1, wn = wave & 1;
    const int i = lane & 15, kq = (lane >> 4) * 8;

    const uint16_t *ar[4], *br[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        ar[t] = A + (size_t)(mb * kTile + wm * 64 + t * 16 + i) * K + kq;
        br[t] = B + (size_t)(nb * kTile + wn * 64 + t * 16 + i) * K + kq;
    }
    f32x4 acc[4][4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // K is a multiple of 64: k steps of 32 come in pairs (ping-pong operands).
    GemmOperands o0, o1;
    gemm_load<CPU_AWARE>(o0, ar, br, 0);
    for (int k0 = 0; k0 < K; k0 += 64) {
        gemm_load<CPU_AWARE>(o1, ar, br, k0 + 32);
        gemm_mma(acc, o0);
        if (k0 + 64 < K) gemm_load<CPU_AWARE>(o0, ar, br, k0 + 64);
        gemm_mma(acc, o1);
    }

#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int col = nb * kTile + wn * 64 + tn * 16 + i;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mb * kTile + wm * 64 + tm * 16 + (lane >> 4) * 4 + r;
                C[(size_t)row * N + col] = acc[tm][tn][r];
            }
        }
}

}  // namespace

hipError_t launch_gemm_nt(const uint16_t *A, const uint16_t *B, float *C, int M, int N, int K,
                          bool cpu_aware, hipStream_t st) {
    const int blocks = (M / kTile) * (N / kTile);
    if (cpu_aware) gemm_nt_kernel<true><<<blocks, 256, 0, st>>>(A, B, C, M, N, K);
    else gemm_nt_kernel<false><<<blocks, 256, 0, st>>>(A, B, C, M, N, K);
    return hipGetLastError();
}

}  // namespace dkv
