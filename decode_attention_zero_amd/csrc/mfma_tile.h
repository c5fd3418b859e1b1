// An LDS-staged matrix-core tile product on gfx950, shared by the host-operand
// GEMM (gemm.hip) and the large-batch QKV projection (proj.hip):
//
//   acc += A[m0 .. m0 + 64 WM) x B[n0 .. n0 + 128)^T over k in [k0, k0 + 64 nk)
//
// with A and B bf16, row-major, both with leading dimension ld (elements), and
// fp32 accumulation. A workgroup of 2 WM wavefronts (WM along M, 2 along N)
// computes the (64 WM) x 128 tile; each wavefront a 64 x 64 block (4 x 4
// tiles of v_mfma_f32_16x16x32_bf16). The k loop runs in steps of 64: each
// step's A and B tiles are loaded from memory once per workgroup (16-byte
// chunks, eight lanes per 128-byte row), staged in LDS (rows padded to 144
// bytes, so the MFMA operand reads -- lane l takes row l % 16, k chunk l / 16
// -- are free of bank conflicts) and read from there by every wavefront that
// needs them. Loads run two steps ahead of the matrix cores: while step s is
// multiplied out of one LDS buffer, step s + 1 (already in registers) is
// written to the other and step s + 2 is in flight; one barrier per step.
// Every element of the tile is one fp32 sum over k in the same order whatever
// the tile order or where the operands live.
#pragma once

#include "device_common.h"

namespace dkv {
namespace tile {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kN = 128;                      // B rows per tile
constexpr int kStepK = 64;                   // k per step
constexpr int kRowBytes = kStepK * 2 + 16;   // staged row, padded

template <int WM>
struct Shape {
    static constexpr int BM = 64 * WM;                        // A rows per tile
    static constexpr int NT = 128 * WM;                       // threads
    static constexpr int ACH = BM * (kStepK / 8) / NT;        // A chunks per thread per step
    static constexpr int BCH = kN * (kStepK / 8) / NT;        // B chunks per thread per step
    static constexpr int STAGE = (BM + kN) * kRowBytes;       // LDS bytes per buffer
    static_assert(ACH >= 1 && BCH >= 1, "tile too small for its threads");
};

// Where this lane's accumulators land: acc[tm][tn][r] is element
// (m0 + 64 wm + 16 tm + 4 kq + r, n0 + 64 wn + 16 tn + i) of the product.
struct Lane {
    int wm, wn, i, kq;
    __device__ __forceinline__ Lane() {
        const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
        wm = wave >> 1;
        wn = wave & 1;
        i = lane & 15;
        kq = lane >> 4;
    }
};

// One step's operands in registers. With GUARD_A, rows of A at or past
// a_rows load zeros (without it, every row of the tile must exist); NT_A
// loads A with nontemporal loads (an operand that streams past the L2).
template <int WM, bool NT_A, bool GUARD_A>
struct Step {
    using S = Shape<WM>;
    uint4 a[S::ACH], b[S::BCH];

    __device__ __forceinline__ void load(const uint16_t *A, const uint16_t *B, int ld, int m0, int a_rows, int n0,
                                         int k0) {
        const int t = threadIdx.x;
#pragma unroll
        for (int c = 0; c < S::ACH; ++c) {
            const int chunk = t + c * S::NT;
            const int m = m0 + (chunk >> 3);
            const uint16_t *p = A + (size_t)m * ld + k0 + (chunk & 7) * 8;
            if (GUARD_A && m >= a_rows) a[c] = make_uint4(0u, 0u, 0u, 0u);
            else a[c] = NT_A ? load_stream(p) : *reinterpret_cast<const uint4 *>(p);
        }
#pragma unroll
        for (int c = 0; c < S::BCH; ++c) {
            const int chunk = t + c * S::NT;
            b[c] = *reinterpret_cast<const uint4 *>(B + (size_t)(n0 + (chunk >> 3)) * ld + k0 + (chunk & 7) * 8);
        }
    }

    __device__ __forceinline__ void stage(char *buf) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int c = 0; c < S::ACH; ++c) {
            const int chunk = t + c * S::NT;
            *reinterpret_cast<uint4 *>(buf + (chunk >> 3) * kRowBytes + (chunk & 7) * 16) = a[c];
        }
#pragma unroll
        for (int c = 0; c < S::BCH; ++c) {
            const int chunk = t + c * S::NT;
            *reinterpret_cast<uint4 *>(buf + (S::BM + (chunk >> 3)) * kRowBytes + (chunk & 7) * 16) = b[c];
        }
    }
};

// The wavefront's 4 x 4 MFMA tiles over one staged 64-wide k step.
__device__ __forceinline__ void multiply(f32x4 (&acc)[4][4], const char *a_rows, const char *b_rows) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        __builtin_amdgcn_sched_barrier(0);     // one half step's operands in registers at a time
        uint4 af[4], bf[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) af[t] = *reinterpret_cast<const uint4 *>(a_rows + t * 16 * kRowBytes + h * 64);
#pragma unroll
        for (int t = 0; t < 4; ++t) bf[t] = *reinterpret_cast<const uint4 *>(b_rows + t * 16 * kRowBytes + h * 64);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, af[tm]),
                                                                      __builtin_bit_cast(bf16x8, bf[tn]),
                                                                      acc[tm][tn], 0, 0, 0);
    }
}

// The tile product over nk >= 1 steps from k0, into zeroed or running
// accumulators, through the workgroup's two LDS buffers.
template <int WM, bool NT_A, bool GUARD_A>
__device__ __forceinline__ void product(f32x4 (&acc)[4][4], char (&lds)[2][Shape<WM>::STAGE], const uint16_t *A,
                                        const uint16_t *B, int ld, int m0, int a_rows, int n0, int k0, int nk) {
    const Lane ln;
    const int a_off = (ln.wm * 64 + ln.i) * kRowBytes + ln.kq * 16;
    const int b_off = (Shape<WM>::BM + ln.wn * 64 + ln.i) * kRowBytes + ln.kq * 16;
    // Register sets x and y alternate between the steps: at step s the other
    // set holds step s + 1, this one receives step s + 2.
    Step<WM, NT_A, GUARD_A> x, y;
    x.load(A, B, ld, m0, a_rows, n0, k0);
    x.stage(lds[0]);
    if (nk > 1) x.load(A, B, ld, m0, a_rows, n0, k0 + kStepK);
    __syncthreads();
    for (int s = 0; s < nk; s += 2) {
        // step s from lds[0]; x holds step s + 1
        if (s + 2 < nk) y.load(A, B, ld, m0, a_rows, n0, k0 + (s + 2) * kStepK);
        multiply(acc, lds[0] + a_off, lds[0] + b_off);
        if (s + 1 < nk) x.stage(lds[1]);
        __syncthreads();
        if (s + 1 >= nk) break;
        // step s + 1 from lds[1]; y holds step s + 2
        if (s + 3 < nk) x.load(A, B, ld, m0, a_rows, n0, k0 + (s + 3) * kStepK);
        multiply(acc, lds[1] + a_off, lds[1] + b_off);
        if (s + 2 < nk) y.stage(lds[0]);
        __syncthreads();
    }
}

}  // namespace tile
}  // namespace dkv
