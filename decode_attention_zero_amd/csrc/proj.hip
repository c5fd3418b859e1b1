// QKV projection of one decode step on gfx950: y_b = W_qkv x_b for every
// sequence b, fp32 accumulation of exact bf16 products, written as fp32 sums
// (one slab per range of the hidden dimension) for the fresh-token kernel,
// which adds them, keeps the query in fp32 and rounds the new token's K and
// V once. The projection that produces the new token's K/V is part of the
// decode step, as in the core-method section of the DirectKV digest
// ("长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）"); up to a few hundred
// sequences the step is bound by reading W from HBM, so three forms (1a VALU
// GEMV below batch 8, 1c split-k MFMA from batch 8, and 1b one 16-sequence
// MFMA tile, which a layout takes up to batch 15 when
// DKV_PROJ_SPLITK_MIN_BATCH moves the split-k threshold up) are built to
// stream W once at full bandwidth; past that the product is bound by the
// matrix cores, and a fourth form (1d, from 192 sequences) tiles both
// operands in LDS.
#include "mfma_tile.h"

namespace dkv {
namespace {

// Below batch 16 every form writes one slab: y of output row n of sequence b.
__device__ __forceinline__ void store_projection(const StepArgs &a, int n, int b, float y) {
    a.proj_part[(size_t)b * a.n_qkv + n] = y;
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

// 1a. Small batches (below 8 sequences): a GEMV on VALU. W is read with
// nontemporal loads (W read cold, batches 1-4: 1-5 % faster than plain loads;
// the MFMA kernels below keep plain loads, with which they measured 2-16 %
// faster). A workgroup owns 4 W rows and BT
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

    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.0f;

    const uint16_t *w0 = a.w + (size_t)row0 * a.hidden;
#pragma unroll 2
    for (int k = kbeg + lane * 8; k < kbeg + krange; k += 512) {
        float wf[4][8];
#pragma unroll
        for (int r = 0; r < 4; ++r) unpack8(load_stream(w0 + (size_t)r * a.hidden + k), wf[r]);
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

// Matrix-core operands below use the 16x16x32 MFMA layout: lane l supplies
// A[i = l%16][k = 8*(l/16) .. +7] and B[k = 8*(l/16) .. +7][j = l%16], and
// receives D[i = 4*(l/16) + r][j = l%16], r < 4. A is a W tile (W rows are
// contiguous in k, so a lane's operand is one 16-byte load), B is x^T.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NK>
__device__ __forceinline__ void load_slice(uint4 (&v)[NK], const uint16_t *row, int k0) {
#pragma unroll
    for (int u = 0; u < NK; ++u) v[u] = *reinterpret_cast<const uint4 *>(row + k0 + 32 * u);
}

// 1b. Up to 16 sequences (one tile of 16), below the split-k threshold: each workgroup owns 16 W
// rows; its KSPLIT wavefronts split the hidden dimension into equal ranges,
// and each walks its range in KC-wide chunks (128, or 256 for ranges of 2048
// and more). A wave stages its x chunk (the
// 16 sequences' 128 k values, loaded as contiguous 256-byte row pieces; rows
// past the batch as zeros) in its own LDS slot and reads the MFMA B operands
// from there; the next x chunk is prefetched into registers and the next W
// chunk is in flight (ping-pong registers) while the current chunk's MFMAs
// run. The KSPLIT partial tiles are added through LDS in wave order. (Loading
// the x operand straight from L2 in the MFMA layout, 16 rows x 64 B per load,
// measured 17.7 us for the projection of a decode step at batch 8 and hidden
// 4096, HIP events, against 14.5 us this way; at hidden 8192 the two are
// within 5 %. The MFMA k order, and so every bit, is the same.)
template <int KSPLIT, int KC = 128>
__global__ __launch_bounds__(64 * KSPLIT) void qkv_proj_stream_kernel(StepArgs a) {
    constexpr int NK = KC / 32;         // MFMA k steps per chunk
    constexpr int XROW = KC * 2 + 16;   // staged x row, bytes (padded by 16)
    constexpr int XPT = 16 * KC / 8 / 64;   // 16-byte x pieces per lane per chunk
    __shared__ __attribute__((aligned(16))) char xs[KSPLIT][16][XROW];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int row0 = blockIdx.x * 16;
    const int krange = a.hidden / KSPLIT;      // a multiple of 128 (checked at launch)
    const int kb = wave * krange;
    const int nch = krange / KC;

    const uint16_t *wrow = a.w + (size_t)(row0 + i) * a.hidden + kb + kq;
    char *xw = xs[wave][0];
    uint4 xr[XPT];
    auto load_x = [&](int c) {
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int v = lane + 64 * j;
            const int r = v / (KC / 8), cc = v % (KC / 8);
            xr[j] = r < a.batch ? *reinterpret_cast<const uint4 *>(a.x + (size_t)r * a.hidden + kb + c * KC + cc * 8)
                                : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int v = lane + 64 * j;
            *reinterpret_cast<uint4 *>(xw + (v / (KC / 8)) * XROW + (v % (KC / 8)) * 16) = xr[j];
        }
    };
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const uint4 (&wv)[NK]) {
#pragma unroll
        for (int u = 0; u < NK; ++u) {
            const uint4 xv = *reinterpret_cast<const uint4 *>(xw + i * XROW + (32 * u + kq) * 2);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[u]),
                                                          __builtin_bit_cast(bf16x8, xv), acc, 0, 0, 0);
        }
    };

    uint4 wa[NK], wb[NK];
    load_x(0);
    load_slice(wa, wrow, 0);
    store_x();
    __syncthreads();
    if (nch > 1) {
        load_x(1);
        load_slice(wb, wrow, KC);
    }
    // Chunk c from `cur` and the staged x; then x chunk c + 1 replaces it in
    // LDS, and chunk c + 2's loads go out into `cur` and the x registers.
    auto step = [&](uint4 (&cur)[NK], int c) {
        compute(cur);
        if (c + 1 < nch) {
            __syncthreads();
            store_x();
            __syncthreads();
        }
        if (c + 2 < nch) {
            load_x(c + 2);
            load_slice(cur, wrow, (c + 2) * KC);
        }
    };
    for (int c = 0; c < nch; c += 2) {
        step(wa, c);
        if (c + 1 < nch) step(wb, c + 1);
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

// 1c. From 8 sequences: W crosses HBM once; what limits a plain tiling is
// x. Every 16-row W tile needs the whole batch's x slice, so reading x per
// wavefront from L2 costs B/16 times the W bytes (measured on MI355X at hidden
// 4096: 19 -> 41 us from batch 16 to 64, linear in that x traffic; W alone is
// 6.3 us at 8 TB/s). Here a workgroup of four wavefronts owns 64 W
// rows (16 per wave) and one of KS equal ranges of the hidden dimension, and
// walks its range in KC-wide chunks: each chunk of x (up to 64 sequences) is
// staged once in LDS and read by all four waves, which cuts x's L2 traffic to
// B/64 of W. The next x chunk is prefetched into registers and the next W
// chunk is in flight (ping-pong register buffers) while the current chunk's
// MFMAs run. Each workgroup writes its fp32 partial tile to its range's slab
// of the step's scratch, and the fresh-token kernel adds the KS slabs of its
// group's rows in range order. Other ways of adding the partials measured
// slower: the last workgroup of each row block to finish doing it (2-10x: its
// device-scope fences write back the L2), one workgroup per row block holding
// every range (~2x: 96 workgroups fill too few CUs), and the split kernel's
// consumers adding them when they read q (every split item re-reads KS
// partials: +4 % on the all-HBM split kernel).
constexpr int kProjRowBlocks = 4;        // 16-row W blocks per workgroup, one per wavefront

// NBT tiles of 16 sequences (batch tile b0 = blockIdx.z * 16 * NBT), KC-wide chunks.
template <int NBT, int KC>
__global__ __launch_bounds__(64 * kProjRowBlocks) void qkv_proj_splitk_kernel(StepArgs a, int krange) {
    constexpr int NT = 64 * kProjRowBlocks;
    constexpr int NK = KC / 32;                 // MFMA k steps per chunk
    constexpr int XROW = KC * 2 + 16;           // staged x row, bytes (padded by 16)
    constexpr int XV = 16 * NBT * KC / 8;       // 16-byte pieces of one x chunk
    constexpr int XPT = (XV + NT - 1) / NT;     // of those, per thread
    __shared__ __attribute__((aligned(16))) char xs[16 * NBT][XROW];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int i = lane & 15;
    const int kq = (lane >> 4) * 8;
    const int row0 = (blockIdx.x * kProjRowBlocks + wave) * 16;
    const int ks = blockIdx.y;
    const int b0 = blockIdx.z * 16 * NBT;
    const int kb = ks * krange;
    const int nch = krange / KC;
    const uint16_t *wrow = a.w + (size_t)(row0 + i) * a.hidden + kb + kq;

    // x chunk c: piece v is sequence b0 + v / (KC/8), k offset 8 * (v % (KC/8));
    // sequences past the batch stage zeros (their columns are never stored).
    uint4 xr[XPT];
    auto load_x = [&](int c) {
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int v = threadIdx.x + j * NT;
            const int r = v / (KC / 8), cc = v % (KC / 8);
            xr[j] = (v < XV && b0 + r < a.batch)
                        ? *reinterpret_cast<const uint4 *>(a.x + (size_t)(b0 + r) * a.hidden + kb + c * KC + cc * 8)
                        : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto store_x = [&]() {
#pragma unroll
        for (int j = 0; j < XPT; ++j) {
            const int v = threadIdx.x + j * NT;
            if (v < XV) *reinterpret_cast<uint4 *>(&xs[v / (KC / 8)][(v % (KC / 8)) * 16]) = xr[j];
        }
    };

    f32x4 acc[NBT];
#pragma unroll
    for (int t = 0; t < NBT; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const uint4 (&wv)[NK]) {
#pragma unroll
        for (int u = 0; u < NK; ++u)
#pragma unroll
            for (int t = 0; t < NBT; ++t) {
                const uint4 xv = *reinterpret_cast<const uint4 *>(&xs[16 * t + i][(32 * u + kq) * 2]);
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wv[u]),
                                                                 __builtin_bit_cast(bf16x8, xv), acc[t], 0, 0, 0);
            }
    };

    uint4 wa[NK], wb[NK];
    load_x(0);
    load_slice(wa, wrow, 0);
    store_x();
    __syncthreads();
    if (nch > 1) {
        load_x(1);
        load_slice(wb, wrow, KC);
    }
    // Chunk c from `cur` and the staged x; then x chunk c + 1 replaces it in
    // LDS, and chunk c + 2's loads go out into `cur` and the x registers.
    auto step = [&](uint4 (&cur)[NK], int c) {
        compute(cur);
        if (c + 1 < nch) {
            __syncthreads();
            store_x();
            __syncthreads();
        }
        if (c + 2 < nch) {
            load_x(c + 2);
            load_slice(cur, wrow, (c + 2) * KC);
        }
    };
    for (int c = 0; c < nch; c += 2) {
        step(wa, c);
        if (c + 1 < nch) step(wb, c + 1);
    }

#pragma unroll
    for (int t = 0; t < NBT; ++t) {
        const int b = b0 + 16 * t + i;
        if (b < a.batch) {
            float *pp = a.proj_part + ((size_t)ks * a.batch + b) * a.n_qkv + row0 + 4 * (lane >> 4);
            *reinterpret_cast<float4 *>(pp) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
        }
    }
}

// 1d. From kProjTiledMinBatch sequences the product is no longer bound by
// reading W but by the matrix cores, and the split-k kernel's 64 x 64
// (W rows x sequences) workgroup tile re-reads W for every 64 sequences.
// Here a workgroup computes a (64 WM sequences) x (128 W rows) tile of y over
// one range of the hidden dimension with the LDS-staged matrix-core tile
// product of mfma_tile.h (x and W staged per 64-wide k step; sequences past
// the batch load zeros and are not stored). When the W tiles divide into the
// 8 XCDs, all sequence tiles of one W tile go to one XCD (the dispatcher
// deals workgroups to the XCDs in turn), so each W tile is fetched into one
// L2 and re-read from there.
constexpr int kProjTiledMinBatch = 192;

template <int WM>
__global__ __launch_bounds__(128 * WM, WM == 4 ? 2 : 1) void qkv_proj_tiled_kernel(StepArgs a, int krange,
                                                                                  int w_tiles, int b_tiles) {
    using T = tile::Shape<WM>;
    __shared__ __attribute__((aligned(16))) char lds[2][T::STAGE];
    const int id = blockIdx.x;
    int bt, wt;
    if (w_tiles % 8 == 0) {
        const int xcd = id % 8, local = id / 8;
        bt = local % b_tiles;
        wt = xcd + 8 * (local / b_tiles);
    } else {
        bt = id % b_tiles;
        wt = id / b_tiles;
    }
    const int b0 = bt * T::BM, n0 = wt * tile::kN;
    const int ks = blockIdx.y;

    f32x4 acc[4][4];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    // krange is a multiple of 64. Only the last sequence tile can run past the
    // batch; the others skip the row check (which cost the HBM-operand GEMM
    // 18 % on MI355X).
    const int k0 = ks * krange, nk = krange / tile::kStepK;
    if (b0 + T::BM <= a.batch) tile::product<WM, false, false>(acc, lds, a.x, a.w, a.hidden, b0, a.batch, n0, k0, nk);
    else tile::product<WM, false, true>(acc, lds, a.x, a.w, a.hidden, b0, a.batch, n0, k0, nk);

    // acc[tm][tn][r]: sequence b0 + 64 wm + 16 tm + 4 kq + r, W row n0 + 64 wn + 16 tn + i.
    const tile::Lane ln;
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int b = b0 + ln.wm * 64 + tm * 16 + ln.kq * 4 + r;
            if (b >= a.batch) continue;
            float *row = a.proj_part + ((size_t)ks * a.batch + b) * a.n_qkv + n0 + ln.wn * 64 + ln.i;
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) row[tn * 16] = acc[tm][tn][r];
        }
}

// Number of ranges of the hidden dimension: the largest of 8, 4, 2, 1 that
// leaves whole KC-wide chunks and ranges of at least `min_range`.
int splitk_ranges(int hidden, int kc, int min_range) {
    for (int ks = kProjMaxSplits; ks > 1; ks >>= 1)
        if (hidden % (ks * kc) == 0 && hidden / ks >= min_range) return ks;
    return 1;
}

// 256-wide chunks in up to 8 ranges of at least 256 (8 ranges from hidden
// 2048), and at most 8 (range, batch tile) pairs per row block: every range
// writes a slab of the whole batch, which the fresh-token kernel reads back,
// and every batch tile reads W again, so past one 64-sequence tile fewer
// ranges win. Measured on MI355X (W cycled through copies so that it is read
// from HBM, decode-step HIP events, projection + fresh-token kernel, hidden
// 4096 / 8192): up to batch 64, 8 ranges best or equal (batch 8, 14.4 /
// 36.5 us for the projection against 15.1 / 43.1 with 4 ranges; batch 64,
// 27.1 / 53.7 against 27.0 / 57.1); batch 128, 4 ranges 34.2 / 82.6 against
// 38.5 / 87.7 with 8; batch 256, 2 ranges 50.5 / 136.5 against 61.7 /
// 148.7; batch 512, one range 85.3 / 228.1 against 107.3 / 283.2; batch
// 1024, one range 145.6 / 425.0 against 199.3 / 542.9.
template <int NBT>
int launch_splitk(const StepArgs &a, hipStream_t st) {
    const int tiles = (a.batch + 16 * NBT - 1) / (16 * NBT);
    int ks = splitk_ranges(a.hidden, 256, 256);
    while (ks > 1 && ks * tiles > kProjMaxSplits) ks >>= 1;
    if (a.proj_ranges > 0 && a.hidden % (a.proj_ranges * 256) == 0) ks = a.proj_ranges;
    const dim3 grid(a.n_qkv / (16 * kProjRowBlocks), ks, tiles);
    qkv_proj_splitk_kernel<NBT, 256><<<grid, 64 * kProjRowBlocks, 0, st>>>(a, a.hidden / ks);
    return ks;
}

// Tiles of 256 sequences x 128 W rows (one workgroup of 8 wavefronts per CU:
// 108 KiB of LDS). Two ranges of the hidden dimension when that halves the
// work per round of workgroups (256 at a time), else one: more ranges mean
// more fp32 slabs written and read back, and measured slower.
// DKV_PROJ_RANGES overrides the count.
constexpr int kTiledWM = 4;

int tiled_ranges(const StepArgs &a, int tiles) {
    auto rounds = [](int wgs) { return (wgs + 255) / 256; };
    return 2 * rounds(tiles) > rounds(2 * tiles) && a.hidden % (2 * tile::kStepK) == 0 ? 2 : 1;
}

int tiled_tiles(const StepArgs &a) {
    return (a.batch + 64 * kTiledWM - 1) / (64 * kTiledWM) * (a.n_qkv / tile::kN);
}

// The tiled form from 192 sequences, once its workgroups fill half the CUs;
// below that the split-k kernel is faster. Measured on MI355X (W cycled
// through copies so that it is read from HBM, decode-step HIP events,
// projection + fresh-token kernel, split-k / tiled with the row check on
// every tile): hidden 4096 (48 W tiles), batch 256, 52.0 / 57.9 us; 384,
// 81.0 / 60.8; 512, 84.1 / 62.9; 1024, 143.9 / 107.2; hidden 8192 (80 W
// tiles), batch 128, 83.5 / 91.6; 192, 110.9 / 98.4; 256, 134.4 / 105.5;
// 512, 225.7 / 186.9; 1024, 423.6 / 304.8. With the check on the last tile
// only, the tiled kernel takes 56.7 / 60.0 / 98.4 us at hidden 4096, batch
// 384 / 512 / 1024, and 104.7 / 170.6 / 273.4 us at hidden 8192, batch 256 /
// 512 / 1024.
bool tiled_pays(const StepArgs &a) {
    if (a.batch < kProjTiledMinBatch || a.n_qkv % tile::kN != 0) return false;
    const int tiles = tiled_tiles(a);
    return tiles * tiled_ranges(a, tiles) >= 128;
}

int launch_tiled(const StepArgs &a, hipStream_t st) {
    const int b_tiles = (a.batch + 64 * kTiledWM - 1) / (64 * kTiledWM);
    const int w_tiles = a.n_qkv / tile::kN;
    const int tiles = b_tiles * w_tiles;
    const int r = a.proj_ranges > 0 && a.hidden % (a.proj_ranges * tile::kStepK) == 0 ? a.proj_ranges
                                                                                    : tiled_ranges(a, tiles);
    const dim3 grid(tiles, r);
    qkv_proj_tiled_kernel<kTiledWM><<<grid, 128 * kTiledWM, 0, st>>>(a, a.hidden / r, w_tiles, b_tiles);
    return r;
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

int projection_form(const StepArgs &a) {
    if (a.batch < a.proj_mfma_min_batch) return kProjGemv;
    if (a.batch < a.proj_splitk_min_batch && a.batch <= 16) return kProjStream;
    return tiled_pays(a) ? kProjTiled : kProjSplitk;
}

hipError_t launch_projection(const StepArgs &a, int *ranges, hipStream_t st) {
    if (a.hidden % 512 != 0 || a.n_qkv % (16 * kProjRowBlocks) != 0 || !a.proj_part) return hipErrorInvalidValue;
    *ranges = 1;
    switch (projection_form(a)) {
        case kProjStream: {
            // One sequence tile: streamed over k by up to 4 wavefronts per row block.
            int ksplit = 4;
            while (ksplit > 1 && a.hidden % (128 * ksplit) != 0) ksplit >>= 1;
            const dim3 grid(a.n_qkv / 16);
            // 256-wide chunks once each wave's range reaches 2048 (hidden 8192 at
            // batch 8: 45.7 -> 42.1 us; at hidden 4096, ranges of 1024, 128-wide
            // chunks stay ahead: 16.7 vs 18.9 us; decode-step HIP events, W
            // evicted from the caches).
            if (ksplit == 4 && a.hidden % 1024 == 0 && a.hidden / 4 >= 2048)
                qkv_proj_stream_kernel<4, 256><<<grid, 256, 0, st>>>(a);
            else switch (ksplit) {
                case 1: qkv_proj_stream_kernel<1><<<grid, 64, 0, st>>>(a); break;
                case 2: qkv_proj_stream_kernel<2><<<grid, 128, 0, st>>>(a); break;
                default: qkv_proj_stream_kernel<4><<<grid, 256, 0, st>>>(a); break;
            }
            break;
        }
        case kProjTiled:
            *ranges = launch_tiled(a, st);
            break;
        case kProjSplitk:
            if (a.batch <= 16) *ranges = launch_splitk<1>(a, st);
            else if (a.batch <= 32) *ranges = launch_splitk<2>(a, st);
            else *ranges = launch_splitk<4>(a, st);
            break;
        default:
            if (a.batch <= 4) (void)launch_gemv<4>(a, st);
            else if (a.batch <= 8) (void)launch_gemv<8>(a, st);
            else (void)launch_gemv<16>(a, st);
            break;
    }
    return hipGetLastError();
}

}  // namespace dkv
