// Device helpers shared by the decode-step kernels (gfx950, wave64).
#pragma once

#include "dkv_internal.h"

namespace dkv {

constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// KV pages are streamed once per step: nontemporal 16-byte loads keep them
// from displacing reusable lines and measured ~13 % more HBM read bandwidth
// on gfx950 than plain loads for the same page-run pattern.
// The load goes through a global (address space 1) pointer: a generic
// pointer would make it a flat load, which also counts on the LDS counter, so
// any later wait for an LDS access would wait for every page load in flight.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1))) global_u32x4;
__device__ __forceinline__ uint4 load_stream(const void *p) {
    const u32x4 v = __builtin_nontemporal_load((global_u32x4 *)p);
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

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
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

// Work queue of the looping split kernels: the workgroup takes the next item
// index (one atomic per item); every workgroup ends on an index past the last
// item. The step's fresh-token kernel zeroes the counter first (reset_items),
// so the queue needs no memset and a captured step replays as it ran. Both
// use system scope, which makes them go through to memory, so the workgroups
// on all eight XCDs (each with its own L2) share one counter.
__device__ __forceinline__ int take_item(const StepArgs &a, int *slot) {
    __syncthreads();                   // the previous index has been read by every wave
    if (threadIdx.x == 0)
        *slot = (int)__hip_atomic_fetch_add(a.item_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    __syncthreads();
    return *slot;
}

__device__ __forceinline__ void reset_items(const StepArgs &a) {
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
        __hip_atomic_store(a.item_counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Work items of a step: split s of sequence b covers cached tokens
// [s T, min((s + 1) T, L)) with T = split_tokens and L = ctx_lens[b]; a
// sequence has ceil(L / T) of them, none when L is out of range. The
// fresh-token kernel lists them, sequence-major, in StepArgs::item_list; the
// split kernels map workgroup (KV head g, list entry j) to entry j, so every
// workgroup of the launch that has work comes before every one that has none
// (a grid with empty items interleaved among the real ones streamed 9 % fewer
// bytes per second on MI355X).
__device__ __forceinline__ int splits_of(const StepArgs &a, int b) {
    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) return 0;
    return (L + a.split_tokens - 1) / a.split_tokens;
}

// Entry j of the item list: false past its end. The entry is read at an
// index clamped into the list, so that both loads are in flight together.
__device__ __forceinline__ bool listed_item(const StepArgs &a, int j, int &b, int &s) {
    const uint32_t n = a.item_list[0];
    const uint32_t e = a.item_list[1 + min(j, a.batch * a.max_splits - 1)];
    if ((uint32_t)j >= n) return false;
    b = (int)(e >> 16);
    s = (int)(e & 0xFFFFu);
    return true;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Sequences whose ctx_lens entry is out of range raise the layout's flag.
__device__ __forceinline__ void check_context_range(const StepArgs &a, int b) {
    const int L = a.ctx_lens[b];
    if (L < 0 || L >= a.capacity[b]) atomicOr(a.status, 1u);
}

}  // namespace dkv
