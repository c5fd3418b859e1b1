/*
 * synth.c -- seeded, counter-based synthetic inputs (bf16 normals, uniform
 * integers) for the decode-step workloads.
 *
 * This module holds no part of the decode computation: it only turns
 * (seed, tensor id, stream id, element index) into numbers. Both the oracle's
 * tests and the GPU path's tests/benchmark draw their inputs from it, so that
 * the two sides see the same values without sharing any arithmetic.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), key = the 64-bit seed, counter =
 * (element block lo, element block hi, stream id, tensor id). One call yields
 * four 32-bit words; element 4*blk + j takes word j. Normals come from the
 * Box-Muller transform of word pairs (0,1) and (2,3) in fp64, then round to
 * nearest even straight from fp64 to bf16.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += PHILOX_W0;
            k1 += PHILOX_W1;
        }
        uint64_t p0 = (uint64_t)PHILOX_M0 * c0;
        uint64_t p1 = (uint64_t)PHILOX_M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

static void block_words(uint64_t seed, uint32_t tensor, uint32_t stream,
                        uint64_t blk, uint32_t w[4])
{
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), stream, tensor};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    synth_philox4x32_10(ctr, key, w);
}

/* The four standard normals of Philox block blk: Box-Muller of word pairs
 * (0, 1) -> elements 0 (cos) and 1 (sin), (2, 3) -> elements 2 and 3. */
static void normal_block(uint64_t seed, uint32_t tensor, uint32_t stream, uint64_t blk,
                         double z[4])
{
    uint32_t w[4];
    block_words(seed, tensor, stream, blk, w);
    for (int pair = 0; pair < 2; ++pair) {
        const double u1 = ((double)w[2 * pair] + 1.0) * (1.0 / 4294967296.0);  /* (0, 1] */
        const double u2 = (double)w[2 * pair + 1] * (1.0 / 4294967296.0);      /* [0, 1) */
        const double r = sqrt(-2.0 * log(u1));
        const double t = 6.283185307179586476925286766559 * u2;
        z[2 * pair] = r * cos(t);
        z[2 * pair + 1] = r * sin(t);
    }
}

/* Standard normal for element idx of (seed, tensor, stream). */
static double normal_at(uint64_t seed, uint32_t tensor, uint32_t stream, uint64_t idx)
{
    double z[4];
    normal_block(seed, tensor, stream, idx >> 2, z);
    return z[idx & 3];
}

/* fp64 -> bf16, round to nearest even straight from the 53-bit significand
 * (no double rounding through fp32). Finite inputs of normal bf16 range
 * (|x| >= 2^-126) take the bit path; others the exact slow path. */
static uint16_t to_bf16_slow(double x)
{
    if (x == 0.0) return signbit(x) ? 0x8000u : 0u;
    int e;
    (void)frexp(x, &e);
    int qe = e - 8;
    if (qe < -133) qe = -133;
    const double v = ldexp(nearbyint(ldexp(x, -qe)), qe);
    const float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static uint16_t to_bf16(double x)
{
    uint64_t b;
    memcpy(&b, &x, sizeof b);
    const int bexp = (int)((b >> 52) & 0x7FF);
    if (bexp < 1023 - 126 || bexp > 1023 + 126) return to_bf16_slow(x);
    /* keep 7 fraction bits: drop 45, round half to even on the dropped bits */
    const uint64_t drop = 45;
    const uint64_t half = (uint64_t)1 << (drop - 1);
    const uint64_t low = b & (((uint64_t)1 << drop) - 1);
    uint64_t keep = b >> drop;                      /* sign | exp(11) | frac(7) */
    if (low > half || (low == half && (keep & 1))) keep += 1;   /* may carry into exp */
    const uint64_t sign = keep >> 18;
    const int64_t e11 = (int64_t)((keep >> 7) & 0x7FF);
    const uint64_t frac7 = keep & 0x7F;
    const uint64_t e8 = (uint64_t)(e11 - 1023 + 127);
    if (e8 >= 255) return to_bf16_slow(x);
    return (uint16_t)((sign << 15) | (e8 << 7) | frac7);
}

/* Elements [offset, offset + n) of one stream, block by block, on the
 * calling thread. */
static void fill_range(uint64_t seed, uint32_t tensor, uint32_t stream, uint64_t offset,
                       uint64_t n, double sigma, uint16_t *out)
{
    if (n == 0) return;
    const uint64_t end = offset + n;
    for (uint64_t bi = offset >> 2; (bi << 2) < end; ++bi) {
        double z[4];
        normal_block(seed, tensor, stream, bi, z);
        for (int j = 0; j < 4; ++j) {
            const uint64_t idx = (bi << 2) + (uint64_t)j;
            if (idx >= offset && idx < end) out[idx - offset] = to_bf16(sigma * z[j]);
        }
    }
}

/* out[i] = bf16(sigma * N(seed, tensor, stream, offset + i)), i < n. */
void synth_normal_bf16(uint64_t seed, uint32_t tensor, uint32_t stream,
                       uint64_t offset, uint64_t n, double sigma,
                       uint16_t *out, int n_threads)
{
    if (n_threads < 1) n_threads = 1;
    const uint64_t chunk = 1u << 16;
    const int64_t n_chunks = (int64_t)((n + chunk - 1) / chunk);
    #pragma omp parallel for num_threads(n_threads) schedule(dynamic, 1)
    for (int64_t c = 0; c < n_chunks; ++c) {
        const uint64_t a = (uint64_t)c * chunk;
        const uint64_t m = n - a < chunk ? n - a : chunk;
        fill_range(seed, tensor, stream, offset + a, m, sigma, out + a);
    }
}

/* Row-strided variant: n_rows rows of row_len elements; row r starts at
 * element offset + r * src_stride of the stream and is written at
 * out + r * dst_stride. Lets a caller draw one head's slice of a larger
 * logical tensor without generating the rest. */
void synth_normal_bf16_rows(uint64_t seed, uint32_t tensor, uint32_t stream,
                            uint64_t offset, uint64_t n_rows, uint64_t row_len,
                            uint64_t src_stride, double sigma,
                            uint16_t *out, uint64_t dst_stride, int n_threads)
{
    if (n_threads < 1) n_threads = 1;
    #pragma omp parallel for num_threads(n_threads) schedule(static, 256)
    for (int64_t r = 0; r < (int64_t)n_rows; ++r)
        fill_range(seed, tensor, stream, offset + (uint64_t)r * src_stride, row_len, sigma,
                   out + (uint64_t)r * dst_stride);
}

/* fp64 normals (for distribution tests of the generator itself). */
void synth_normal_f64(uint64_t seed, uint32_t tensor, uint32_t stream,
                      uint64_t offset, uint64_t n, double *out)
{
    for (uint64_t i = 0; i < n; ++i) out[i] = normal_at(seed, tensor, stream, offset + i);
}

/* Uniform integer in [lo, hi] for element idx (multiply-shift reduction of
 * one 32-bit word; bias below 2^-32 * (hi - lo + 1)). */
static int64_t uniform_at(uint64_t seed, uint32_t tensor, uint32_t stream,
                          uint64_t idx, int64_t lo, int64_t hi)
{
    uint32_t w[4];
    block_words(seed, tensor, stream, idx >> 2, w);
    const uint64_t range = (uint64_t)(hi - lo) + 1u;
    return lo + (int64_t)(((uint64_t)w[idx & 3] * range) >> 32);
}

void synth_uniform_i32(uint64_t seed, uint32_t tensor, uint32_t stream,
                       uint64_t offset, uint64_t n, int64_t lo, int64_t hi,
                       int32_t *out)
{
    for (uint64_t i = 0; i < n; ++i)
        out[i] = (int32_t)uniform_at(seed, tensor, stream, offset + i, lo, hi);
}

/* Small integers in [lo, hi] stored as bf16 (exact for |v| <= 256). */
void synth_int_bf16(uint64_t seed, uint32_t tensor, uint32_t stream,
                    uint64_t offset, uint64_t n, int32_t lo, int32_t hi,
                    uint16_t *out, int n_threads)
{
    if (n_threads < 1) n_threads = 1;
    #pragma omp parallel for num_threads(n_threads) schedule(static, 65536)
    for (int64_t i = 0; i < (int64_t)n; ++i)
        out[i] = to_bf16((double)uniform_at(seed, tensor, stream, offset + (uint64_t)i, lo, hi));
}
