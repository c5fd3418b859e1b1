/*
 * oracle.c -- plain fp64 CPU oracle for one decode step of zero-copy decode
 * attention (QKV projection followed by softmax attention over the cached
 * keys/values plus the freshly projected token).
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library. The GPU path
 * never calls, links or includes anything from here, and nothing here uses
 * any code of the GPU path.
 *
 * Sources. The pages describe the method only in prose:
 *  - "长上下文 LLM 的零拷贝 KV Cache 卸载（OSDI 2026）" (DirectKV digest,
 *    awesome-system-papers), section 核心方法 (core method): the attention
 *    kernel reads CPU-resident KV in place, and the QKV projection that
 *    generates the new K/V is fused with the attention that consumes them.
 *  - "KV Cache 内存层级" series overview (10100.com), section 2.1 去搬运：
 *    DirectKV: one launch does the QKV projection and the attention.
 * Neither page writes down a formula. What is computed here is therefore the
 * textbook definition of a single-query decode step with grouped KV heads:
 *     y      = W x                          (W row-major [N_qkv][hidden])
 *     q_h    = y[h*d : (h+1)*d]             h < Hq
 *     k_new  = y[Hq*d + g*d : ...]          g < Hkv
 *     v_new  = y[(Hq+Hkv)*d + g*d : ...]
 *     keys   = K_0 .. K_{L-1} (cache), K_L = k_new(g(h)), g(h) = floor(h / (Hq/Hkv))
 *     s_j    = (q_h . K_j) / sqrt(d)
 *     o_h    = sum_j exp(s_j - max s) V_j / sum_j exp(s_j - max s)
 * All arithmetic is fp64; inputs are exact bf16 values; nothing is rounded.
 * The softmax is two-pass and unsplit, so any split/merge a fast path uses is
 * checked against it rather than assumed.
 *
 * Pins: every function below is checked by the CPU tests against closed forms
 * (one-token context, equal scores, shift invariance, affine-in-V, planted
 * token, permutation), against library routines (numpy matmul for the
 * projection, torch's fp64 scaled-dot-product attention on tiny shapes), and by
 * mutation tests that compile deliberately broken copies of this file (a
 * dropped term, a wrong scale, sign, index or operand order) and require some
 * pin to fail for each.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- bf16 <-> fp64 -------------------------------------------------------
 * bf16 is the upper 16 bits of an IEEE-754 binary32. Decoding is exact. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round-to-nearest-even from fp64 straight to bf16 (8 significant bits),
 * without an intermediate fp32 rounding (which could round twice). Finite
 * inputs only; results beyond the bf16 range become +-inf. */
uint16_t oracle_f64_to_bf16(double x)
{
    if (x == 0.0) {
        return signbit(x) ? 0x8000u : 0x0000u;
    }
    int e;
    (void)frexp(x, &e);                /* |x| = m * 2^e, m in [0.5, 1) */
    int qexp = e - 8;                  /* quantum of an 8-bit significand */
    if (qexp < -133) qexp = -133;      /* bf16 subnormal quantum 2^-133 */
    double r = nearbyint(ldexp(x, -qexp));   /* default mode: ties to even */
    double v = ldexp(r, qexp);
    float f = (float)v;                /* exact: at most 9 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* ---- projection ------------------------------------------------------------
 * y[n] = sum_k W[n][k] * x[k], fp64 accumulation in index order. */
void oracle_qkv_projection(const uint16_t *x, const uint16_t *W,
                           int64_t hidden, int64_t n_out, double *y)
{
#pragma omp parallel for schedule(static) if (n_out * hidden > (1 << 20))
    for (int64_t n = 0; n < n_out; ++n) {
        const uint16_t *w = W + n * hidden;
        double acc = 0.0;
        for (int64_t k = 0; k < hidden; ++k) {
            acc += oracle_bf16_to_f64(w[k]) * oracle_bf16_to_f64(x[k]);
        }
        y[n] = acc;
    }
}

/* ---- attention over one query head ----------------------------------------
 * Key/value j for j in [0, L) is row j of the cache (bf16, rows tok_stride
 * elements apart); j == L is the fresh token (fp64). */
static double key_elem(const uint16_t *K, int64_t tok_stride, int64_t L,
                       const double *k_new, int64_t j, int64_t i)
{
    return j < L ? oracle_bf16_to_f64(K[j * tok_stride + i]) : k_new[i];
}

static double score(const double *q, int64_t d, const uint16_t *K,
                    int64_t tok_stride, int64_t L, const double *k_new,
                    int64_t j, double scale)
{
    double acc = 0.0;
    for (int64_t i = 0; i < d; ++i) {
        acc += q[i] * key_elem(K, tok_stride, L, k_new, j, i);
    }
    return acc * scale;
}

double oracle_softmax_scale(int64_t d)
{
    return 1.0 / sqrt((double)d);
}

/* Softmax attention of query q over keys/values 0..L (L cached + the fresh
 * one). Two passes: scores and their maximum, then normalised weights.
 * Returns 0, or -1 (out untouched) when the score buffer cannot be had. */
int oracle_attention_head(const double *q, int64_t d,
                          const uint16_t *K, const uint16_t *V,
                          int64_t tok_stride, int64_t L,
                          const double *k_new, const double *v_new,
                          double *out)
{
    const double scale = oracle_softmax_scale(d);
    const int64_t n = L + 1;
    double *s = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!s) return -1;
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = score(q, d, K, tok_stride, L, k_new, j, scale);
        if (s[j] > m) m = s[j];
    }
    double denom = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        s[j] = exp(s[j] - m);
        denom += s[j];
    }
    for (int64_t i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double v = j < L ? oracle_bf16_to_f64(V[j * tok_stride + i]) : v_new[i];
            acc += s[j] * v;
        }
        out[i] = acc / denom;
    }
    free(s);
    return 0;
}

/* Unnormalised softmax state of keys/values [t0, t1) of the same sequence of
 * L+1 keys: m = max s_j, l = sum exp(s_j - m), o = sum exp(s_j - m) V_j.
 * Used to check that merging such states over any partition gives the
 * unsplit result. */
void oracle_attention_partial(const double *q, int64_t d,
                              const uint16_t *K, const uint16_t *V,
                              int64_t tok_stride, int64_t L,
                              const double *k_new, const double *v_new,
                              int64_t t0, int64_t t1,
                              double *m_out, double *l_out, double *o)
{
    const double scale = oracle_softmax_scale(d);
    double m = -INFINITY;
    for (int64_t j = t0; j < t1; ++j) {
        double s = score(q, d, K, tok_stride, L, k_new, j, scale);
        if (s > m) m = s;
    }
    double l = 0.0;
    for (int64_t i = 0; i < d; ++i) o[i] = 0.0;
    for (int64_t j = t0; j < t1; ++j) {
        double p = exp(score(q, d, K, tok_stride, L, k_new, j, scale) - m);
        l += p;
        for (int64_t i = 0; i < d; ++i) {
            double v = j < L ? oracle_bf16_to_f64(V[j * tok_stride + i]) : v_new[i];
            o[i] += p * v;
        }
    }
    *m_out = m;
    *l_out = l;
}

/* Merge n_parts states (m_s, l_s, o_s[d]) in index order:
 * M = max m_s; out = sum e^(m_s - M) o_s / sum e^(m_s - M) l_s. */
void oracle_merge_partials(int64_t n_parts, int64_t d, const double *m,
                           const double *l, const double *o, double *out)
{
    double M = -INFINITY;
    for (int64_t s = 0; s < n_parts; ++s)
        if (m[s] > M) M = m[s];
    double denom = 0.0;
    for (int64_t s = 0; s < n_parts; ++s) denom += exp(m[s] - M) * l[s];
    for (int64_t i = 0; i < d; ++i) {
        double acc = 0.0;
        for (int64_t s = 0; s < n_parts; ++s) acc += exp(m[s] - M) * o[s * d + i];
        out[i] = acc / denom;
    }
}

/* GQA mapping: query head h reads KV head floor(h / (Hq / Hkv)). */
int64_t oracle_kv_head_of(int64_t h, int64_t n_q_heads, int64_t n_kv_heads)
{
    return h / (n_q_heads / n_kv_heads);
}

/* One decode step for a batch of B sequences.
 *   x        [B][hidden]                bf16 hidden states
 *   W        [(Hq+2Hkv)*d][hidden]      bf16 fused QKV weight
 *   ctx_lens [B]                        cached tokens per sequence (L_b)
 *   K, V     [B][Lmax][Hkv][d]          bf16 cache in logical order
 * Outputs (fp64): attn_out [B][Hq*d], k_new/v_new [B][Hkv*d] (may be NULL),
 * q_out [B][Hq*d] (may be NULL).
 * Returns 0, or -1 on an invalid argument. */
int oracle_decode_step(int64_t B, int64_t hidden, int64_t n_q_heads,
                       int64_t n_kv_heads, int64_t d,
                       const uint16_t *x, const uint16_t *W,
                       const int32_t *ctx_lens,
                       const uint16_t *K, const uint16_t *V, int64_t Lmax,
                       double *attn_out, double *k_new_out, double *v_new_out,
                       double *q_out, int n_threads)
{
    if (B < 0 || hidden <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || d <= 0 ||
        n_q_heads % n_kv_heads != 0)
        return -1;
    for (int64_t b = 0; b < B; ++b)
        if (ctx_lens[b] < 0 || ctx_lens[b] > Lmax) return -1;
    const int64_t n_out = (n_q_heads + 2 * n_kv_heads) * d;
    double *y = (double *)malloc((size_t)(B > 0 ? B : 1) * (size_t)n_out * sizeof(double));
    if (!y) return -1;
    if (n_threads < 1) n_threads = 1;

    #pragma omp parallel for num_threads(n_threads) schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b)
        oracle_qkv_projection(x + b * hidden, W, hidden, n_out, y + b * n_out);

    const int64_t tok_stride = n_kv_heads * d;
    int failed = 0;
    #pragma omp parallel for num_threads(n_threads) schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * n_q_heads; ++bh) {
        const int64_t b = bh / n_q_heads, h = bh % n_q_heads;
        const int64_t g = oracle_kv_head_of(h, n_q_heads, n_kv_heads);
        const double *yb = y + b * n_out;
        const double *q = yb + h * d;
        const double *kn = yb + n_q_heads * d + g * d;
        const double *vn = yb + (n_q_heads + n_kv_heads) * d + g * d;
        const uint16_t *Kb = K + (b * Lmax) * tok_stride + g * d;
        const uint16_t *Vb = V + (b * Lmax) * tok_stride + g * d;
        if (oracle_attention_head(q, d, Kb, Vb, tok_stride, ctx_lens[b], kn, vn,
                                  attn_out + b * n_q_heads * d + h * d) != 0) {
            #pragma omp atomic write
            failed = 1;
        }
    }
    for (int64_t b = 0; b < B; ++b) {
        const double *yb = y + b * n_out;
        if (q_out) memcpy(q_out + b * n_q_heads * d, yb, (size_t)(n_q_heads * d) * sizeof(double));
        if (k_new_out)
            memcpy(k_new_out + b * n_kv_heads * d, yb + n_q_heads * d,
                   (size_t)(n_kv_heads * d) * sizeof(double));
        if (v_new_out)
            memcpy(v_new_out + b * n_kv_heads * d, yb + (n_q_heads + n_kv_heads) * d,
                   (size_t)(n_kv_heads * d) * sizeof(double));
    }
    free(y);
    return failed ? -1 : 0;
}

/* ---- GEMM entries --------------------------------------------------------
 * C = A x B^T for the host-operand GEMM experiment ("KV Cache 内存层级"
 * overview, opening section, Fig. 2(a); 2.1 去搬运：DirectKV, CPU-aware
 * tiling): out[e] = sum_k A[rows[e]][k] * B[cols[e]][k], A [M][K] and B [N][K]
 * bf16 bit patterns, row-major; fp64 sums in k order. Only the requested
 * entries are computed, so a 10240-square product can be sampled. */
void oracle_gemm_nt_entries(const uint16_t *A, const uint16_t *B, int64_t K,
                            const int64_t *rows, const int64_t *cols, int64_t n,
                            double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < n; ++e) {
        const uint16_t *a = A + rows[e] * K;
        const uint16_t *b = B + cols[e] * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_bf16_to_f64(a[k]) * oracle_bf16_to_f64(b[k]);
        out[e] = acc;
    }
}

