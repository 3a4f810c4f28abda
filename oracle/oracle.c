/*
 * oracle.c -- plain, slow, CPU-only fp64 reference for batch-invariant forward
 * reductions.  TEST INFRASTRUCTURE ONLY: called by the test suite, by the
 * smoke check and by the bench's CPU-baseline leg; never by the product path.
 * It shares no code, header, table or constant with the HIP library.
 *
 * Every function computes the plain mathematical definition of its operation
 * in double precision from the exact stored input values (bf16 and fp32 widen
 * to fp64 without error).  No blocking, no fusion, no reordering beyond the
 * definition: loops run in index order.  Outer loops over independent rows /
 * heads are spread over OpenMP threads, which cannot change any result because
 * no reduction crosses threads.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "Reproducible LLM Inference - Batch Invariance, the Cost of Determinism,
 *       and Where Bitwise Identity Is Actually Required" (hidekazu-konishi.com)
 *  [P3] "Your Answer Depends on Who Else Is in the Batch" (praveentn.live)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2 };

static double widen_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load(const void *base, int dtype, int64_t i)
{
    switch (dtype) {
    case ORC_F32: return (double)((const float *)base)[i];
    case ORC_BF16: return widen_bf16(((const uint16_t *)base)[i]);
    default: return ((const double *)base)[i];
    }
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Round a double to the nearest bfloat16, ties to even, in ONE step (no pass
 * through fp32, which could round twice).  bfloat16 has 8 significand bits and
 * fp32's exponent range: normal minimum 2^-126, subnormal step 2^-133, largest
 * finite (2 - 2^-7) * 2^127.
 */
static uint16_t round_to_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double a = fabs(x);
    if (isinf(a))
        return sign | 0x7f80;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);              /* a = f * 2^e, f in [0.5, 1) -> leading bit 2^(e-1) */
    int lead = e - 1;
    if (lead < -126)
        lead = -126;           /* subnormal range: fixed step 2^-133 */
    double step = ldexp(1.0, lead - 7);
    double q = nearbyint(a / step);  /* default rounding mode: to nearest, ties even */
    double r = q * step;
    if (r > 3.3895313892515355e38) /* beyond (2 - 2^-7) * 2^127 after rounding */
        return sign | 0x7f80;
    float f = (float)r;        /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7fff);
}

void orc_round_bf16(const double *x, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = round_to_bf16(x[i]);
}

/*
 * RMSNorm, [P1] section 5.4 (root mean square over the feature dimension) and
 * [P3] "Where the reductions are" (a per-token sum of squares over the hidden
 * dimension) and "A Concrete Example" (divide by the square root of the mean):
 *     y[r,i] = x[r,i] * w[i] / sqrt( (1/H) * sum_j x[r,j]^2 + eps )
 * eps sits inside the root (the pages never write the formula; standard form).
 */
void orc_rmsnorm(const void *x, int x_dtype, int64_t x_row_stride,
                 const void *w, int w_dtype, double *y, int64_t rows, int64_t hidden,
                 double eps)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double ss = 0.0;
        for (int64_t j = 0; j < hidden; ++j) {
            double v = load(x, x_dtype, r * x_row_stride + j);
            ss += v * v;
        }
        double denom = sqrt(ss / (double)hidden + eps);
        for (int64_t i = 0; i < hidden; ++i)
            y[r * hidden + i] = load(x, x_dtype, r * x_row_stride + i) * load(w, w_dtype, i) / denom;
    }
}

/*
 * Matmul C = A . W^T with W stored [N, K] (one row per output feature), the
 * contraction over K of [P1] section 5.4 and [P3] "Where the reductions are":
 *     C[m,n] = sum_k A[m,k] * W[n,k]
 * Rows of C are independent of one another ([P1] section 3.3); every output
 * element is its own sequential sum, so the threads share nothing.
 */
void orc_matmul(const void *A, int a_dtype, int64_t lda, const void *W, int w_dtype,
                int64_t ldw, double *C, int64_t ldc, int64_t M, int64_t N, int64_t K)
{
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += load(A, a_dtype, m * lda + k) * load(W, w_dtype, n * ldw + k);
            C[m * ldc + n] = s;
        }
    }
}

/* Logical token j of request r, kv head g, through the block table: the page
 * is table[r][j / page], the slot j % page ([P1] section 5.5: the KV cache and
 * page table are the arrangement attention reduces over).  K pages are stored
 * token-major, [page][kv head][slot][d]; V pages head-dim-major,
 * [page][kv head][d][slot] (the documented cache layouts). */
static const uint16_t *k_row(const uint16_t *cache, const int32_t *table, int64_t bt_stride,
                             int64_t r, int64_t j, int g, int hkv, int page, int d)
{
    int64_t phys = table[r * bt_stride + j / page];
    return cache + ((phys * hkv + g) * (int64_t)page + j % page) * (int64_t)d;
}

static double v_elem(const uint16_t *cache, const int32_t *table, int64_t bt_stride,
                     int64_t r, int64_t j, int g, int hkv, int page, int d, int i)
{
    int64_t phys = table[r * bt_stride + j / page];
    return widen_bf16(cache[((phys * hkv + g) * (int64_t)d + i) * (int64_t)page + j % page]);
}

/*
 * Decode attention for one query token per row, grouped-query heads (query
 * head h reads kv head h / (Hq/Hkv)), over a paged cache of length L_r:
 *     s_j = scale * <q_h, k_j>,  j < L_r
 *     out_h = sum_j softmax(s)_j v_j
 * This is the exact result every split-KV scheme of [P1] section 5.5 and [P3]
 * "The attention detail that gets missed" reaches up to rounding, so the
 * oracle computes it unsplit.  q is [rows, Hq, D] with row stride q_row_stride
 * (elements); out is [rows, Hq, D] fp64.
 */
void orc_decode_attn(const uint16_t *q, int64_t q_row_stride,
                     const uint16_t *k_cache, const uint16_t *v_cache,
                     const int32_t *block_table, int64_t bt_stride, const int32_t *kv_lens,
                     double *out, int64_t rows, int hq, int hkv, int d, int page, double scale)
{
    int group = hq / hkv;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        for (int h = 0; h < hq; ++h) {
            int g = h / group;
            int64_t L = kv_lens[r];
            const uint16_t *qh = q + r * q_row_stride + (int64_t)h * d;
            double *s = (double *)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
            double m = -INFINITY;
            for (int64_t j = 0; j < L; ++j) {
                const uint16_t *kj = k_row(k_cache, block_table, bt_stride, r, j, g, hkv, page, d);
                double dot = 0.0;
                for (int i = 0; i < d; ++i)
                    dot += widen_bf16(qh[i]) * widen_bf16(kj[i]);
                s[j] = scale * dot;
                if (s[j] > m)
                    m = s[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                s[j] = exp(s[j] - m);
                l += s[j];
            }
            double *o = out + (r * hq + h) * (int64_t)d;
            for (int i = 0; i < d; ++i)
                o[i] = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                double p = s[j] / l;
                for (int i = 0; i < d; ++i)
                    o[i] += p * v_elem(v_cache, block_table, bt_stride, r, j, g, hkv, page, d, i);
            }
            free(s);
        }
    }
}

/*
 * Split plan with a fixed split SIZE ([P1] section 5.5, [P3] "The attention
 * detail that gets missed"): split s covers [s*S, min((s+1)*S, L)); only the
 * count ceil(L/S) varies with L, the boundaries never move.  Writes the start
 * of every split and returns the count.
 */
int64_t orc_split_plan(int64_t L, int64_t S, int64_t *starts, int64_t cap)
{
    int64_t n = (L + S - 1) / S;
    for (int64_t s = 0; s < n && s < cap; ++s)
        starts[s] = s * S;
    return n;
}

/*
 * The same decode attention evaluated split by split: for each split a
 * partial state (running max m_s, sum l_s = sum_j exp(s_j - m_s), accumulator
 * acc_s = sum_j exp(s_j - m_s) v_j), then the partials combined with the
 * log-sum-exp rescaling
 *     M = max_s m_s,  l = sum_s e^{m_s - M} l_s,  acc = sum_s e^{m_s - M} acc_s,
 *     out = acc / l.
 * With splits_per_group > 1 the combine has two levels: the splits of each
 * group of that many consecutive splits (absolute: splits k*G .. k*G + G - 1)
 * are combined into a group partial by the same rule, and the group partials
 * are then combined by it.  The pages name split-KV and fixed split size but do
 * not print the combine; this is its standard exact form.  Used only to check,
 * in fp64, that splitting at any fixed size, and grouping the splits, reaches
 * the unsplit result.
 */
static void lse_combine(const double *ms, const double *ls, const double *acc, int64_t n, int d,
                        double *M_out, double *l_out, double *acc_out)
{
    double M = -INFINITY;
    for (int64_t s = 0; s < n; ++s)
        if (ms[s] > M)
            M = ms[s];
    double l = 0.0;
    for (int i = 0; i < d; ++i)
        acc_out[i] = 0.0;
    for (int64_t s = 0; s < n; ++s) {
        double c = exp(ms[s] - M);
        l += c * ls[s];
        for (int i = 0; i < d; ++i)
            acc_out[i] += c * acc[s * d + i];
    }
    *M_out = M;
    *l_out = l;
}

void orc_decode_attn_split_groups(const uint16_t *q, int64_t q_row_stride,
                                  const uint16_t *k_cache, const uint16_t *v_cache,
                                  const int32_t *block_table, int64_t bt_stride,
                                  const int32_t *kv_lens, double *out, int64_t rows, int hq,
                                  int hkv, int d, int page, double scale, int64_t split,
                                  int64_t splits_per_group);

void orc_decode_attn_split(const uint16_t *q, int64_t q_row_stride,
                           const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *block_table, int64_t bt_stride, const int32_t *kv_lens,
                           double *out, int64_t rows, int hq, int hkv, int d, int page,
                           double scale, int64_t split)
{
    orc_decode_attn_split_groups(q, q_row_stride, k_cache, v_cache, block_table, bt_stride,
                                 kv_lens, out, rows, hq, hkv, d, page, scale, split, 1);
}

void orc_decode_attn_split_groups(const uint16_t *q, int64_t q_row_stride,
                                  const uint16_t *k_cache, const uint16_t *v_cache,
                                  const int32_t *block_table, int64_t bt_stride,
                                  const int32_t *kv_lens, double *out, int64_t rows, int hq,
                                  int hkv, int d, int page, double scale, int64_t split,
                                  int64_t splits_per_group)
{
    int group = hq / hkv;
    #pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        for (int h = 0; h < hq; ++h) {
            int g = h / group;
            int64_t L = kv_lens[r];
            int64_t n = (L + split - 1) / split;
            const uint16_t *qh = q + r * q_row_stride + (int64_t)h * d;
            double *ms = (double *)malloc(sizeof(double) * (size_t)n);
            double *ls = (double *)malloc(sizeof(double) * (size_t)n);
            double *acc = (double *)calloc((size_t)(n * d), sizeof(double));
            for (int64_t sidx = 0; sidx < n; ++sidx) {
                int64_t j0 = sidx * split, j1 = j0 + split < L ? j0 + split : L;
                double m = -INFINITY;
                for (int64_t j = j0; j < j1; ++j) {
                    const uint16_t *kj = k_row(k_cache, block_table, bt_stride, r, j, g, hkv, page, d);
                    double dot = 0.0;
                    for (int i = 0; i < d; ++i)
                        dot += widen_bf16(qh[i]) * widen_bf16(kj[i]);
                    if (scale * dot > m)
                        m = scale * dot;
                }
                double l = 0.0;
                for (int64_t j = j0; j < j1; ++j) {
                    const uint16_t *kj = k_row(k_cache, block_table, bt_stride, r, j, g, hkv, page, d);
                    double dot = 0.0;
                    for (int i = 0; i < d; ++i)
                        dot += widen_bf16(qh[i]) * widen_bf16(kj[i]);
                    double p = exp(scale * dot - m);
                    l += p;
                    for (int i = 0; i < d; ++i)
                        acc[sidx * d + i] += p * v_elem(v_cache, block_table, bt_stride, r, j, g,
                                                        hkv, page, d, i);
                }
                ms[sidx] = m;
                ls[sidx] = l;
            }
            /* each group of splits_per_group consecutive splits into one partial,
               then the groups */
            const int64_t G = splits_per_group;
            int64_t ng = (n + G - 1) / G;
            double *gm = (double *)malloc(sizeof(double) * (size_t)ng);
            double *gl = (double *)malloc(sizeof(double) * (size_t)ng);
            double *gacc = (double *)malloc(sizeof(double) * (size_t)(ng * d));
            for (int64_t k = 0; k < ng; ++k) {
                int64_t s0 = k * G, cnt = n - s0 < G ? n - s0 : G;
                lse_combine(ms + s0, ls + s0, acc + s0 * d, cnt, d, &gm[k], &gl[k], gacc + k * d);
            }
            double M, l;
            double *o = out + (r * hq + h) * (int64_t)d;
            lse_combine(gm, gl, gacc, ng, d, &M, &l, o);
            for (int i = 0; i < d; ++i)
                o[i] /= l;
            free(gm);
            free(gl);
            free(gacc);
            free(ms);
            free(ls);
            free(acc);
        }
    }
}

/*
 * Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011), written here from
 * that definition: a 128-bit counter (c0, c1, c2, c3) and a 64-bit key (k0, k1)
 * go through ten rounds; each round multiplies c0 and c2 by the two round
 * multipliers as 32x32 -> 64-bit products, and the new counter is
 *     (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0));
 * between rounds the key advances by the two Weyl constants (golden ratio and
 * sqrt(3) - 1 in 32-bit fixed point).  The result is the final counter.
 */
void orc_philox4x32_10(const uint32_t *ctr, const uint32_t *key, uint32_t *out)
{
    const uint64_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        const uint64_t p0 = M0 * (uint64_t)c[0];
        const uint64_t p1 = M1 * (uint64_t)c[2];
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c[0] = n0;
        c[1] = n1;
        c[2] = n2;
        c[3] = n3;
    }
    memcpy(out, c, sizeof c);
}

/*
 * Gumbel noise of vocabulary entries 0 .. n-1 for one (seed, position) pair
 * (seeded Gumbel-max sampling: [P1] section 9.3 "Non-Greedy Sampling Can Be
 * Deterministic Too" -- noise from a counter-based hash instead of a stateful
 * generator makes a sample a pure function of the logits and the seed).  Entry
 * i takes word
 * i mod 4 of Philox4x32-10 with counter (i / 4, position low 32 bits, position
 * high 32 bits, 0) and key (seed low 32 bits, seed high 32 bits); the word's top
 * 23 bits give u = (floor(w / 2^9) + 1/2) / 2^23 in (0, 1), and the noise is
 * the standard Gumbel quantile g = -ln(-ln u).
 */
static double gumbel_of_word(uint32_t w)
{
    const double u = ((double)(w >> 9) + 0.5) / 8388608.0;
    return -log(-log(u));
}

void orc_gumbel_noise(uint64_t seed, int64_t position, int64_t n, double *g)
{
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int64_t i = 0; i < n; ++i) {
        const uint32_t ctr[4] = {(uint32_t)(i / 4), (uint32_t)(uint64_t)position,
                                 (uint32_t)((uint64_t)position >> 32), 0u};
        uint32_t w[4];
        orc_philox4x32_10(ctr, key, w);
        g[i] = gumbel_of_word(w[i % 4]);
    }
}

/*
 * Seeded Gumbel-max sampling of each row: token = argmax_i (logit_i / T + g_i),
 * g from orc_gumbel_noise(seed_r, position_r); T <= 0 means greedy (argmax of
 * the logits).  NaN logits are never chosen; among equal scores the lowest index
 * wins; a row of NaNs gives token 0.  Also returns the best score and the gap to
 * the runner-up (infinite when there is none), from which a test can tell a
 * clear decision from a near tie.
 */
void orc_sample_gumbel(const float *logits, int64_t ld, int64_t rows, int64_t vocab,
                       const uint64_t *seeds, const int64_t *positions, const float *temps,
                       int32_t *tokens, double *best, double *gap)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const double T = (double)temps[r];
        double *g = (double *)malloc((size_t)(vocab > 0 ? vocab : 1) * sizeof(double));
        if (T > 0.0)
            orc_gumbel_noise(seeds[r], positions[r], vocab, g);
        double b1 = -INFINITY, b2 = -INFINITY;
        int64_t i1 = -1;
        for (int64_t i = 0; i < vocab; ++i) {
            const double x = (double)logits[r * ld + i];
            if (isnan(x))
                continue;
            const double s = T > 0.0 ? x / T + g[i] : x;
            if (i1 < 0 || s > b1) {
                if (i1 >= 0)
                    b2 = b1;
                b1 = s;
                i1 = i;
            } else if (s > b2) {
                b2 = s;
            }
        }
        tokens[r] = i1 < 0 ? 0 : (int32_t)i1;
        best[r] = b1;
        gap[r] = b1 - b2;
        free(g);
    }
}
