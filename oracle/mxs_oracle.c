/*
 * mxs_oracle.c -- plain, slow CPU oracle for the MXSens hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library. The HIP library and its
 * Python binding never call it, and the two share no code, header, table or
 * helper: inputs reach both sides only through the seeded generators.
 *
 * Source of the method: "MXSens: Sensitivity-Aware Mixed-Precision
 * Quantization for Efficient LLM Inference", as summarised on
 *   [NL]  gist.science/nl/paper/2607.17733, "Technische Samenvatting"
 *         (section numbers below refer to it),
 *   [REV] romaanj.github.io/reviews/mxsens ("Method", "Key idea"),
 *   [RP]  researchpod.app summary (bullet "Triplet Quantization"),
 *   [KR]  insight.artgrammer.co.kr/papers/21466 (English abstract).
 * Where the pages leave a step open, the reading taken is stated next to the
 * code as "Reading:". All parity is pinned by the CPU test suite against
 * closed forms, brute force and invariants (see tests/test_oracle_*.py).
 *
 * Conventions
 *   X  [rows, ld] fp32 row-major (bf16 inputs are widened to fp32 exactly by
 *      the caller), K = number of columns, a multiple of 32.
 *   Every sum is taken in fp64; every product that feeds a sum is exact.
 *   Return value 0 = success, -1 = bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_BLOCK 32   /* MXINT block: 32 values share one power-of-two scale
                         ([NL] §1 and §2.2) */

/* ------------------------------------------------------------------------ */
/* 1. MXINT block quantizer                                                  */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §1: MX formats embed one shared power-of-two scale per block of 32
 * values; §2.2: mantissa widths of 4, 6 and 8 bits. The pages do not print
 * the scale rule; Reading (the plain MX rule for an m-bit signed integer
 * element): with E = floor(log2(amax)), the shared scale is 2^s with
 * s = E - (m - 2), so that amax / 2^s lies in [2^(m-2), 2^(m-1)), the top
 * binade of an m-bit two's-complement integer. Each element becomes
 * c = clamp(round_half_even(v / 2^s), -(2^(m-1)-1), 2^(m-1)-1); the value
 * -2^(m-1) is never produced (symmetric range). The scale is stored as an
 * E8M0 byte s + 127, with s clamped to [-127, 127].
 * Reading for degenerate blocks: all-zero block -> byte 0x00 and codes 0;
 * a block holding NaN or +-Inf -> byte 0xFF (the E8M0 NaN code) and codes 0.
 */
static int or_cmax(int m) { return (1 << (m - 1)) - 1; }

int or_quantize_block(const float *v, int n, int m, int8_t *codes, uint8_t *scale_byte)
{
    if (!v || !codes || !scale_byte || n < 1 || n > OR_BLOCK) return -1;
    if (m != 4 && m != 6 && m != 8) return -1;
    for (int i = 0; i < n; ++i) {
        if (!isfinite(v[i])) {
            *scale_byte = 0xFF;
            memset(codes, 0, (size_t)n);
            return 0;
        }
    }
    float amax = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale_byte = 0x00;
        memset(codes, 0, (size_t)n);
        return 0;
    }
    /* floor(log2(amax)) read off the binary exponent: frexpf gives
       amax = f * 2^e with f in [0.5, 1), exact also for subnormals. */
    int e;
    (void)frexpf(amax, &e);
    int E = e - 1;
    int s = E - (m - 2);
    if (s < -127) s = -127;
    if (s > 127) s = 127;
    *scale_byte = (uint8_t)(s + 127);
    const int cmax = or_cmax(m);
    for (int i = 0; i < n; ++i) {
        /* v * 2^-s is exact in fp64 (24-bit significand, exponent in range) */
        double t = ldexp((double)v[i], -s);
        double r = nearbyint(t); /* default rounding mode: to nearest, ties to even */
        if (r > cmax) r = cmax;
        if (r < -cmax) r = -cmax;
        codes[i] = (int8_t)r;
    }
    return 0;
}

/* value represented by code c under E8M0 scale byte b (fp64, exact) */
static double or_dequant(int c, uint8_t b)
{
    if (b == 0xFF) return NAN;
    return ldexp((double)c, (int)b - 127);
}

double or_dequant_value(int code, uint8_t scale_byte) { return or_dequant(code, scale_byte); }

/* ------------------------------------------------------------------------ */
/* 2. Summation order shared by calibrate and score                          */
/* ------------------------------------------------------------------------ */
/*
 * Reading: the pages define the statistic as a plain sum and fix no order.
 * So that the column ranking built on it is reproducible, every column sum
 * here is taken in this order:
 *   rows are cut into chunks of 256 consecutive rows (the last may be short);
 *   inside a chunk, partial sum p_i (i = 0..7) adds the rows whose offset in
 *   the chunk is congruent to i mod 8, in increasing row order, from +0;
 *   the chunk total is ((p0+p1)+(p2+p3)) + ((p4+p5)+(p6+p7));
 *   score: the running total adds chunk totals in chunk order;
 *   calibrate: chunks form runs of 16 consecutive chunks (4096 rows; the
 *   last run of a call may be short); a run total adds its chunk totals in
 *   chunk order, starting from the first, and the running total adds run
 *   totals in run order.
 * All terms are exact squares (of fp32 values or exact fp32 residuals), so
 * only the fp64 additions round.
 */
#define OR_CHUNK 256
#define OR_PARTS 8
#define OR_RUN 16     /* chunks per run of the calibration sum */

static double or_chunk_total(const double p[OR_PARTS])
{
    return ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

/* ------------------------------------------------------------------------ */
/* 3. Calibration: Hessian diagonal                                          */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §2.1 ("Kolomgewijze Sensitiviteit"): sensitivity is built on the
 * diagonal of the empirical Hessian H = X^T X, so Hdiag[k] = sum_t X[t,k]^2
 * over calibration tokens t. Reading: no 1/T normalisation and no damping.
 * hdiag is accumulated in place, so calibration may arrive in several calls;
 * each call cuts its own rows into chunks and runs (section 2) and adds its
 * run totals in order.
 */
int or_calibrate(const float *X, int64_t M, int64_t K, int64_t ldx, double *hdiag)
{
    if (!X || !hdiag || M < 0 || K < 1 || ldx < K) return -1;
    #pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * OR_PARTS * (size_t)K);
        double *run = (double *)malloc(sizeof(double) * (size_t)K);
        #pragma omp for schedule(static)
        for (int64_t kb = 0; kb < K; kb += 64) {
            int64_t ke = kb + 64 < K ? kb + 64 : K;
            for (int64_t r0 = 0; r0 < M; r0 += OR_CHUNK) {
                int64_t r1 = r0 + OR_CHUNK < M ? r0 + OR_CHUNK : M;
                int64_t c = r0 / OR_CHUNK;             /* chunk index within the call */
                for (int64_t k = kb; k < ke; ++k)
                    for (int i = 0; i < OR_PARTS; ++i) p[i * K + k] = 0.0;
                for (int64_t t = r0; t < r1; ++t) {
                    int i = (int)((t - r0) % OR_PARTS);
                    for (int64_t k = kb; k < ke; ++k) {
                        double x = (double)X[t * ldx + k];
                        p[i * K + k] += x * x;
                    }
                }
                for (int64_t k = kb; k < ke; ++k) {
                    double q[OR_PARTS];
                    for (int i = 0; i < OR_PARTS; ++i) q[i] = p[i * K + k];
                    double tot = or_chunk_total(q);
                    run[k] = c % OR_RUN == 0 ? tot : run[k] + tot;   /* run total */
                    if (c % OR_RUN == OR_RUN - 1 || r1 == M) hdiag[k] += run[k];
                }
            }
        }
        free(run);
        free(p);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 4. Column sensitivity score                                               */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §2.1: columns with large Hessian-diagonal entries are the ones where
 * quantisation noise costs most output error. The pages only say that the score
 * is built on the diagonal; Reading: score_k = Hdiag_k * E_k with
 * E_k = sum_n (W[n,k] - Q4(W)[n,k])^2, where Q4(W) is W quantised to uniform
 * 4-bit MXINT in 32-blocks along K in the original column order (the
 * quantiser that is actually deployed for a 4-bit column). sum_k score_k is
 * then the diagonal-Hessian estimate of the output error of uniform MXINT4.
 * E_k is summed in the order of section 2; the product is rounded once.
 */
int or_score(const float *W, int64_t N, int64_t K, int64_t ldw,
             const double *hdiag, double *score)
{
    if (!W || !hdiag || !score || N < 1 || K < OR_BLOCK || K % OR_BLOCK || ldw < K) return -1;
    double *E = (double *)calloc((size_t)K, sizeof(double));
    double *res = (double *)malloc(sizeof(double) * OR_CHUNK * (size_t)K);
    if (!E || !res) { free(E); free(res); return -1; }
    for (int64_t r0 = 0; r0 < N; r0 += OR_CHUNK) {
        int64_t r1 = r0 + OR_CHUNK < N ? r0 + OR_CHUNK : N;
        /* residual of every row of the chunk under uniform MXINT4 */
        #pragma omp parallel for schedule(static)
        for (int64_t t = r0; t < r1; ++t) {
            for (int64_t b = 0; b < K / OR_BLOCK; ++b) {
                const float *v = W + t * ldw + b * OR_BLOCK;
                int8_t c[OR_BLOCK];
                uint8_t sb;
                or_quantize_block(v, OR_BLOCK, 4, c, &sb);
                for (int j = 0; j < OR_BLOCK; ++j)
                    res[(t - r0) * K + b * OR_BLOCK + j] = (double)v[j] - or_dequant(c[j], sb);
            }
        }
        #pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < K; ++k) {
            double q[OR_PARTS] = {0, 0, 0, 0, 0, 0, 0, 0};
            for (int64_t t = r0; t < r1; ++t) {
                double d = res[(t - r0) * K + k];
                q[(t - r0) % OR_PARTS] += d * d;
            }
            E[k] += or_chunk_total(q);
        }
    }
    for (int64_t k = 0; k < K; ++k) score[k] = hdiag[k] * E[k];
    free(E); free(res);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 5. Budget -> block counts                                                 */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §2.3: widths are assigned under a target average bitwidth B; the top
 * 32 columns of every layer always get 8 bits (§2.2: one MXINT block, so the
 * extreme outliers share one high-precision block); 6-bit columns are
 * budgeted; the rest get 4 bits. The per-layer budget arrives as fractions
 * f8, f6 in basis points (bp8, bp6). Reading: counts are whole 32-column
 * blocks and the layer's average may not exceed B = 8 f8 + 6 f6 + 4 f4:
 *   nb = K/32
 *   U  = floor(nb * (2 bp8 + bp6) / 10000)   budget above 4 bits, in units of
 *                                            "+2 bits on one block"
 *   n8 = bp8 > 0 ? max(1, floor(nb bp8 / 10000)) : 0, then n8 <= floor(U/2)
 *   n6 = min(U - 2 n8, nb - n8);   n4 = nb - n8 - n6.
 */
int or_budget_blocks(int64_t K, int32_t bp8, int32_t bp6, int32_t nblk[3])
{
    if (!nblk || K < OR_BLOCK || K % OR_BLOCK) return -1;
    if (bp8 < 0 || bp6 < 0 || (int64_t)bp8 + bp6 > 10000) return -1;
    int64_t nb = K / OR_BLOCK;
    int64_t U = nb * (2 * (int64_t)bp8 + bp6) / 10000;
    int64_t n8 = 0;
    if (bp8 > 0) {
        n8 = nb * bp8 / 10000;
        if (n8 < 1) n8 = 1;
    }
    if (n8 > U / 2) n8 = U / 2;
    int64_t n6 = U - 2 * n8;
    if (n6 > nb - n8) n6 = nb - n8;
    nblk[0] = (int32_t)n8;
    nblk[1] = (int32_t)n6;
    nblk[2] = (int32_t)(nb - n8 - n6);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 6. Allocation: ranking, bit map, block-uniform permutation                */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §2.3: sort the columns of the layer by score; the first 32 n8 get 8
 * bits, the next 32 n6 get 6 bits, the rest 4 bits. [NL] §2.3 (last line)
 * and [REV] "Key idea": the allocation uses MXINT's block structure, so every
 * 32-column block must hold one width. Reading: columns are gathered by a
 * permutation (perm[j] = source column of position j) that lists the 8-bit
 * columns in ascending index, then the 6-bit ones, then the 4-bit ones; an
 * all-4-bit map therefore gives the identity and uniform MXINT4.
 * Reading for ties and odd values: the order is "score descending, then
 * index ascending", with scores compared as a total order on the fp64 bit
 * pattern (NaN above +Inf above every finite value).
 */
static uint64_t or_order_key(double s)
{
    uint64_t u;
    memcpy(&u, &s, sizeof u);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

static const double *or_sort_scores;
static int or_rank_cmp(const void *a, const void *b)
{
    int32_t i = *(const int32_t *)a, j = *(const int32_t *)b;
    uint64_t ki = or_order_key(or_sort_scores[i]), kj = or_order_key(or_sort_scores[j]);
    if (ki != kj) return ki > kj ? -1 : 1; /* larger score first */
    return i < j ? -1 : (i > j);           /* then smaller index */
}

/* the same with the block counts given (n8 blocks of 8 bits, n6 of 6) */
int or_allocate_blocks(const double *score, int64_t K, int32_t n8, int32_t n6,
                       uint8_t *bits, int32_t *perm)
{
    if (!score || !bits || !perm || K < OR_BLOCK || K % OR_BLOCK) return -1;
    if (n8 < 0 || n6 < 0 || (int64_t)n8 + n6 > K / OR_BLOCK) return -1;
    const int32_t nb3[2] = {n8, n6};
    int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    if (!order) return -1;
    for (int64_t k = 0; k < K; ++k) order[k] = (int32_t)k;
    or_sort_scores = score;
    qsort(order, (size_t)K, sizeof(int32_t), or_rank_cmp);
    const int64_t c8 = (int64_t)OR_BLOCK * nb3[0], c6 = (int64_t)OR_BLOCK * nb3[1];
    for (int64_t r = 0; r < K; ++r)
        bits[order[r]] = (uint8_t)(r < c8 ? 8 : (r < c8 + c6 ? 6 : 4));
    int64_t j = 0;
    static const uint8_t cls[3] = {8, 6, 4};
    for (int c = 0; c < 3; ++c)
        for (int64_t k = 0; k < K; ++k)
            if (bits[k] == cls[c]) perm[j++] = (int32_t)k;
    free(order);
    return 0;
}

int or_allocate(const double *score, int64_t K, int32_t bp8, int32_t bp6,
                uint8_t *bits, int32_t *perm)
{
    int32_t nb3[3];
    if (or_budget_blocks(K, bp8, bp6, nb3)) return -1;
    return or_allocate_blocks(score, K, nb3[0], nb3[1], bits, perm);
}

/* ------------------------------------------------------------------------ */
/* 7. Quantize a matrix with a permutation and pack into planes              */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §2.2-§2.3 with the permutation of section 6. Row r, permuted block b
 * (b < n8: 8 bits, b < n8+n6: 6 bits, else 4 bits) takes
 * v = X[r, perm[32 b .. 32 b + 31]] and quantises it with the block quantiser.
 * The same map serves weights and activations (Reading: one map per linear
 * layer, because the product pairs input channel k of X with column k of W;
 * [RP] bullet "weights and activations"); activation scales are computed per
 * row and block from the values at hand (MX semantics, [NL] §1).
 * Reading for storage (the pages give none):
 *   q8[r, 32 i + j]      = c_j of the i-th 8-bit block (int8)
 *   q6[r, 24 i + 3 g ..] = 24-bit little-endian word c0 | c1<<6 | c2<<12 |
 *                          c3<<18 of codes 4g..4g+3, 6-bit two's complement
 *   q4[r, 16 i + h]      = (c_{2h} & 15) | (c_{2h+1} & 15) << 4
 *   sc[r, b]             = E8M0 byte of permuted block b.
 */
int or_quantize(const float *X, int64_t R, int64_t K, int64_t ldx, const int32_t *perm,
                int32_t n8, int32_t n6, int32_t n4,
                int8_t *q8, int64_t ld8, uint8_t *q6, int64_t ld6,
                uint8_t *q4, int64_t ld4, uint8_t *sc, int64_t lds)
{
    if (!X || !sc || R < 0 || K < OR_BLOCK || K % OR_BLOCK || ldx < K) return -1;
    int64_t nb = K / OR_BLOCK;
    if (n8 < 0 || n6 < 0 || n4 < 0 || (int64_t)n8 + n6 + n4 != nb) return -1;
    if ((n8 && (!q8 || ld8 < 32 * (int64_t)n8)) || (n6 && (!q6 || ld6 < 24 * (int64_t)n6)) ||
        (n4 && (!q4 || ld4 < 16 * (int64_t)n4)) || lds < nb) return -1;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            float v[OR_BLOCK];
            for (int j = 0; j < OR_BLOCK; ++j) {
                int64_t src = perm ? perm[b * OR_BLOCK + j] : b * OR_BLOCK + j;
                v[j] = X[r * ldx + src];
            }
            int m = b < n8 ? 8 : (b < (int64_t)n8 + n6 ? 6 : 4);
            int8_t c[OR_BLOCK];
            uint8_t s;
            or_quantize_block(v, OR_BLOCK, m, c, &s);
            sc[r * lds + b] = s;
            if (m == 8) {
                int8_t *dst = q8 + r * ld8 + 32 * b;
                for (int j = 0; j < OR_BLOCK; ++j) dst[j] = c[j];
            } else if (m == 6) {
                uint8_t *dst = q6 + r * ld6 + 24 * (b - n8);
                for (int g = 0; g < 8; ++g) {
                    uint32_t w = 0;
                    for (int i = 0; i < 4; ++i) w |= ((uint32_t)c[4 * g + i] & 63u) << (6 * i);
                    dst[3 * g + 0] = (uint8_t)(w & 255u);
                    dst[3 * g + 1] = (uint8_t)((w >> 8) & 255u);
                    dst[3 * g + 2] = (uint8_t)((w >> 16) & 255u);
                }
            } else {
                uint8_t *dst = q4 + r * ld4 + 16 * (b - n8 - n6);
                for (int h = 0; h < 16; ++h)
                    dst[h] = (uint8_t)(((uint32_t)c[2 * h] & 15u) | (((uint32_t)c[2 * h + 1] & 15u) << 4));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 8. Unpack planes back to codes (used by the GEMM definition below)        */
/* ------------------------------------------------------------------------ */
static int or_sext(uint32_t x, int bits)
{
    uint32_t sign = 1u << (bits - 1);
    return (int)((x ^ sign)) - (int)sign;
}

/* codes[K] of row r, in permuted order */
int or_unpack_row(int64_t r, int64_t K, int32_t n8, int32_t n6, int32_t n4,
                  const int8_t *q8, int64_t ld8, const uint8_t *q6, int64_t ld6,
                  const uint8_t *q4, int64_t ld4, int32_t *codes)
{
    if (K % OR_BLOCK || (int64_t)n8 + n6 + n4 != K / OR_BLOCK || !codes) return -1;
    for (int64_t b = 0; b < K / OR_BLOCK; ++b) {
        int32_t *dst = codes + b * OR_BLOCK;
        if (b < n8) {
            for (int j = 0; j < OR_BLOCK; ++j) dst[j] = q8[r * ld8 + 32 * b + j];
        } else if (b < (int64_t)n8 + n6) {
            const uint8_t *src = q6 + r * ld6 + 24 * (b - n8);
            for (int g = 0; g < 8; ++g) {
                uint32_t w = (uint32_t)src[3 * g] | ((uint32_t)src[3 * g + 1] << 8) |
                             ((uint32_t)src[3 * g + 2] << 16);
                for (int i = 0; i < 4; ++i) dst[4 * g + i] = or_sext((w >> (6 * i)) & 63u, 6);
            }
        } else {
            const uint8_t *src = q4 + r * ld4 + 16 * (b - n8 - n6);
            for (int h = 0; h < 16; ++h) {
                dst[2 * h] = or_sext(src[h] & 15u, 4);
                dst[2 * h + 1] = or_sext((uint32_t)src[h] >> 4, 4);
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 9. Block-scaled mixed GEMM: Y = Qa(X) Qw(W)^T                              */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §1 and §5, [REV] "Comparison": the scales live in the MX format and
 * the product consumes codes and scales directly, with no separate
 * dequantisation pass. Plain definition (exact up to fp64 summation):
 *   Y[t,n] = sum_k deq(A)[t,k] * deq(W)[n,k],  deq = code * 2^(byte - 127),
 * over the permuted K axis (A and W share the permutation, so the sum equals
 * the one over the original channels). Every product is exact in fp64; the
 * sum runs over k in increasing order. Yabs[t,n] = sum_k |deq(A)||deq(W)| is
 * returned for the componentwise acceptance bound (may be NULL).
 */
typedef struct {
    int64_t rows, K;
    int32_t n8, n6, n4;
    const int8_t *q8; int64_t ld8;
    const uint8_t *q6; int64_t ld6;
    const uint8_t *q4; int64_t ld4;
    const uint8_t *sc; int64_t lds;
} or_qmat;

static int or_dequant_matrix(const or_qmat *A, double *out /* [rows, K] */)
{
    int32_t *codes = (int32_t *)malloc(sizeof(int32_t) * (size_t)A->K);
    if (!codes) return -1;
    for (int64_t r = 0; r < A->rows; ++r) {
        if (or_unpack_row(r, A->K, A->n8, A->n6, A->n4, A->q8, A->ld8, A->q6, A->ld6,
                          A->q4, A->ld4, codes)) { free(codes); return -1; }
        for (int64_t k = 0; k < A->K; ++k)
            out[r * A->K + k] = or_dequant(codes[k], A->sc[r * A->lds + k / OR_BLOCK]);
    }
    free(codes);
    return 0;
}

int or_mixed_gemm(int64_t M, int64_t N, int64_t K, int32_t n8, int32_t n6, int32_t n4,
                  const int8_t *a8, int64_t la8, const uint8_t *a6, int64_t la6,
                  const uint8_t *a4, int64_t la4, const uint8_t *asc, int64_t las,
                  const int8_t *w8, int64_t lw8, const uint8_t *w6, int64_t lw6,
                  const uint8_t *w4, int64_t lw4, const uint8_t *wsc, int64_t lws,
                  double *Y, int64_t ldy, double *Yabs)
{
    if (M < 0 || N < 0 || K < OR_BLOCK || K % OR_BLOCK || !Y || ldy < N) return -1;
    if ((int64_t)n8 + n6 + n4 != K / OR_BLOCK || n8 < 0 || n6 < 0 || n4 < 0) return -1;
    or_qmat A = {M, K, n8, n6, n4, a8, la8, a6, la6, a4, la4, asc, las};
    or_qmat B = {N, K, n8, n6, n4, w8, lw8, w6, lw6, w4, lw4, wsc, lws};
    double *da = (double *)malloc(sizeof(double) * (size_t)(M * K + 1));
    double *dw = (double *)malloc(sizeof(double) * (size_t)(N * K + 1));
    if (!da || !dw || or_dequant_matrix(&A, da) || or_dequant_matrix(&B, dw)) {
        free(da); free(dw); return -1;
    }
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aab = 0.0;
            const double *x = da + t * K, *w = dw + n * K;
            for (int64_t k = 0; k < K; ++k) {
                acc += x[k] * w[k];
                aab += fabs(x[k]) * fabs(w[k]);
            }
            Y[t * ldy + n] = acc;
            if (Yabs) Yabs[t * ldy + n] = aab;
        }
    }
    free(da); free(dw);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 10. KV-cache quantisation                                                 */
/* ------------------------------------------------------------------------ */
/*
 * W4A4KV4 ([NL] §4, [REV] "Validation"): keys and values are stored as
 * 4-bit MXINT. Reading: uniform 4-bit, blocks of 32 consecutive elements
 * along head_dim, no permutation; codes [T, H, D/2] packed like the 4-bit
 * plane above, scales [T, H, D/32].
 */
int or_quantize_kv(const float *kv, int64_t T, int64_t H, int64_t D,
                   uint8_t *codes, uint8_t *scales)
{
    if (!kv || !codes || !scales || T < 0 || H < 1 || D < OR_BLOCK || D % OR_BLOCK) return -1;
    return or_quantize(kv, T * H, D, D, NULL, 0, 0, (int32_t)(D / OR_BLOCK), NULL, 0, NULL, 0,
                       codes, D / 2, scales, D / OR_BLOCK);
}

/* ------------------------------------------------------------------------ */
/* 11. Layer-wise allocation under a global control parameter R              */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §2.1 ("Laaggewijze sensitiviteit"): a layer's sensitivity is the L2
 * error at the model output when that layer alone is quantized. [NL] §2.3:
 * widths are assigned under a target average bitwidth B with one global
 * parameter R; every layer keeps its 32 most sensitive columns at 8 bits,
 * and its number of 6-bit columns is proportional to its sensitivity,
 * scaled by R so that the global average meets B.
 *
 * Reading (the model output needs a trained model, which is not built):
 *   S_l = || X W^T - Q4(X) Q4(W)^T ||_F^2 over calibration tokens X, with Q4
 *         uniform MXINT4 on both operands (the layer quantized on its own);
 *   n8_l = 1,  n6_l = min(nb_l - 1, floor(R S_l + 1/2))  (whole blocks),
 *   R = the largest value whose average over all weights (each layer
 *       weighted by rows_l * K_l, mantissa bits only) does not exceed B.
 * The average is a step function of R that jumps where R S_l = j - 1/2; R
 * is found by bisection over those breakpoints: in ascending order (ties
 * taken together), a breakpoint is accepted while the extra bits it adds
 * still fit; the first that does not fit ends the search. The budget in
 * extra bits above 4 is floor((B - 4) * sum_l rows_l K_l).
 */

/* sum_{t,n} (sum_k X[t,k] W[n,k] - Yq[t,n])^2: fp64, t then n ascending */
int or_output_error(const float *X, int64_t M, int64_t K, int64_t ldx,
                    const float *W, int64_t N, int64_t ldw,
                    const double *Yq, int64_t ldy, double *err)
{
    if (!X || !W || !Yq || !err || M < 0 || N < 0 || K < 1 || ldx < K || ldw < K || ldy < N) return -1;
    double *row = (double *)malloc(sizeof(double) * (size_t)(N + 1));
    if (!row) return -1;
    double total = 0.0;
    for (int64_t t = 0; t < M; ++t) {
        #pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += (double)X[t * ldx + k] * (double)W[n * ldw + k];
            row[n] = acc;
        }
        for (int64_t n = 0; n < N; ++n) {
            const double d = row[n] - Yq[t * ldy + n];
            total += d * d;
        }
    }
    free(row);
    *err = total;
    return 0;
}

typedef struct {
    double key;     /* (j - 1/2) / S_l */
    int32_t layer;
    int32_t j;
} or_bp;

static int or_bp_cmp(const void *a, const void *b)
{
    const or_bp *x = (const or_bp *)a, *y = (const or_bp *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->layer != y->layer) return x->layer < y->layer ? -1 : 1;
    return x->j < y->j ? -1 : (x->j > y->j);
}

int or_layer_budget(int32_t L, const double *S, const int64_t *rows, const int64_t *K, double B,
                    int32_t *nblk /* [L][3] */, double *R_out)
{
    if (L < 1 || !S || !rows || !K || !nblk || !(B >= 4.0) || !(B <= 8.0)) return -1;
    double total = 0.0, need8 = 0.0;
    int64_t nbp = 0;
    for (int32_t l = 0; l < L; ++l) {
        if (rows[l] < 1 || K[l] < OR_BLOCK || K[l] % OR_BLOCK || !(S[l] >= 0.0) || isinf(S[l])) return -1;
        total += (double)rows[l] * (double)K[l];
        need8 += 4.0 * OR_BLOCK * (double)rows[l];      /* one 8-bit block: +4 bits on 32 columns */
        if (S[l] > 0.0) nbp += K[l] / OR_BLOCK - 1;
    }
    const double allowed = floor((B - 4.0) * total);
    if (need8 > allowed) return -1;
    or_bp *bp = (or_bp *)malloc(sizeof(or_bp) * (size_t)(nbp + 1));
    if (!bp) return -1;
    int64_t c = 0;
    for (int32_t l = 0; l < L; ++l) {
        nblk[3 * l] = 1;
        nblk[3 * l + 1] = 0;
        if (S[l] > 0.0)
            for (int32_t j = 1; j < K[l] / OR_BLOCK; ++j) {
                bp[c].key = ((double)j - 0.5) / S[l];
                bp[c].layer = l;
                bp[c].j = j;
                ++c;
            }
    }
    qsort(bp, (size_t)nbp, sizeof(or_bp), or_bp_cmp);
    double used = need8, R = 0.0;
    for (int64_t i = 0; i < nbp;) {
        int64_t e = i;
        double add = 0.0;
        while (e < nbp && bp[e].key == bp[i].key) {       /* a group of equal breakpoints */
            add += 2.0 * OR_BLOCK * (double)rows[bp[e].layer];   /* 6-bit block: +2 bits on 32 columns */
            ++e;
        }
        if (used + add > allowed) break;
        used += add;
        R = bp[i].key;
        for (int64_t q = i; q < e; ++q) nblk[3 * bp[q].layer + 1] = bp[q].j;
        i = e;
    }
    for (int32_t l = 0; l < L; ++l) nblk[3 * l + 2] = (int32_t)(K[l] / OR_BLOCK) - 1 - nblk[3 * l + 1];
    if (R_out) *R_out = R;
    free(bp);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* 12. Attention over the 4-bit K/V cache (one query token)                  */
/* ------------------------------------------------------------------------ */
/*
 * [NL] §4 (W4A4KV4) and [KR] abstract: keys and values are kept as 4-bit
 * MXINT (section 10). Reading: they are consumed by plain scaled dot-product
 * attention of one query token per head, heads grouped onto the KV heads
 * (query head h reads KV head h / (Hq / Hkv)); K and V enter dequantized
 * exactly (code * 2^(byte - 127), a 0x00 byte gives 0, a 0xFF byte NaN):
 *   s_t   = scale * sum_d q[h,d] K[t,g,d]
 *   p_t   = exp(s_t - max_t s) / sum_t exp(s_t - max_t s)
 *   o[h,d] = sum_t p_t V[t,g,d]
 * in fp64, t ascending.
 */
static double or_kv_value(const uint8_t *codes, const uint8_t *scales, int64_t t, int64_t g, int64_t Hkv,
                          int64_t D, int64_t d)
{
    const uint8_t byte = codes[(t * Hkv + g) * (D / 2) + d / 2];
    const int c = or_sext((d & 1) ? (uint32_t)(byte >> 4) : (uint32_t)(byte & 15u), 4);
    return or_dequant(c, scales[(t * Hkv + g) * (D / OR_BLOCK) + d / OR_BLOCK]);
}

int or_attend_kv4(const float *q, const uint8_t *kc, const uint8_t *ks, const uint8_t *vc, const uint8_t *vs,
                  int64_t T, int64_t Hq, int64_t Hkv, int64_t D, double scale, double *out)
{
    if (!q || !kc || !ks || !vc || !vs || !out || T < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv ||
        D < OR_BLOCK || D % OR_BLOCK) return -1;
    double *s = (double *)malloc(sizeof(double) * (size_t)T);
    if (!s) return -1;
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t g = h / (Hq / Hkv);
        double m = -INFINITY;
        for (int64_t t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int64_t d = 0; d < D; ++d) acc += (double)q[h * D + d] * or_kv_value(kc, ks, t, g, Hkv, D, d);
            s[t] = scale * acc;
            if (s[t] > m) m = s[t];
        }
        double l = 0.0;
        for (int64_t t = 0; t < T; ++t) { s[t] = exp(s[t] - m); l += s[t]; }
        for (int64_t d = 0; d < D; ++d) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; ++t) acc += s[t] * or_kv_value(vc, vs, t, g, Hkv, D, d);
            out[h * D + d] = acc / l;
        }
    }
    free(s);
    return 0;
}
