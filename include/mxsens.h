/*
 * mxsens.h -- C ABI of libmxsens, the MI355X (gfx950) hot path of MXSens.
 *
 * MXSens ("MXSens: Sensitivity-Aware Mixed-Precision Quantization for
 * Efficient LLM Inference") gives every input channel of a linear layer a
 * 4-, 6- or 8-bit MXINT mantissa, chosen from a Hessian-diagonal
 * sensitivity score, and keeps every 32-value MXINT block at one width.
 * Page citations below:
 *   [NL]  gist.science/nl/paper/2607.17733, "Technische Samenvatting", §n
 *   [REV] romaanj.github.io/reviews/mxsens, named paragraph
 *   [RP]  researchpod.app summary, named bullet
 *
 * Common rules
 *   - Device pointers: every array argument is device memory, except the
 *     host-side `nblk` of mxs_budget_blocks and the mxs_qmat structs, which
 *     are read on the host during the call.
 *   - Ownership: the caller owns every buffer. The library allocates no
 *     memory; workspaces are passed in after a size query.
 *   - Streams: every call enqueues its kernels on `stream` (0 = the null
 *     stream) and returns without synchronising. Outputs are ready when the
 *     stream reaches that point.
 *   - Errors: argument errors are detected before anything is enqueued; a
 *     failed launch returns MXS_ERR_DEVICE. On error, outputs are undefined
 *     and mxs_last_error() (thread-local) describes the cause. No C++
 *     exception crosses this boundary.
 *   - Layout: matrices are row-major with a leading dimension (elements per
 *     row, >= the row width). X is [tokens, K] (activations), W is [N, K]
 *     (out x in), column k is input channel k. K is a multiple of 32.
 *   - Element types: MXS_F32 (fp32) or MXS_BF16 (bfloat16) inputs; bf16
 *     values are widened to fp32 exactly. Sums are fp64 where stated.
 *   - Thread safety: reentrant; the library holds no mutable global state
 *     other than the thread-local error string and, for
 *     mxs_mixed_gemm_noalloc, one device scratch array per GPU (see there).
 */
#ifndef MXSENS_H
#define MXSENS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mxs_status;
#define MXS_OK               0
#define MXS_ERR_ARG         -1  /* null pointer, unknown enum value            */
#define MXS_ERR_SHAPE       -2  /* K % 32 != 0, negative size, ld < width, ... */
#define MXS_ERR_BUDGET      -3  /* bp8 < 0, bp6 < 0 or bp8 + bp6 > 10000       */
#define MXS_ERR_WORKSPACE   -4  /* workspace missing or smaller than required  */
#define MXS_ERR_DEVICE      -5  /* HIP launch or runtime error                 */
#define MXS_ERR_UNSUPPORTED -6  /* valid but unsupported (alignment, size cap) */

typedef enum { MXS_F32 = 0, MXS_BF16 = 1 } mxs_dtype;

/*
 * A matrix quantised with one bit map: `rows` rows of K permuted channels,
 * made of n8 8-bit blocks, then n6 6-bit blocks, then n4 4-bit blocks
 * (n8 + n6 + n4 = K/32). Storage (all device memory, row-major):
 *   q8 [rows, ld8 >= 32 n8]  int8 codes, byte j of 8-bit block i at 32 i + j
 *   q6 [rows, ld6 >= 24 n6]  6-bit codes: block i at 24 i; codes 4g..4g+3
 *                            form the little-endian 24-bit word
 *                            c0 | c1<<6 | c2<<12 | c3<<18 at byte 24 i + 3 g
 *   q4 [rows, ld4 >= 16 n4]  4-bit codes: block i at 16 i; byte h holds
 *                            c_2h in bits 0-3 and c_2h+1 in bits 4-7
 *   sc [rows, lds >= K/32]   E8M0 scale byte s + 127 of permuted block b
 * Codes are two's complement in [-(2^(m-1)-1), 2^(m-1)-1]; the value of a
 * code c in a block with scale byte e is c * 2^(e-127); e = 0xFF marks a
 * block that held NaN or Inf (its value is NaN).
 * Pointers of empty planes (count 0) may be NULL.
 */
typedef struct mxs_qmat {
    int64_t rows;
    int64_t K;
    int32_t n8, n6, n4;
    int32_t reserved;   /* must be 0 */
    int8_t  *q8; int64_t ld8;
    uint8_t *q6; int64_t ld6;
    uint8_t *q4; int64_t ld4;
    uint8_t *sc; int64_t lds;
} mxs_qmat;

/* Text for a status code (static storage). */
const char *mxs_status_string(mxs_status status);

/* Description of the last error on the calling thread ("" if none). */
const char *mxs_last_error(void);

/* Library ABI version: 1. */
int32_t mxs_version(void);

/*
 * Budget -> whole-block counts for one layer of K channels ([NL] §2.2-§2.3:
 * the 32 most sensitive columns of each layer take 8 bits, a budgeted number
 * of columns take 6 bits, the rest 4 bits, under a target average width B).
 * bp8 and bp6 are the 8- and 6-bit column shares in basis points. Reading:
 *   nb = K/32; U = floor(nb (2 bp8 + bp6) / 10000);
 *   n8 = bp8 > 0 ? max(1, floor(nb bp8 / 10000)) : 0, capped at floor(U/2);
 *   n6 = min(U - 2 n8, nb - n8); n4 = nb - n8 - n6,
 * so the layer average never exceeds B = 8 f8 + 6 f6 + 4 f4.
 * Host-only and pure: nblk is host memory {n8, n6, n4}.
 * Errors: MXS_ERR_ARG (nblk NULL), MXS_ERR_SHAPE (K <= 0 or K % 32),
 * MXS_ERR_BUDGET.
 */
mxs_status mxs_budget_blocks(int64_t K, int32_t bp8, int32_t bp6, int32_t nblk[3]);

/* Workspace bytes needed by mxs_calibrate / mxs_score for these sizes. */
size_t mxs_calibrate_workspace(int64_t M, int64_t K);
size_t mxs_score_workspace(int64_t N, int64_t K);

/*
 * Calibration ([NL] §2.1, column-wise sensitivity): accumulate the diagonal
 * of the empirical Hessian H = X^T X,
 *     hdiag[k] += sum_t X[t, k]^2,   t < M,
 * with no normalisation or damping. X: [M, ldx] device array of `dtype`;
 * hdiag: [K] fp64 device array, read and written (zero it before the first
 * call; later calls add more calibration tokens). Summation order (so that
 * rankings built on it are reproducible bit for bit): rows in chunks of 256;
 * inside a chunk eight partial sums over rows congruent mod 8, combined as
 * ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)); chunks in runs of 16 (4096 rows, the
 * last run of a call may be short), a run total adding its chunk totals in
 * chunk order from the first; run totals added to hdiag in run order.
 * Squares are exact in fp64. ws: >= mxs_calibrate_workspace(M, K) bytes of
 * device memory, 256-byte aligned, contents scratch. M = 0 is a no-op.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE (K <= 0, K % 32, ldx < K, M < 0),
 * MXS_ERR_WORKSPACE, MXS_ERR_DEVICE.
 */
mxs_status mxs_calibrate(const void *X, mxs_dtype dtype, int64_t M, int64_t K, int64_t ldx,
                         double *hdiag, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Column sensitivity ([NL] §2.1: columns with large Hessian-diagonal entries
 * turn quantisation noise into the largest output error). Reading for the
 * score, which the pages leave open:
 *     score[k] = hdiag[k] * sum_n (W[n, k] - Q4(W)[n, k])^2
 * where Q4 is uniform 4-bit MXINT in 32-blocks along K in the original
 * channel order. The residual is exact in fp32, its square exact in fp64,
 * the sum over n is taken in chunks as in mxs_calibrate, with the chunk
 * totals added in chunk order (no runs), from 0; the product is rounded
 * once. W: [N, ldw] of `dtype`; hdiag, score: [K] fp64 device arrays.
 * ws: >= mxs_score_workspace(N, K) bytes. A block holding NaN/Inf yields NaN
 * for its 32 columns.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE (N <= 0, K % 32, ldw < K),
 * MXS_ERR_WORKSPACE, MXS_ERR_DEVICE.
 */
mxs_status mxs_score(const void *W, mxs_dtype dtype, int64_t N, int64_t K, int64_t ldw,
                     const double *hdiag, double *score, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Allocation ([NL] §2.3): rank the K columns by score (descending; ties by
 * ascending index; scores compared as a total order on the fp64 bit pattern,
 * NaN above +Inf above all finite values), give the first 32 n8 columns 8
 * bits, the next 32 n6 6 bits and the rest 4 bits, with (n8, n6, n4) from
 * mxs_budget_blocks. Block-uniform permutation ([NL] §2.3 last paragraph,
 * [REV] "Key idea": the allocation rides on MXINT's block structure): perm
 * lists the 8-bit columns in ascending index, then the 6-bit, then the
 * 4-bit ones, so every 32-block of the permuted order has one width and an
 * all-4 map gives the identity.
 * score: [K] fp64 device; bits: [K] uint8 device out (values 8, 6, 4);
 * perm: [K] int32 device out, gather form (perm[j] = source column of
 * position j). K <= 131072.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE, MXS_ERR_BUDGET, MXS_ERR_UNSUPPORTED
 * (K too large), MXS_ERR_DEVICE.
 */
mxs_status mxs_allocate(const double *score, int64_t K, int32_t bp8, int32_t bp6,
                        uint8_t *bits, int32_t *perm, hipStream_t stream);

/*
 * mxs_allocate with the block counts given instead of the budget: the first
 * 32 n8 ranked columns get 8 bits, the next 32 n6 6 bits, the rest 4 bits
 * (for a layer-wise budget from mxs_layer_budget). Same ranking, bit map,
 * permutation, layout and stream semantics as mxs_allocate.
 * Errors: MXS_ERR_ARG (NULL), MXS_ERR_SHAPE (K % 32), MXS_ERR_BUDGET
 * (n8, n6 < 0 or n8 + n6 > K/32), MXS_ERR_UNSUPPORTED (K > 131072),
 * MXS_ERR_DEVICE.
 */
mxs_status mxs_allocate_blocks(const double *score, int64_t K, int32_t n8, int32_t n6,
                               uint8_t *bits, int32_t *perm, hipStream_t stream);

/*
 * Layer sensitivity ([NL] §2.1, layer-wise sensitivity: the output error
 * when one layer alone is quantized). Reading: without a trained model the
 * model-output error is replaced by the layer's own output error on
 * calibration tokens,
 *     err = sum_{t,n} (sum_k X[t,k] W[n,k] - Yq[t,n])^2,
 * where Yq is the product of the quantized operands from mxs_mixed_gemm
 * (uniform MXINT4 on both for the layer sensitivity S of mxs_layer_budget).
 * The product is formed on the fp32 matrix cores (bf16 inputs widen
 * exactly; each element carries at most the rounding of a K-term fp32 sum),
 * the squared differences are summed in fp64 in a fixed order, so the
 * result is deterministic. With fewer than 1024 output tiles of 64 x 64 the
 * products are split along K into up to 4 slices whose fp32 partial sums
 * (held in the workspace) are added in slice order. A calibration-time call.
 * X: [M, ldx], W: [N, ldw], both of `dtype`, rows 16-byte aligned; Yq:
 * [M, ldy] fp32; err: one fp64 on the device (written). ws >=
 * mxs_output_error_workspace(M, N) bytes. All device pointers, owned by
 * the caller; asynchronous on `stream`. The workspace holds one fp64 per
 * tile and, when the product is split, 16 KiB of fp32 partial products per
 * tile and slice (fewer than 2048 tile slices, under 32 MiB); it must be
 * 16-byte aligned.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE (M or N < 0, K % 32, ld too small),
 * MXS_ERR_UNSUPPORTED (alignment of X or W, M > 65535 * 64),
 * MXS_ERR_WORKSPACE (too small or misaligned), MXS_ERR_DEVICE.
 */
size_t mxs_output_error_workspace(int64_t M, int64_t N);
mxs_status mxs_output_error(const void *X, const void *W, mxs_dtype dtype, int64_t M, int64_t N,
                            int64_t K, int64_t ldx, int64_t ldw, const float *Yq, int64_t ldy,
                            double *err, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Layer-wise budget under one global control parameter R ([NL] §2.3: the
 * 32 most sensitive columns of every layer get 8 bits; a layer's number of
 * 6-bit columns is proportional to its sensitivity, scaled by R so that the
 * average width meets the target B). Reading: layer l gets n8 = 1 and
 * n6 = min(nb_l - 1, floor(R S_l + 1/2)) blocks (nb_l = K_l / 32), for the
 * largest R whose average mantissa width over all weights (layer l weighted
 * by rows_l K_l) does not exceed B; the budget in bits above 4 is
 * floor((B - 4) sum_l rows_l K_l). R is found exactly, by bisection over
 * the breakpoints R S_l = j - 1/2 (equal breakpoints taken together).
 * Host call: S, rows, K: [L] host arrays (S_l >= 0 finite, e.g. from
 * mxs_output_error); nblk: [L][3] host out (n8, n6, n4 per layer); R: host
 * out, may be NULL.
 * Errors: MXS_ERR_ARG (NULL, L < 1, S negative or not finite),
 * MXS_ERR_SHAPE (rows < 1, K % 32), MXS_ERR_BUDGET (B outside [4, 8] or
 * too small for one 8-bit block per layer).
 */
mxs_status mxs_layer_budget(int32_t L, const double *S, const int64_t *rows, const int64_t *K,
                            double B, int32_t *nblk, double *R);

/*
 * MXINT quantisation of weights or activations ([NL] §1: one shared
 * power-of-two scale per block of 32; §2.2: 4/6/8-bit mantissas; [RP]
 * "Triplet Quantization": weights and activations). Row r, permuted block b
 * with width m takes v = X[r, perm[32 b .. 32 b + 31]] and stores
 *     s = clamp(floor(log2 max|v|) - (m - 2), -127, 127)   (E8M0 byte s+127)
 *     c_i = clamp(round_half_even(v_i / 2^s), -(2^(m-1)-1), 2^(m-1)-1)
 * (reading of the MX rule; all-zero block -> byte 0, NaN/Inf -> byte 0xFF,
 * codes 0), packed as described at mxs_qmat. Activation scales are computed
 * per token and block from the values at hand.
 * X: [out->rows, ldx] of `dtype`; perm: [K] int32 device array or NULL for
 * the identity; out: host struct describing the caller's output planes
 * (rows, K, n8, n6, n4, pointers, strides), all written by the call.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE, MXS_ERR_DEVICE.
 */
mxs_status mxs_quantize(const void *X, mxs_dtype dtype, int64_t ldx, const int32_t *perm,
                        const mxs_qmat *out, hipStream_t stream);

/* Workspace bytes needed by mxs_mixed_gemm for these shapes (may be 0). */
size_t mxs_mixed_gemm_workspace(const mxs_qmat *A, const mxs_qmat *W);

/*
 * Block-scaled mixed-precision GEMM ([NL] §1 and §5, [REV] "Comparison":
 * the block scales are applied inside the product, with no separate
 * dequantisation pass):
 *     Y[t, n] = sum_b 2^(sa[t,b] + sw[n,b]) * sum_{j in b} ca[t, j] cw[n, j]
 * where A (activations, A->rows = M tokens) and W (weights, W->rows = N) are
 * quantised with the same K, the same (n8, n6, n4) and the same permutation.
 * Each block's dot product is exact (from 64 tokens on: int8 MFMA with
 * int32 sums for the 4-bit blocks, exact bf16 products for the 8- and 6-bit
 * blocks; below: int32 sums); the terms are combined in fp32 (error ~
 * sqrt(K/32) ulp relative to sum |A||W|). Products with fewer than 256
 * output tiles of 256 x 128 split K into up to 8 ranges whose fp32 sums,
 * kept in the workspace, are added in range order.
 * Y: [M, ldy] fp32 device output, ldy >= N.
 * ws: >= mxs_mixed_gemm_workspace(A, W) bytes (NULL if that is 0).
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE (K or block counts differ, ldy < N),
 * MXS_ERR_UNSUPPORTED (plane pointers or strides not 16/4/8-byte aligned
 * for q8/q6/q4, more than 4194304 rows in A), MXS_ERR_WORKSPACE,
 * MXS_ERR_DEVICE.
 */
mxs_status mxs_mixed_gemm(const mxs_qmat *A, const mxs_qmat *W, float *Y, int64_t ldy,
                          void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the product
 * of mxs_mixed_gemm, same kernels and the same result bit for bit, with its
 * workspace taken from a scratch array the library holds in device memory
 * (MXS_NOALLOC_SCRATCH_BYTES per GPU, kept until the process ends) instead
 * of a caller buffer. The call allocates nothing. The caller still owns A,
 * W and Y (device memory, layout and alignment as for mxs_mixed_gemm).
 * Shapes whose mxs_mixed_gemm_workspace(A, W) exceeds
 * MXS_NOALLOC_SCRATCH_BYTES are rejected with MXS_ERR_UNSUPPORTED (for
 * example every decode shape of the Llama-2-70B MLP up to 32 tokens and the
 * 2048 x 4096 x 4096 prefill fit; 2048-token prefill at N = 28672 does not).
 * The scratch array belongs to the GPU of `stream` (the calling thread's
 * current device for the null stream); its device address is looked up once
 * per GPU on the first call there. Every call on one GPU shares that GPU's
 * array and leaves its contents behind; nothing in it needs clearing before a
 * call. Calls that overlap on one GPU (other threads, or streams that run
 * concurrently) race on the array: the caller serialises them.
 * Errors: as mxs_mixed_gemm, plus MXS_ERR_UNSUPPORTED (workspace above the
 * scratch size) and MXS_ERR_DEVICE (the scratch address lookup failed).
 */
#define MXS_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
mxs_status mxs_mixed_gemm_noalloc(const mxs_qmat *A, const mxs_qmat *W, float *Y, int64_t ldy,
                                  hipStream_t stream);

/*
 * Weights prepared once for the prefill product ([NL] §1 and §5: no
 * separate dequantisation pass inside the product). mxs_mixed_gemm expands
 * both operands' codes into the prefill kernel's operand (bf16 values for
 * the 8- and 6-bit blocks, exponent-aligned int8 codes with fp32 window
 * scales for the 4-bit blocks) in every call. Weights do not change
 * between calls, so mxs_prepare_weights builds W's half once, and
 * mxs_mixed_gemm_prepared and mxs_mixed_gemm_fused_prepared reuse it for any
 * number of tokens. Their results are bit-identical to mxs_mixed_gemm and
 * mxs_mixed_gemm_fused on the same planes.
 * wprep: device buffer of mxs_prepare_weights_size(W) bytes (0 when W has
 * no rows), 256-byte aligned, owned by the caller. Its contents are private
 * to the library (W's prepared rows, padded to 128 rows and to a multiple
 * of 128 bytes, then fp32 scales per 32-byte unit and row). It stays valid while W's
 * planes and shape are unchanged; a buffer prepared from other planes of the
 * same shape gives wrong results but no out-of-bounds access.
 * mxs_mixed_gemm_prepared: A, W, Y, ldy as for mxs_mixed_gemm (W's planes
 * are still read by the kernels for up to 63 rows of A), ws >=
 * mxs_mixed_gemm_prepared_workspace(A, W) bytes, 256-byte aligned (A's
 * prepared operand only). mxs_mixed_gemm_fused_prepared: arguments as
 * mxs_mixed_gemm_fused, ws >= mxs_mixed_gemm_fused_prepared_workspace(M,
 * dtype, W) bytes. All asynchronous on `stream`.
 * Errors: as the calls without preparation, plus MXS_ERR_WORKSPACE when
 * wprep is NULL, too small or misaligned. mxs_prepare_weights_size returns
 * 0 for a NULL W or a K that is not a positive multiple of 32.
 */
size_t mxs_prepare_weights_size(const mxs_qmat *W);
mxs_status mxs_prepare_weights(const mxs_qmat *W, void *wprep, size_t wprep_bytes, hipStream_t stream);
size_t mxs_mixed_gemm_prepared_workspace(const mxs_qmat *A, const mxs_qmat *W);
mxs_status mxs_mixed_gemm_prepared(const mxs_qmat *A, const mxs_qmat *W, const void *wprep, size_t wprep_bytes,
                                   float *Y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes needed by mxs_mixed_gemm_mx for these shapes (may be 0). */
size_t mxs_mixed_gemm_mx_workspace(const mxs_qmat *A, const mxs_qmat *W);

/*
 * The same product as mxs_mixed_gemm, with the prefill kernels (64 or more
 * rows in A) on the block-scaled micro-float matrix cores, which apply one
 * E8M0 scale per 32 elements of every row and column inside the instruction
 * (the MX format's shared block scale, [NL] §1). Codes are re-encoded exactly
 * as fp6 E2M3 elements (a 4-bit code as one element, a 6- or 8-bit code as
 * two digits whose weight goes into the scale byte); every product and each
 * 64-element partial sum is exact, only the fp32 accumulation rounds (once
 * per instruction). Up to 63 rows it runs the kernels of mxs_mixed_gemm.
 * Shapes with fewer than 64 output tiles of 256 x 256 split K into up to 8
 * ranges whose fp32 sums, kept in the workspace, are added in range order,
 * so the result is deterministic.
 * Arguments, layout, ownership, stream semantics and errors as for
 * mxs_mixed_gemm, with ws >= mxs_mixed_gemm_mx_workspace(A, W) bytes.
 */
mxs_status mxs_mixed_gemm_mx(const mxs_qmat *A, const mxs_qmat *W, float *Y, int64_t ldy,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Activation quantisation fused into the product ([NL] §1 and §2.3, [RP]
 * "Triplet Quantization": activations quantised with the weight's channel
 * map): Y = mixed_gemm(quantize(X, perm at W's block counts), W), the same
 * result bit for bit as mxs_quantize into planes followed by mxs_mixed_gemm.
 * With 64 or more rows (and, for the row staging, K <= 65536 with
 * K * (2 + element size) <= 96 KiB) the activation rows are quantised
 * straight into the prefill kernel's operand, so no
 * activation planes are written or read; other shapes quantise into planes
 * kept in the workspace and run the mxs_mixed_gemm kernels.
 * X: [M, ldx >= K] row-major of `dtype` (device); perm: [K] int32 gather
 * form (X column perm[j] becomes position j) or NULL for the identity;
 * W: quantised weights (device planes, the plane alignment mxs_mixed_gemm
 * asks for); Y: [M, ldy >= N] fp32 (device). ws >=
 * mxs_mixed_gemm_fused_workspace(M, dtype, W) bytes, 256-byte aligned, owned
 * by the caller; asynchronous on `stream`.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE, MXS_ERR_UNSUPPORTED (more than 2^22
 * rows, misaligned planes), MXS_ERR_WORKSPACE, MXS_ERR_DEVICE.
 */
size_t mxs_mixed_gemm_fused_workspace(int64_t M, mxs_dtype dtype, const mxs_qmat *W);
mxs_status mxs_mixed_gemm_fused(const void *X, mxs_dtype dtype, int64_t M, int64_t ldx, const int32_t *perm,
                                const mxs_qmat *W, float *Y, int64_t ldy, void *ws, size_t ws_bytes,
                                hipStream_t stream);
size_t mxs_mixed_gemm_fused_prepared_workspace(int64_t M, mxs_dtype dtype, const mxs_qmat *W);
mxs_status mxs_mixed_gemm_fused_prepared(const void *X, mxs_dtype dtype, int64_t M, int64_t ldx,
                                         const int32_t *perm, const mxs_qmat *W, const void *wprep,
                                         size_t wprep_bytes, float *Y, int64_t ldy, void *ws, size_t ws_bytes,
                                         hipStream_t stream);

/*
 * KV-cache quantisation (W4A4KV4, [NL] §4 and [REV] "Validation": keys and
 * values stored as 4-bit MXINT). Reading: uniform 4-bit, blocks of 32
 * consecutive elements along the head dimension, no permutation.
 * kv: [T, H, D] contiguous of `dtype`; codes: [T, H, D/2] uint8 (4-bit
 * packing of mxs_qmat); scales: [T, H, D/32] uint8 E8M0. D % 32 == 0.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE, MXS_ERR_DEVICE.
 */
mxs_status mxs_quantize_kv(const void *kv, mxs_dtype dtype, int64_t T, int64_t H, int64_t D,
                           uint8_t *codes, uint8_t *scales, hipStream_t stream);

/*
 * Attention of one query token over the 4-bit K/V cache ([NL] §4,
 * W4A4KV4: keys and values kept as 4-bit MXINT, as written by
 * mxs_quantize_kv). Reading: plain scaled dot-product attention, query head
 * h reading KV head h / (Hq / Hkv):
 *     s_t = scale * sum_d q[h,d] K[t,g,d],  p = softmax_t(s),
 *     out[h,d] = sum_t p_t V[t,g,d],
 * with K, V dequantized exactly (code * 2^(byte - 127)). Exact products
 * (the fp32 query and softmax weights enter the bf16 matrix cores as exact
 * three-part sums) with fp32 sums, every sum in a fixed order
 * (deterministic); the result matches the fp64 definition within the
 * rounding of the score dot products, the exponentials and the T-term
 * sums.
 * q: [Hq, D] fp32; kc, vc: [T, Hkv, D/2] uint8 codes (16-byte aligned);
 * ks, vs: [T, Hkv, D/32] uint8 E8M0 scales; out: [Hq, D] fp32 (16-byte
 * aligned). All device pointers owned by the caller; ws >=
 * mxs_attend_kv4_workspace(T, Hq, Hkv, D) bytes, 16-byte aligned;
 * asynchronous on `stream`. Hq / Hkv <= 16, D <= 256, D % 32 == 0,
 * T <= 65535 * 64.
 * Errors: MXS_ERR_ARG, MXS_ERR_SHAPE, MXS_ERR_UNSUPPORTED, MXS_ERR_WORKSPACE,
 * MXS_ERR_DEVICE.
 */
size_t mxs_attend_kv4_workspace(int64_t T, int64_t Hq, int64_t Hkv, int64_t D);
mxs_status mxs_attend_kv4(const float *q, const uint8_t *kc, const uint8_t *ks, const uint8_t *vc,
                          const uint8_t *vs, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                          float *out, void *ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXSENS_H */
