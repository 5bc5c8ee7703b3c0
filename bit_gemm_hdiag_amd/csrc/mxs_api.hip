// mxs_api.hip -- extern "C" entry points of libmxsens: argument checks,
// workspace sizing and kernel launches on the caller's stream.
#include <stdarg.h>
#include <stdio.h>
#include <math.h>
#include <string.h>

#include <mutex>

#include "mxs_internal.h"

// Workspace of mxs_mixed_gemm_noalloc: one copy per GPU in device memory,
// loaded with the code object and kept until the process ends. Host code
// never passes the name itself to a kernel (on the host it stands for a
// host-side handle, not a device address); it uses the address from
// hipGetSymbolAddress, looked up per device below.
static __device__ __align__(256) uint8_t scratch[MXS_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

mxs_status fail(mxs_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

mxs_status ok() {
    g_err[0] = '\0';
    return MXS_OK;
}

mxs_status device_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(MXS_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(mxs_dtype d) { return d == MXS_F32 || d == MXS_BF16; }

int64_t nchunks(int64_t rows) { return mxs::ceil_div(rows, mxs::kChunkRows); }

size_t colsum_ws(int64_t rows, int64_t K, bool score) {
    if (rows <= 0 || K <= 0) return 0;
    const int64_t n = nchunks(rows);
    if (n <= 1) return 0;
    const int64_t per = n < mxs::kMaxChunksPerLaunch ? n : mxs::kMaxChunksPerLaunch;
    return (size_t)(per + (score ? 1 : 0)) * (size_t)K * sizeof(double);
}

bool aligned(const void *p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// Device address of `scratch` on the GPU of `stream`, looked up once per GPU
// with that GPU current (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];

hipError_t scratch_address(hipStream_t stream, void **out) {
    int dev = -1, cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (stream) {
        if ((e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
    } else {
        dev = cur;
    }
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

mxs_status check_qmat(const mxs_qmat *q, const char *name) {
    if (!q) return fail(MXS_ERR_ARG, "%s is NULL", name);
    if (q->rows < 0 || q->K <= 0 || q->K % 32) return fail(MXS_ERR_SHAPE, "%s: rows=%lld K=%lld (K must be a positive multiple of 32)", name, (long long)q->rows, (long long)q->K);
    if (q->n8 < 0 || q->n6 < 0 || q->n4 < 0 || (int64_t)q->n8 + q->n6 + q->n4 != q->K / 32)
        return fail(MXS_ERR_SHAPE, "%s: block counts %d/%d/%d do not sum to K/32=%lld", name, q->n8, q->n6, q->n4, (long long)(q->K / 32));
    if (q->reserved != 0) return fail(MXS_ERR_ARG, "%s: reserved field must be 0", name);
    if (q->rows == 0) return MXS_OK;   // nothing is read or written
    if (!q->sc) return fail(MXS_ERR_ARG, "%s: scale plane is NULL", name);
    if (q->lds < q->K / 32) return fail(MXS_ERR_SHAPE, "%s: lds < K/32", name);
    if (q->n8 && (!q->q8 || q->ld8 < 32LL * q->n8)) return fail(q->q8 ? MXS_ERR_SHAPE : MXS_ERR_ARG, "%s: 8-bit plane missing or ld8 < 32*n8", name);
    if (q->n6 && (!q->q6 || q->ld6 < 24LL * q->n6)) return fail(q->q6 ? MXS_ERR_SHAPE : MXS_ERR_ARG, "%s: 6-bit plane missing or ld6 < 24*n6", name);
    if (q->n4 && (!q->q4 || q->ld4 < 16LL * q->n4)) return fail(q->q4 ? MXS_ERR_SHAPE : MXS_ERR_ARG, "%s: 4-bit plane missing or ld4 < 16*n4", name);
    return MXS_OK;
}

}  // namespace

extern "C" {

const char *mxs_status_string(mxs_status s) {
    switch (s) {
        case MXS_OK: return "MXS_OK";
        case MXS_ERR_ARG: return "MXS_ERR_ARG";
        case MXS_ERR_SHAPE: return "MXS_ERR_SHAPE";
        case MXS_ERR_BUDGET: return "MXS_ERR_BUDGET";
        case MXS_ERR_WORKSPACE: return "MXS_ERR_WORKSPACE";
        case MXS_ERR_DEVICE: return "MXS_ERR_DEVICE";
        case MXS_ERR_UNSUPPORTED: return "MXS_ERR_UNSUPPORTED";
        default: return "MXS_UNKNOWN_STATUS";
    }
}

const char *mxs_last_error(void) { return g_err; }

int32_t mxs_version(void) { return 1; }

mxs_status mxs_budget_blocks(int64_t K, int32_t bp8, int32_t bp6, int32_t nblk[3]) {
    if (!nblk) return fail(MXS_ERR_ARG, "nblk is NULL");
    if (K <= 0 || K % 32) return fail(MXS_ERR_SHAPE, "K=%lld must be a positive multiple of 32", (long long)K);
    if (bp8 < 0 || bp6 < 0 || (int64_t)bp8 + bp6 > 10000)
        return fail(MXS_ERR_BUDGET, "budget bp8=%d bp6=%d outside [0, 10000]", bp8, bp6);
    const int64_t nb = K / 32;
    const int64_t U = nb * (2 * (int64_t)bp8 + bp6) / 10000;
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
    return ok();
}

size_t mxs_calibrate_workspace(int64_t M, int64_t K) { return colsum_ws(M, K, false); }
size_t mxs_score_workspace(int64_t N, int64_t K) { return colsum_ws(N, K, true); }

mxs_status mxs_calibrate(const void *X, mxs_dtype dtype, int64_t M, int64_t K, int64_t ldx,
                         double *hdiag, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return fail(MXS_ERR_ARG, "unknown dtype %d", (int)dtype);
    if (M < 0 || K <= 0 || K % 32 || ldx < K)
        return fail(MXS_ERR_SHAPE, "calibrate: M=%lld K=%lld ldx=%lld", (long long)M, (long long)K, (long long)ldx);
    if (!hdiag || (M > 0 && !X)) return fail(MXS_ERR_ARG, "calibrate: NULL pointer");
    const size_t need = colsum_ws(M, K, false);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 16)))
        return fail(MXS_ERR_WORKSPACE, "calibrate: workspace needs %zu bytes (got %zu)", need, ws ? ws_bytes : 0);
    if (M == 0) return ok();
    return device_status(mxs::launch_calibrate(X, dtype, M, K, ldx, hdiag, static_cast<double *>(ws), stream), "calibrate");
}

mxs_status mxs_score(const void *W, mxs_dtype dtype, int64_t N, int64_t K, int64_t ldw,
                     const double *hdiag, double *score, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return fail(MXS_ERR_ARG, "unknown dtype %d", (int)dtype);
    if (N <= 0 || K <= 0 || K % 32 || ldw < K)
        return fail(MXS_ERR_SHAPE, "score: N=%lld K=%lld ldw=%lld", (long long)N, (long long)K, (long long)ldw);
    if (!W || !hdiag || !score) return fail(MXS_ERR_ARG, "score: NULL pointer");
    const size_t need = colsum_ws(N, K, true);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 16)))
        return fail(MXS_ERR_WORKSPACE, "score: workspace needs %zu bytes (got %zu)", need, ws ? ws_bytes : 0);
    return device_status(mxs::launch_score(W, dtype, N, K, ldw, hdiag, score, static_cast<double *>(ws), stream), "score");
}

mxs_status mxs_allocate(const double *score, int64_t K, int32_t bp8, int32_t bp6, uint8_t *bits,
                        int32_t *perm, hipStream_t stream) {
    int32_t nb3[3];
    mxs_status s = mxs_budget_blocks(K, bp8, bp6, nb3);
    if (s != MXS_OK) return s;
    if (!score || !bits || !perm) return fail(MXS_ERR_ARG, "allocate: NULL pointer");
    if (K > 131072) return fail(MXS_ERR_UNSUPPORTED, "allocate: K=%lld above 131072", (long long)K);
    return device_status(mxs::launch_allocate(score, K, 32 * nb3[0], 32 * nb3[1], bits, perm, stream), "allocate");
}

mxs_status mxs_allocate_blocks(const double *score, int64_t K, int32_t n8, int32_t n6, uint8_t *bits,
                               int32_t *perm, hipStream_t stream) {
    if (K <= 0 || K % 32) return fail(MXS_ERR_SHAPE, "allocate_blocks: K=%lld must be a positive multiple of 32", (long long)K);
    if (n8 < 0 || n6 < 0 || (int64_t)n8 + n6 > K / 32)
        return fail(MXS_ERR_BUDGET, "allocate_blocks: n8=%d n6=%d outside 0..K/32=%lld", n8, n6, (long long)(K / 32));
    if (!score || !bits || !perm) return fail(MXS_ERR_ARG, "allocate_blocks: NULL pointer");
    if (K > 131072) return fail(MXS_ERR_UNSUPPORTED, "allocate_blocks: K=%lld above 131072", (long long)K);
    return device_status(mxs::launch_allocate(score, K, 32 * n8, 32 * n6, bits, perm, stream), "allocate_blocks");
}

mxs_status mxs_layer_budget(int32_t L, const double *S, const int64_t *rows, const int64_t *K, double B,
                            int32_t *nblk, double *R) {
    if (L < 1 || !S || !rows || !K || !nblk) return fail(MXS_ERR_ARG, "layer_budget: L < 1 or NULL pointer");
    for (int32_t l = 0; l < L; ++l) {
        if (!(S[l] >= 0.0) || S[l] == HUGE_VAL) return fail(MXS_ERR_ARG, "layer_budget: S[%d] is negative or not finite", l);
        if (rows[l] < 1 || K[l] < 32 || K[l] % 32)
            return fail(MXS_ERR_SHAPE, "layer_budget: layer %d has rows=%lld K=%lld", l, (long long)rows[l], (long long)K[l]);
    }
    if (!(B >= 4.0 && B <= 8.0)) return fail(MXS_ERR_BUDGET, "layer_budget: B=%g outside [4, 8]", B);
    if (mxs::layer_budget(L, S, rows, K, B, nblk, R))
        return fail(MXS_ERR_BUDGET, "layer_budget: B=%g cannot pay for one 8-bit block per layer", B);
    return ok();
}

size_t mxs_output_error_workspace(int64_t M, int64_t N) {
    return mxs::output_error_workspace(M > 0 ? M : 0, N > 0 ? N : 0);
}

mxs_status mxs_output_error(const void *X, const void *W, mxs_dtype dtype, int64_t M, int64_t N, int64_t K,
                            int64_t ldx, int64_t ldw, const float *Yq, int64_t ldy, double *err, void *ws,
                            size_t ws_bytes, hipStream_t stream) {
    if (!dtype_ok(dtype)) return fail(MXS_ERR_ARG, "output_error: unknown dtype %d", (int)dtype);
    if (M < 0 || N < 0 || K < 32 || K % 32 || ldx < K || ldw < K || ldy < N)
        return fail(MXS_ERR_SHAPE, "output_error: M=%lld N=%lld K=%lld ldx=%lld ldw=%lld ldy=%lld", (long long)M,
                    (long long)N, (long long)K, (long long)ldx, (long long)ldw, (long long)ldy);
    if (!err || !ws || (M > 0 && !X) || (N > 0 && !W) || (M > 0 && N > 0 && !Yq))
        return fail(MXS_ERR_ARG, "output_error: NULL pointer");
    const size_t es = dtype == MXS_BF16 ? 2 : 4;
    if ((M > 0 && (!aligned(X, 16) || (ldx * es) % 16)) || (N > 0 && (!aligned(W, 16) || (ldw * es) % 16)))
        return fail(MXS_ERR_UNSUPPORTED, "output_error: X and W rows need 16-byte alignment");
    if (M > (int64_t)65535 * 64) return fail(MXS_ERR_UNSUPPORTED, "output_error: M=%lld above 65535 * 64", (long long)M);
    if (ws_bytes < mxs::output_error_workspace(M, N) || !aligned(ws, 16))
        return fail(MXS_ERR_WORKSPACE, "output_error: workspace smaller than %zu bytes or not 16-byte aligned",
                    mxs::output_error_workspace(M, N));
    return device_status(mxs::launch_output_error(X, W, dtype, M, N, K, ldx, ldw, Yq, ldy, err, ws, stream),
                         "output_error");
}

size_t mxs_attend_kv4_workspace(int64_t T, int64_t Hq, int64_t Hkv, int64_t D) {
    if (T <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
    return mxs::attend_kv4_workspace(T, Hq, Hkv, D);
}

mxs_status mxs_attend_kv4(const float *q, const uint8_t *kc, const uint8_t *ks, const uint8_t *vc,
                          const uint8_t *vs, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                          float *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    if (!q || !kc || !ks || !vc || !vs || !out || !ws) return fail(MXS_ERR_ARG, "attend_kv4: NULL pointer");
    if (T < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || D < 32 || D % 32)
        return fail(MXS_ERR_SHAPE, "attend_kv4: T=%lld Hq=%lld Hkv=%lld D=%lld", (long long)T, (long long)Hq,
                    (long long)Hkv, (long long)D);
    if (!mxs::attend_kv4_supported(Hq, Hkv, D) || !aligned(kc, 16) || !aligned(vc, 16) || !aligned(q, 4) ||
        !aligned(out, 16))
        return fail(MXS_ERR_UNSUPPORTED, "attend_kv4: needs Hq/Hkv <= 16, D <= 256, 16-byte aligned codes and output");
    if (T > (int64_t)65535 * 64) return fail(MXS_ERR_UNSUPPORTED, "attend_kv4: T=%lld too long", (long long)T);
    if (ws_bytes < mxs::attend_kv4_workspace(T, Hq, Hkv, D) || !aligned(ws, 16))
        return fail(MXS_ERR_WORKSPACE, "attend_kv4: workspace too small or not 16-byte aligned");
    return device_status(mxs::launch_attend_kv4(q, kc, ks, vc, vs, T, Hq, Hkv, D, scale, out, ws, stream),
                         "attend_kv4");
}

mxs_status mxs_quantize(const void *X, mxs_dtype dtype, int64_t ldx, const int32_t *perm,
                        const mxs_qmat *out, hipStream_t stream) {
    if (!dtype_ok(dtype)) return fail(MXS_ERR_ARG, "unknown dtype %d", (int)dtype);
    mxs_status s = check_qmat(out, "quantize out");
    if (s != MXS_OK) return s;
    if (ldx < out->K) return fail(MXS_ERR_SHAPE, "quantize: ldx=%lld < K=%lld", (long long)ldx, (long long)out->K);
    if (out->rows > 0 && !X) return fail(MXS_ERR_ARG, "quantize: X is NULL");
    return device_status(mxs::launch_quantize(X, dtype, ldx, perm, *out, stream), "quantize");
}

size_t mxs_mixed_gemm_workspace(const mxs_qmat *A, const mxs_qmat *W) {
    if (!A || !W) return 0;
    return mxs::gemm_workspace(*A, *W, false);
}

size_t mxs_mixed_gemm_prepared_workspace(const mxs_qmat *A, const mxs_qmat *W) {
    if (!A || !W) return 0;
    return mxs::gemm_workspace(*A, *W, true);
}

size_t mxs_prepare_weights_size(const mxs_qmat *W) {
    if (!W || W->rows < 0 || W->K <= 0 || W->K % 32) return 0;
    return mxs::wprep_bytes(*W);
}

// Operand loads are 16/4/8-byte vector loads per row.
static mxs_status check_planes_aligned(const mxs_qmat *m, const char *name) {
    if ((m->n8 && (!aligned(m->q8, 16) || m->ld8 % 16)) || (m->n6 && (!aligned(m->q6, 4) || m->ld6 % 4)) ||
        (m->n4 && (!aligned(m->q4, 8) || m->ld4 % 8)))
        return fail(MXS_ERR_UNSUPPORTED, "%s: planes need q8/ld8 16-byte, q6/ld6 4-byte and q4/ld4 8-byte alignment", name);
    return MXS_OK;
}

// Argument checks shared by both GEMM entry points.
static mxs_status check_gemm(const mxs_qmat *A, const mxs_qmat *W, const float *Y, int64_t ldy, const void *ws,
                             size_t ws_bytes, size_t need, const char *name) {
    mxs_status s = check_qmat(A, "A");
    if (s != MXS_OK) return s;
    if ((s = check_qmat(W, "W")) != MXS_OK) return s;
    if (A->K != W->K || A->n8 != W->n8 || A->n6 != W->n6 || A->n4 != W->n4)
        return fail(MXS_ERR_SHAPE, "%s: A and W differ in K or block counts", name);
    if (ldy < W->rows || (!Y && A->rows > 0 && W->rows > 0)) return fail(Y ? MXS_ERR_SHAPE : MXS_ERR_ARG, "%s: Y NULL or ldy < N", name);
    if ((s = check_planes_aligned(A, name)) != MXS_OK || (s = check_planes_aligned(W, name)) != MXS_OK) return s;
    if (A->rows > (int64_t)1 << 22) return fail(MXS_ERR_UNSUPPORTED, "%s: more than 4194304 rows in A", name);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256)))
        return fail(MXS_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", name, need, ws ? ws_bytes : 0);
    return MXS_OK;
}

// The prepared-weights buffer: mxs_prepare_weights_size(W) bytes, 256-byte
// aligned.
static mxs_status check_wprep(const mxs_qmat *W, const void *wprep, size_t wprep_bytes, const char *name) {
    const size_t need = mxs::wprep_bytes(*W);
    if (need && (!wprep || wprep_bytes < need || !aligned(wprep, 256)))
        return fail(MXS_ERR_WORKSPACE, "%s: prepared weights need %zu bytes, 256-byte aligned (got %zu)", name, need,
                    wprep ? wprep_bytes : 0);
    return MXS_OK;
}

mxs_status mxs_mixed_gemm(const mxs_qmat *A, const mxs_qmat *W, float *Y, int64_t ldy, void *ws,
                          size_t ws_bytes, hipStream_t stream) {
    const size_t need = A && W ? mxs::gemm_workspace(*A, *W, false) : 0;
    const mxs_status s = check_gemm(A, W, Y, ldy, ws, ws_bytes, need, "mixed_gemm");
    if (s != MXS_OK) return s;
    return device_status(mxs::launch_mixed_gemm(*A, *W, nullptr, Y, ldy, ws, stream), "mixed_gemm");
}

mxs_status mxs_prepare_weights(const mxs_qmat *W, void *wprep, size_t wprep_bytes, hipStream_t stream) {
    mxs_status s = check_qmat(W, "W");
    if (s != MXS_OK) return s;
    if ((s = check_planes_aligned(W, "prepare_weights")) != MXS_OK) return s;
    if ((s = check_wprep(W, wprep, wprep_bytes, "prepare_weights")) != MXS_OK) return s;
    return device_status(mxs::launch_prepare_weights(*W, wprep, stream), "prepare_weights");
}

mxs_status mxs_mixed_gemm_prepared(const mxs_qmat *A, const mxs_qmat *W, const void *wprep, size_t wprep_bytes,
                                   float *Y, int64_t ldy, void *ws, size_t ws_bytes, hipStream_t stream) {
    const size_t need = A && W ? mxs::gemm_workspace(*A, *W, true) : 0;
    mxs_status s = check_gemm(A, W, Y, ldy, ws, ws_bytes, need, "mixed_gemm_prepared");
    if (s != MXS_OK) return s;
    if ((s = check_wprep(W, wprep, wprep_bytes, "mixed_gemm_prepared")) != MXS_OK) return s;
    return device_status(mxs::launch_mixed_gemm(*A, *W, wprep, Y, ldy, ws, stream), "mixed_gemm_prepared");
}

mxs_status mxs_mixed_gemm_noalloc(const mxs_qmat *A, const mxs_qmat *W, float *Y, int64_t ldy,
                                  hipStream_t stream) {
    mxs_status s = check_gemm(A, W, Y, ldy, nullptr, 0, 0, "mixed_gemm_noalloc");   // arguments first
    if (s != MXS_OK) return s;
    const size_t need = mxs::gemm_workspace(*A, *W, false);
    if (need > MXS_NOALLOC_SCRATCH_BYTES)
        return fail(MXS_ERR_UNSUPPORTED, "mixed_gemm_noalloc: these shapes need %zu bytes of workspace, above the "
                    "%zu-byte scratch array (use mxs_mixed_gemm with a caller workspace)", need,
                    (size_t)MXS_NOALLOC_SCRATCH_BYTES);
    void *ws = nullptr;
    if (need) {
        const hipError_t e = scratch_address(stream, &ws);
        if (e != hipSuccess) return device_status(e, "mixed_gemm_noalloc: scratch address");
    }
    return device_status(mxs::launch_mixed_gemm(*A, *W, nullptr, Y, ldy, ws, stream), "mixed_gemm_noalloc");
}

size_t mxs_mixed_gemm_fused_workspace(int64_t M, mxs_dtype dtype, const mxs_qmat *W) {
    if (!W || !dtype_ok(dtype) || M < 0 || W->K <= 0 || W->K % 32) return 0;
    return mxs::gemm_fused_workspace(M, dtype, *W, false);
}

size_t mxs_mixed_gemm_fused_prepared_workspace(int64_t M, mxs_dtype dtype, const mxs_qmat *W) {
    if (!W || !dtype_ok(dtype) || M < 0 || W->K <= 0 || W->K % 32) return 0;
    return mxs::gemm_fused_workspace(M, dtype, *W, true);
}

// Argument checks shared by both fused entry points.
static mxs_status check_fused(const void *X, mxs_dtype dtype, int64_t M, int64_t ldx, const mxs_qmat *W,
                              const float *Y, int64_t ldy, const void *ws, size_t ws_bytes, bool w_prepared,
                              const char *name) {
    if (!dtype_ok(dtype)) return fail(MXS_ERR_ARG, "%s: unknown dtype %d", name, (int)dtype);
    mxs_status s = check_qmat(W, "W");
    if (s != MXS_OK) return s;
    if (M < 0 || ldx < W->K) return fail(MXS_ERR_SHAPE, "%s: M=%lld ldx=%lld K=%lld", name, (long long)M, (long long)ldx, (long long)W->K);
    if (M > (int64_t)1 << 22) return fail(MXS_ERR_UNSUPPORTED, "%s: more than 4194304 rows in X", name);
    const bool work = M > 0 && W->rows > 0;
    if (work && !X) return fail(MXS_ERR_ARG, "%s: X is NULL", name);
    if (ldy < W->rows || (!Y && work)) return fail(Y ? MXS_ERR_SHAPE : MXS_ERR_ARG, "%s: Y NULL or ldy < N", name);
    if ((s = check_planes_aligned(W, name)) != MXS_OK) return s;
    const size_t need = mxs::gemm_fused_workspace(M, dtype, *W, w_prepared);
    if (need && (!ws || ws_bytes < need || !aligned(ws, 256)))
        return fail(MXS_ERR_WORKSPACE, "%s: workspace needs %zu bytes (got %zu)", name, need, ws ? ws_bytes : 0);
    return MXS_OK;
}

mxs_status mxs_mixed_gemm_fused(const void *X, mxs_dtype dtype, int64_t M, int64_t ldx, const int32_t *perm,
                                const mxs_qmat *W, float *Y, int64_t ldy, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
    const mxs_status s = check_fused(X, dtype, M, ldx, W, Y, ldy, ws, ws_bytes, false, "mixed_gemm_fused");
    if (s != MXS_OK) return s;
    return device_status(mxs::launch_mixed_gemm_fused(X, dtype, M, ldx, perm, *W, nullptr, Y, ldy, ws, stream),
                         "mixed_gemm_fused");
}

mxs_status mxs_mixed_gemm_fused_prepared(const void *X, mxs_dtype dtype, int64_t M, int64_t ldx,
                                         const int32_t *perm, const mxs_qmat *W, const void *wprep,
                                         size_t wprep_bytes, float *Y, int64_t ldy, void *ws, size_t ws_bytes,
                                         hipStream_t stream) {
    mxs_status s = check_fused(X, dtype, M, ldx, W, Y, ldy, ws, ws_bytes, true, "mixed_gemm_fused_prepared");
    if (s != MXS_OK) return s;
    if ((s = check_wprep(W, wprep, wprep_bytes, "mixed_gemm_fused_prepared")) != MXS_OK) return s;
    return device_status(mxs::launch_mixed_gemm_fused(X, dtype, M, ldx, perm, *W, wprep, Y, ldy, ws, stream),
                         "mixed_gemm_fused_prepared");
}

size_t mxs_mixed_gemm_mx_workspace(const mxs_qmat *A, const mxs_qmat *W) {
    if (!A || !W) return 0;
    return mxs::gemm_workspace_mx(*A, *W);
}

mxs_status mxs_mixed_gemm_mx(const mxs_qmat *A, const mxs_qmat *W, float *Y, int64_t ldy, void *ws,
                             size_t ws_bytes, hipStream_t stream) {
    const size_t need = A && W ? mxs::gemm_workspace_mx(*A, *W) : 0;
    const mxs_status s = check_gemm(A, W, Y, ldy, ws, ws_bytes, need, "mixed_gemm_mx");
    if (s != MXS_OK) return s;
    return device_status(mxs::launch_mixed_gemm_mx(*A, *W, Y, ldy, ws, ws_bytes, stream), "mixed_gemm_mx");
}

mxs_status mxs_quantize_kv(const void *kv, mxs_dtype dtype, int64_t T, int64_t H, int64_t D,
                           uint8_t *codes, uint8_t *scales, hipStream_t stream) {
    if (!dtype_ok(dtype)) return fail(MXS_ERR_ARG, "unknown dtype %d", (int)dtype);
    if (T < 0 || H <= 0 || D <= 0 || D % 32) return fail(MXS_ERR_SHAPE, "quantize_kv: T=%lld H=%lld D=%lld", (long long)T, (long long)H, (long long)D);
    if (T > 0 && (!kv || !codes || !scales)) return fail(MXS_ERR_ARG, "quantize_kv: NULL pointer");
    mxs_qmat o;
    memset(&o, 0, sizeof o);
    o.rows = T * H;
    o.K = D;
    o.n4 = (int32_t)(D / 32);
    o.q4 = codes;
    o.ld4 = D / 2;
    o.sc = scales;
    o.lds = D / 32;
    return device_status(mxs::launch_quantize(kv, dtype, D, nullptr, o, stream), "quantize_kv");
}

}  // extern "C"
