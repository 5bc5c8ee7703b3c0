// mxs_colsum.hip -- calibration (Hessian diagonal) and column sensitivity
// score on gfx950.
//
// Hdiag[k] = sum_t X[t,k]^2 (gist.science/nl "Technische Samenvatting"
// §2.1, column-wise sensitivity from the diagonal of H = X^T X), and
// score[k] = Hdiag[k] * sum_n (W[n,k] - Q4(W)[n,k])^2 (reading of the same
// section: the squared uniform-MXINT4 error of column k weighted by its
// Hessian diagonal).
//
// Both are HBM-streaming column reductions with a fixed fp64 summation
// order, so results are bit-identical to any implementation of that order:
//   rows in chunks of 256; within a chunk, partial sum p_i over the rows
//   whose offset is i mod 8, in row order from +0; chunk total
//   ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)); chunk totals added in chunk order.
//
// Mapping: a wavefront is 8 row groups x 8 lanes; lane (g, c) owns 8
// consecutive columns (one 16-byte bf16 load per row) and the partial sum
// p_g of its chunk, so each wave streams 8 rows x 64 columns per step and the
// 4 waves of a workgroup cover 256 adjacent columns. The tree is three
// cross-lane xor steps (8, 16, 32). Chunk totals go to a workspace and a
// second kernel adds them in chunk order; a single chunk is written directly.
// In the score kernel the 4 lanes of a quad hold one 32-column MXINT4 block
// of a row, so the block maximum is two DPP steps.
#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

constexpr int kWaveCols = 64;   // columns per wavefront
constexpr int kWgCols = 256;    // columns per workgroup

// Residual of 8 values of one row under uniform MXINT4 (the quad holds the
// block), squared into the fp64 partial sums. d = v - c * 2^s is exact in
// fp32 (fma with a power of two whose result is representable), its square
// exact in fp64.
__device__ __forceinline__ void acc_residual_sq(const float v[8], double acc[8]) {
    int c[8];
    BlockScale bs = quantize8(v, 4, c);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        float d = __builtin_fmaf(-(float)c[i], bs.scale, v[i]);
        d = bs.bad ? __builtin_nanf("") : d;
        double dd = (double)d;
        acc[i] = __builtin_fma(dd, dd, acc[i]);
    }
}

__device__ __forceinline__ void acc_sq(const float v[8], double acc[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        double x = (double)v[i];
        acc[i] = __builtin_fma(x, x, acc[i]);
    }
}

// MODE 0: calibrate, write chunk totals to part[chunk][K]
// MODE 1: calibrate, single chunk: hdiag[k] += total
// MODE 2: score, write chunk totals to part[chunk][K]
// MODE 3: score, single chunk: score[k] = hdiag[k] * total
template <typename T, bool VEC, int MODE>
__global__ __launch_bounds__(256) void k_colsum(const T *__restrict__ X, int64_t M, int64_t K,
                                                int64_t ldx, int64_t chunk0,
                                                double *__restrict__ out,
                                                const double *__restrict__ hdiag) {
    constexpr bool kScore = MODE >= 2;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 3;
    const int64_t col0 = (int64_t)blockIdx.x * kWgCols + wave * kWaveCols + (lane & 7) * 8;
    const int64_t r0 = (chunk0 + blockIdx.y) * kChunkRows;
    const int64_t r1 = r0 + kChunkRows < M ? r0 + kChunkRows : M;

    double acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0;

    if (col0 < K) {  // K % 32 == 0: a quad is either wholly in or wholly out
        const T *p = X + col0;
        int64_t r = r0 + g;
        // eight rows of the lane's chain in flight, consumed in row order
        for (; r + 56 < r1; r += 64) {
            float v[8][8];
#pragma unroll
            for (int u = 0; u < 8; ++u) load8<T, VEC>(p + (r + 8 * u) * ldx, v[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (kScore) acc_residual_sq(v[u], acc);
                else acc_sq(v[u], acc);
            }
        }
        for (; r < r1; r += 8) {
            float v0[8];
            load8<T, VEC>(p + r * ldx, v0);
            if (kScore) acc_residual_sq(v0, acc);
            else acc_sq(v0, acc);
        }
    }

    // ((p0+p1)+(p2+p3)) + ((p4+p5)+(p6+p7)) across the row groups
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        double x = acc[i];
        x = x + __shfl_xor(x, 8);
        x = x + __shfl_xor(x, 16);
        x = x + __shfl_xor(x, 32);
        acc[i] = x;
    }
    if (g != 0 || col0 >= K) return;

    if (MODE == 0 || MODE == 2) {
        double *dst = out + (int64_t)blockIdx.y * K + col0;
#pragma unroll
        for (int i = 0; i < 8; i += 2) *reinterpret_cast<double2 *>(dst + i) = make_double2(acc[i], acc[i + 1]);
    } else if (MODE == 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[col0 + i] = out[col0 + i] + acc[i];
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) out[col0 + i] = hdiag[col0 + i] * (0.0 + acc[i]);
    }
}

// Ordered combination of chunk totals.
// calibrate: acc[k] += part[0][k]; acc[k] += part[1][k]; ...
// score: e = (init ? 0 : E[k]) + part[0][k] + ...; fin ? score = hdiag*e : E = e
template <bool SCORE>
__global__ __launch_bounds__(64) void k_combine(const double *__restrict__ part, int64_t nch,
                                                int64_t K, double *__restrict__ acc,
                                                const double *__restrict__ hdiag,
                                                double *__restrict__ score, int init, int fin) {
    const int64_t k = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (k >= K) return;
    double e = (SCORE && init) ? 0.0 : acc[k];
    int64_t c = 0;
    // loads 16 chunks ahead of the (ordered) additions
    for (; c + 16 <= nch; c += 16) {
        double v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = part[(c + u) * K + k];
#pragma unroll
        for (int u = 0; u < 16; ++u) e = e + v[u];
    }
    for (; c < nch; ++c) e = e + part[c * K + k];
    if (SCORE && fin) score[k] = hdiag[k] * e;
    else acc[k] = e;
}

template <typename T, bool VEC>
hipError_t run_colsum(const T *X, int64_t M, int64_t K, int64_t ldx, bool score_mode,
                      double *result, const double *hdiag, double *ws, hipStream_t st) {
    const int64_t nch = ceil_div(M, kChunkRows);
    const dim3 block(256);
    const unsigned gx = (unsigned)ceil_div(K, kWgCols);
    if (nch == 0) return hipSuccess;
    if (nch == 1) {
        if (score_mode) hipLaunchKernelGGL((k_colsum<T, VEC, 3>), dim3(gx, 1), block, 0, st, X, M, K, ldx, (int64_t)0, result, hdiag);
        else hipLaunchKernelGGL((k_colsum<T, VEC, 1>), dim3(gx, 1), block, 0, st, X, M, K, ldx, (int64_t)0, result, hdiag);
        return hipGetLastError();
    }
    double *E = ws;                       // score: running column error
    double *part = score_mode ? ws + K : ws;
    for (int64_t c0 = 0; c0 < nch; c0 += kMaxChunksPerLaunch) {
        const int64_t n = nch - c0 < kMaxChunksPerLaunch ? nch - c0 : kMaxChunksPerLaunch;
        if (score_mode) hipLaunchKernelGGL((k_colsum<T, VEC, 2>), dim3(gx, (unsigned)n), block, 0, st, X, M, K, ldx, c0, part, hdiag);
        else hipLaunchKernelGGL((k_colsum<T, VEC, 0>), dim3(gx, (unsigned)n), block, 0, st, X, M, K, ldx, c0, part, hdiag);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const unsigned gk = (unsigned)ceil_div(K, 64);
        const int init = c0 == 0, fin = c0 + n >= nch;
        if (score_mode) hipLaunchKernelGGL((k_combine<true>), dim3(gk), dim3(64), 0, st, part, n, K, E, hdiag, result, init, fin);
        else hipLaunchKernelGGL((k_combine<false>), dim3(gk), dim3(64), 0, st, part, n, K, result, hdiag, result, init, fin);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t dispatch_colsum(const void *X, int64_t M, int64_t K, int64_t ldx, bool score_mode,
                           double *result, const double *hdiag, double *ws, hipStream_t st) {
    const T *x = static_cast<const T *>(X);
    const bool vec = (reinterpret_cast<uintptr_t>(X) % 16 == 0) && ((ldx * (int64_t)sizeof(T)) % 16 == 0);
    if (vec) return run_colsum<T, true>(x, M, K, ldx, score_mode, result, hdiag, ws, st);
    return run_colsum<T, false>(x, M, K, ldx, score_mode, result, hdiag, ws, st);
}

}  // namespace

hipError_t launch_calibrate(const void *X, mxs_dtype dt, int64_t M, int64_t K, int64_t ldx,
                            double *hdiag, double *ws, hipStream_t st) {
    if (dt == MXS_BF16) return dispatch_colsum<uint16_t>(X, M, K, ldx, false, hdiag, nullptr, ws, st);
    return dispatch_colsum<float>(X, M, K, ldx, false, hdiag, nullptr, ws, st);
}

hipError_t launch_score(const void *W, mxs_dtype dt, int64_t N, int64_t K, int64_t ldw,
                        const double *hdiag, double *score, double *ws, hipStream_t st) {
    if (dt == MXS_BF16) return dispatch_colsum<uint16_t>(W, N, K, ldw, true, score, hdiag, ws, st);
    return dispatch_colsum<float>(W, N, K, ldw, true, score, hdiag, ws, st);
}

}  // namespace mxs
