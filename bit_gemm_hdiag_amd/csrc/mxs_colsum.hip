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
//   ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)); score: chunk totals added in chunk
//   order; calibrate: runs of 16 chunks, a run total adding its chunk totals
//   in order from the first, run totals added in run order.
//
// Mapping: a wavefront is 8 row groups x 8 lanes; lane (g, c) owns CPL
// consecutive columns (one load per row) and the partial sum p_g of its
// chunk, so each wave streams 8 rows x 8 CPL columns per step and the 4 waves
// of a workgroup cover 32 CPL adjacent columns. The tree is three cross-lane
// xor steps (8, 16, 32). Chunk totals go to a workspace and a second kernel
// adds them in order; a single chunk is written directly. Large calibrations
// give each workgroup a whole run of 16 chunks instead: it adds the run's
// chunk totals in registers and writes one run total, so the workspace
// traffic, whose write-back into a 4 GB read stream cost more than its share
// of the bytes, falls 16-fold (measured 5.71 -> 6.50 TB/s at 262144 x 8192,
// 5.80 -> 6.68 at 262144 x 28672). Smaller ones (fewer than 512 such
// workgroups) keep one chunk per workgroup and let the second kernel form
// the runs: the same order, the same bits.
// CPL = 8 (16-byte bf16 loads): in the score kernel the 4 lanes of a quad
// hold one 32-column MXINT4 block of a row, so the block maximum is two DPP
// steps. (CPL = 4, with twice the waves and an 8-lane block maximum, measured
// slower for the score at 4096 x 4096.)
#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

constexpr int kCpl = 8;   // columns per lane

template <typename T, bool VEC, int CPL>
__device__ __forceinline__ void load_cols(const T *p, float v[CPL]) {
    if constexpr (CPL == 8) {
        load8<T, VEC>(p, v);
    } else if constexpr (VEC && sizeof(T) == 2) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        v[0] = __uint_as_float(u[0] << 16); v[1] = __uint_as_float(u[0] & 0xFFFF0000u);
        v[2] = __uint_as_float(u[1] << 16); v[3] = __uint_as_float(u[1] & 0xFFFF0000u);
    } else if constexpr (VEC) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) v[i] = load1<T>(p + i);
    }
}

// Max over the 8 lanes 8j .. 8j+7 (xor 1 and 2 by DPP quad permutes, xor 4
// by a swizzle).
__device__ __forceinline__ uint32_t oct_max_u32(uint32_t x) {
    x = quad_max_u32(x);
    const uint32_t y = (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (4 << 10) | 0x1F);
    return x > y ? x : y;
}

// Residual of CPL values of one row under uniform MXINT4 (the lanes of the
// block hold the rest of it), squared into the fp64 partial sums.
// d = v - c * 2^s is exact in fp32 (fma with a power of two whose result is
// representable), its square exact in fp64.
// With 8 values per lane the code stays a float: fma(v, 2^-s, 1.5 * 2^23)
// rounds v / 2^s to nearest even in the low mantissa bits, a median against
// 1.5 * 2^23 -+ 7 clamps it and subtracting 1.5 * 2^23 gives c exactly (the
// rule of the packing quantizer); a non-finite block's residual is NaN.
template <int CPL>
__device__ __forceinline__ void acc_residual_sq(const float v[CPL], double acc[CPL]) {
    if constexpr (CPL == 8) {
        uint32_t a = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
            a = a > b ? a : b;
        }
        const BlockScale bs = block_scale(quad_max_u32(a), 4);
        const float magic = 12582912.0f, cm = cmax_of(4);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(v[i], bs.inv, magic), magic - cm, magic + cm);
            float d = __builtin_fmaf(-(t - magic), bs.scale, v[i]);
            d = bs.bad ? __builtin_nanf("") : d;
            const double dd = (double)d;
            acc[i] = __builtin_fma(dd, dd, acc[i]);
        }
        return;
    }
    int c[CPL];
    BlockScale bs;
    {
        uint32_t a = 0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
            a = a > b ? a : b;
        }
        bs = block_scale(oct_max_u32(a), 4);
        const float cm = cmax_of(4);
#pragma unroll
        for (int i = 0; i < CPL; ++i) c[i] = bs.bad ? 0 : (int)code_of(v[i], bs.inv, cm);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        float d = __builtin_fmaf(-(float)c[i], bs.scale, v[i]);
        d = bs.bad ? __builtin_nanf("") : d;
        const double dd = (double)d;
        acc[i] = __builtin_fma(dd, dd, acc[i]);
    }
}

template <int CPL>
__device__ __forceinline__ void acc_sq(const float v[CPL], double acc[CPL]) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const double x = (double)v[i];
        acc[i] = __builtin_fma(x, x, acc[i]);
    }
}

// MODE 0: calibrate, write chunk totals to part[chunk][K]
// MODE 1: calibrate, single chunk: hdiag[k] += total
// MODE 2: score, write chunk totals to part[chunk][K]
// MODE 3: score, single chunk: score[k] = hdiag[k] * total
// MODE 4: calibrate, one run of kRunChunks chunks per workgroup: write run
//         totals to part[run][K]
template <typename T, bool VEC, int MODE, int CPL>
__global__ __launch_bounds__(256) void k_colsum(const T *__restrict__ X, int64_t M, int64_t K,
                                                int64_t ldx, int64_t chunk0,
                                                double *__restrict__ out,
                                                const double *__restrict__ hdiag) {
    constexpr bool kScore = MODE == 2 || MODE == 3;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 3;
    // Workgroup order by XCD: workgroups are dealt to the eight XCDs in
    // turn, so workgroup w (in launch order) works as v = (w mod 8) G / 8 +
    // w / 8; each XCD then streams a contiguous run of whole chunks (all
    // column groups of a chunk's rows) instead of every eighth 512-byte strip
    // of every row. Measured 7 % faster at 262144 x 8192 (4 % at x 28672).
    int64_t bx = blockIdx.x, by = blockIdx.y;
    {
        const int64_t gx = gridDim.x, G = gx * (int64_t)gridDim.y;
        if (G % 8 == 0) {
            const int64_t w = by * gx + bx;
            const int64_t v = (w & 7) * (G >> 3) + (w >> 3);
            bx = v % gx;
            by = v / gx;
        }
    }
    const int64_t col0 = bx * (32 * CPL) + wave * (8 * CPL) + (lane & 7) * CPL;
    constexpr int kChunks = MODE == 4 ? (int)kRunChunks : 1;
    double tot[CPL];   // chunk total, or the run total so far
#pragma unroll
    for (int i = 0; i < CPL; ++i) tot[i] = 0.0;
    for (int cc = 0; cc < kChunks; ++cc) {
    const int64_t r0 = (chunk0 + by * kChunks + cc) * kChunkRows;
    if (r0 >= M) break;   // a short last run (its first chunk always has rows)
    const int64_t r1 = r0 + kChunkRows < M ? r0 + kChunkRows : M;

    double acc[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) acc[i] = 0.0;

    // K % 32 == 0: the lanes of one block are either all in or all out
    // (their shuffles stay inside the wave's active block lanes)
    if (col0 < K) {
        const T *p = X + col0;
        int64_t r = r0 + g;
        if constexpr (kScore && VEC && sizeof(T) == 2 && CPL == 8) {
            // score: the eight rows' raw 16-byte words are all requested
            // before the first is unpacked (the scheduler otherwise
            // interleaves loads with the rounding arithmetic and keeps about
            // half of them in flight); measured 9-28 % faster, bit-identical
            for (; r + 56 < r1; r += 64) {
                u32x4 d[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p + (r + 8 * u) * ldx));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    float v[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] = __uint_as_float(d[u][i] << 16);
                        v[2 * i + 1] = __uint_as_float(d[u][i] & 0xFFFF0000u);
                    }
                    acc_residual_sq<CPL>(v, acc);
                }
            }
        }
        // eight rows of the lane's chain in flight, consumed in row order
        for (; r + 56 < r1; r += 64) {
            float v[8][CPL];
#pragma unroll
            for (int u = 0; u < 8; ++u) load_cols<T, VEC, CPL>(p + (r + 8 * u) * ldx, v[u]);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (kScore) acc_residual_sq<CPL>(v[u], acc);
                else acc_sq<CPL>(v[u], acc);
            }
        }
        for (; r < r1; r += 8) {
            float v0[CPL];
            load_cols<T, VEC, CPL>(p + r * ldx, v0);
            if (kScore) acc_residual_sq<CPL>(v0, acc);
            else acc_sq<CPL>(v0, acc);
        }
    }

    // ((p0+p1)+(p2+p3)) + ((p4+p5)+(p6+p7)) across the row groups; a run
    // adds its chunk totals in chunk order, starting from the first
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        double x = acc[i];
        x = x + __shfl_xor(x, 8);
        x = x + __shfl_xor(x, 16);
        x = x + __shfl_xor(x, 32);
        tot[i] = cc == 0 ? x : tot[i] + x;
    }
    }
    if (g != 0 || col0 >= K) return;

    if (MODE == 0 || MODE == 2 || MODE == 4) {
        double *dst = out + by * K + col0;
#pragma unroll
        for (int i = 0; i < CPL; i += 2) *reinterpret_cast<double2 *>(dst + i) = make_double2(tot[i], tot[i + 1]);
    } else if (MODE == 1) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) out[col0 + i] = out[col0 + i] + tot[i];
    } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) out[col0 + i] = hdiag[col0 + i] * (0.0 + tot[i]);
    }
}

// Ordered combination of the workspace totals.
// score: e = (init ? 0 : E[k]) + part[0][k] + ...; fin ? score = hdiag*e : E = e
// calibrate (RUN = 1, run totals): acc[k] += part[0][k]; acc[k] += part[1][k]; ...
// calibrate (RUN = kRunChunks, chunk totals): each run of RUN consecutive
//   totals (the last may be short) is added in order from its first, then
//   acc[k] += run total, run by run.
// One thread per column; its loads run up to 32 totals ahead of the
// (ordered) additions. (Deeper batches, 64 or 128, and staging 256 totals x
// 32 columns per workgroup in LDS were measured no faster.)
constexpr int kCmbAhead = 32;
static_assert(kCmbAhead % kRunChunks == 0, "a batch of loads holds whole runs");
template <bool SCORE, int RUN>
__global__ __launch_bounds__(64) void k_combine(const double *__restrict__ part, int64_t nch,
                                                 int64_t K, double *__restrict__ acc,
                                                 const double *__restrict__ hdiag,
                                                 double *__restrict__ score, int init, int fin) {
    const int64_t k = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (k >= K) return;
    double e = (SCORE && init) ? 0.0 : acc[k];
    for (int64_t c = 0; c < nch; c += kCmbAhead) {
        double v[kCmbAhead];
#pragma unroll
        for (int u = 0; u < kCmbAhead; ++u)
            if (c + u < nch) v[u] = part[(c + u) * K + k];
        if constexpr (RUN == 1) {
#pragma unroll
            for (int u = 0; u < kCmbAhead; ++u)
                if (c + u < nch) e = e + v[u];
        } else {
            double r = 0.0;
#pragma unroll
            for (int u = 0; u < kCmbAhead; ++u)
                if (c + u < nch) {
                    r = u % RUN == 0 ? v[u] : r + v[u];
                    if (u % RUN == RUN - 1 || c + u == nch - 1) e = e + r;
                }
        }
    }
    if (SCORE && fin) score[k] = hdiag[k] * e;
    else acc[k] = e;
}

// Calibrations with at least this many (run, column group) workgroups take
// one run per workgroup (measured faster from 512 up: 65536 x 8192, 512 of
// them, 5.64 -> 6.19 TB/s; 16384 x 4096, 64 of them, 4.75 -> 1.12)
constexpr int64_t kRunPathMinWgs = 512;

template <typename T, bool VEC, int CPL>
hipError_t run_colsum(const T *X, int64_t M, int64_t K, int64_t ldx, bool score_mode,
                      double *result, const double *hdiag, double *ws, hipStream_t st) {
    const int64_t nch = ceil_div(M, kChunkRows);
    const dim3 block(256);
    const unsigned gx = (unsigned)ceil_div(K, 32 * CPL);
    if (nch == 0) return hipSuccess;
    if (nch == 1) {
        if (score_mode) hipLaunchKernelGGL((k_colsum<T, VEC, 3, CPL>), dim3(gx, 1), block, 0, st, X, M, K, ldx, (int64_t)0, result, hdiag);
        else hipLaunchKernelGGL((k_colsum<T, VEC, 1, CPL>), dim3(gx, 1), block, 0, st, X, M, K, ldx, (int64_t)0, result, hdiag);
        return hipGetLastError();
    }
    double *E = ws;                       // score: running column error
    double *part = score_mode ? ws + K : ws;
    // launches cover whole runs (kMaxChunksPerLaunch is a multiple of kRunChunks)
    for (int64_t c0 = 0; c0 < nch; c0 += kMaxChunksPerLaunch) {
        const int64_t n = nch - c0 < kMaxChunksPerLaunch ? nch - c0 : kMaxChunksPerLaunch;
        const int64_t runs = ceil_div(n, kRunChunks);
        const unsigned gk = (unsigned)ceil_div(K, 64);
        const int init = c0 == 0, fin = c0 + n >= nch;
        const bool by_run = !score_mode && runs * (int64_t)gx >= kRunPathMinWgs;
        if (score_mode) hipLaunchKernelGGL((k_colsum<T, VEC, 2, CPL>), dim3(gx, (unsigned)n), block, 0, st, X, M, K, ldx, c0, part, hdiag);
        else if (by_run) hipLaunchKernelGGL((k_colsum<T, VEC, 4, CPL>), dim3(gx, (unsigned)runs), block, 0, st, X, M, K, ldx, c0, part, hdiag);
        else hipLaunchKernelGGL((k_colsum<T, VEC, 0, CPL>), dim3(gx, (unsigned)n), block, 0, st, X, M, K, ldx, c0, part, hdiag);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (score_mode) hipLaunchKernelGGL((k_combine<true, 1>), dim3(gk), dim3(64), 0, st, part, n, K, E, hdiag, result, init, fin);
        else if (by_run) hipLaunchKernelGGL((k_combine<false, 1>), dim3(gk), dim3(64), 0, st, part, runs, K, result, hdiag, result, init, fin);
        else hipLaunchKernelGGL((k_combine<false, (int)kRunChunks>), dim3(gk), dim3(64), 0, st, part, n, K, result, hdiag, result, init, fin);
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
    if (vec) return run_colsum<T, true, kCpl>(x, M, K, ldx, score_mode, result, hdiag, ws, st);
    return run_colsum<T, false, kCpl>(x, M, K, ldx, score_mode, result, hdiag, ws, st);
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
