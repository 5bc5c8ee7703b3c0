// mxs_quantize.hip -- MXINT 4/6/8-bit block quantisation with the
// block-uniform channel permutation, packed into per-width planes.
//
// gist.science/nl "Technische Samenvatting" §1 (one shared power-of-two
// scale per 32 values), §2.2 (4/6/8-bit mantissas), §2.3 (blocks of one
// width after regrouping the channels); researchpod.app bullet "Triplet
// Quantization" (weights and activations). Per permuted block b with width
// m: s = max(floor(log2 amax) - (m-2), -127), c = clamp(rne(v / 2^s),
// +-(2^(m-1)-1)); E8M0 byte s + 127 (0 for an all-zero block, 0xFF for a block
// with NaN/Inf, whose codes are 0).
//
// Each lane quantises 8 consecutive positions (a quarter block); the block
// maximum is a DPP reduction over the aligned quad. Two kernels:
//  - direct (no permutation): flat grid over (row, 8-column group), 16-byte
//    coalesced loads; also serves KV quantisation (rows = tokens x heads).
//  - gather (with permutation): each lane keeps its 8 source indices in
//    registers and walks a slice of rows, so the permutation is read once
//    per workgroup; the source reads hit L1/L2 lines of the row being read.
#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

struct Planes {
    int64_t K;
    int32_t n8, n6, n4;
    int8_t *q8; int64_t ld8;
    uint8_t *q6; int64_t ld6;
    uint8_t *q4; int64_t ld4;
    uint8_t *sc; int64_t lds;
};

__device__ __forceinline__ void emit(const Planes &P, int64_t row, int64_t blk, int q, const float v[8]) {
    const int m = blk < P.n8 ? 8 : (blk < (int64_t)P.n8 + P.n6 ? 6 : 4);
    uint32_t byte;
    const uint64_t w = quantize_pack8(v, m, byte);
    if (m == 8) {
        store_bytes(reinterpret_cast<uint8_t *>(P.q8) + row * P.ld8 + 32 * blk + 8 * q, w, 8);
    } else if (m == 6) {
        store_bytes(P.q6 + row * P.ld6 + 24 * (blk - P.n8) + 6 * q, w, 6);
    } else {
        store_bytes(P.q4 + row * P.ld4 + 16 * (blk - P.n8 - P.n6) + 4 * q, w, 4);
    }
    if (q == 0) P.sc[row * P.lds + blk] = (uint8_t)byte;
}

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_quant_direct(const T *__restrict__ X, int64_t R, int64_t ldx,
                                                      Planes P) {
    const int64_t G = P.K / 8;                     // 8-column groups per row
    const int64_t total = R * G;
    for (int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x; gid < total;
         gid += (int64_t)gridDim.x * 256) {
        const int64_t row = gid / G;
        const int64_t cg = gid - row * G;
        float v[8];
        load8<T, VEC>(X + row * ldx + cg * 8, v);
        emit(P, row, cg >> 2, (int)(cg & 3), v);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void k_quant_gather(const T *__restrict__ X, int64_t R, int64_t ldx,
                                                      const int32_t *__restrict__ perm,
                                                      int64_t rows_per_block, Planes P) {
    const int64_t cg = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8-position group
    if (cg * 8 >= P.K) return;                                       // whole quads leave together
    int32_t src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // an index outside [0, K) is clamped, never dereferenced
        const uint32_t j = (uint32_t)perm[cg * 8 + i];
        src[i] = (int32_t)(j < (uint32_t)P.K ? j : (uint32_t)P.K - 1u);
    }
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < R ? r0 + rows_per_block : R;
    for (int64_t row = r0; row < r1; ++row) {
        const T *x = X + row * ldx;
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = load1<T>(x + src[i]);
        emit(P, row, cg >> 2, (int)(cg & 3), v);
    }
}

// LDS-staged gather: the permutation (as 16-bit indices, stage_perm) is
// staged once per workgroup, then each row is read with coalesced 16-byte
// loads into LDS and gathered from there. Used when the permutation and one
// row fit in kStageLds.
template <typename T>
__global__ __launch_bounds__(256) void k_quant_gather_lds(const T *__restrict__ X, int64_t R, int64_t ldx,
                                                          const int32_t *__restrict__ perm, Planes P) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int64_t K = P.K;
    uint16_t *sperm = reinterpret_cast<uint16_t *>(lds);
    T *srow = reinterpret_cast<T *>(lds + ((2 * K + 15) / 16) * 16);
    const int tid = threadIdx.x;
    stage_perm(perm, K, sperm, tid);
    const int64_t nvec = K * (int64_t)sizeof(T) / 16;          // 16-byte pieces per row
    const bool vec = reinterpret_cast<uintptr_t>(X) % 16 == 0 && (ldx * (int64_t)sizeof(T)) % 16 == 0;
    for (int64_t row = blockIdx.x; row < R; row += gridDim.x) {
        __syncthreads();                       // previous row's gathers are done
        const T *x = X + row * ldx;
        if (vec) {
            for (int64_t v = tid; v < nvec; v += 256)
                reinterpret_cast<uint4 *>(srow)[v] = reinterpret_cast<const uint4 *>(x)[v];
        } else {
            for (int64_t j = tid; j < K; j += 256) srow[j] = x[j];
        }
        __syncthreads();
        for (int64_t cg = tid; cg * 8 < K; cg += 256) {   // whole quads stay together
            const uint4 pi = *reinterpret_cast<const uint4 *>(sperm + cg * 8);
            const uint32_t w[4] = {pi.x, pi.y, pi.z, pi.w};
            float v[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                v[2 * i] = load1<T>(srow + (w[i] & 0xFFFFu));
                v[2 * i + 1] = load1<T>(srow + (w[i] >> 16));
            }
            emit(P, row, cg >> 2, (int)(cg & 3), v);
        }
    }
}

// The same LDS-staged gather with rows streamed ahead: each thread holds
// its PPT 16-byte pieces of the next DEPTH rows in a register ring, so a
// row's HBM latency overlaps the gathers and stores of the rows before it.
// Requires 16-byte aligned rows. PG: the permutation is read from global
// memory (L2) per group instead of being staged in LDS, so that long rows
// (only the row in LDS) still fit two workgroups per CU; requires a 16-byte
// aligned permutation.
template <typename T, int PPT, int DEPTH, bool PG>
__global__ __launch_bounds__(256) void k_quant_gather_pf(const T *__restrict__ X, int64_t R, int64_t ldx,
                                                         const int32_t *__restrict__ perm, Planes P) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int64_t K = P.K;
    uint16_t *sperm = reinterpret_cast<uint16_t *>(lds);
    u32x4 *srow = reinterpret_cast<u32x4 *>(lds + (PG ? 0 : ((2 * K + 15) / 16) * 16));
    const int tid = threadIdx.x;
    if (!PG) stage_perm(perm, K, sperm, tid);
    const int nvec = (int)(K * (int64_t)sizeof(T) / 16);
    const int64_t G = gridDim.x;
    u32x4 ring[DEPTH][PPT];
    auto fetch = [&](u32x4 (&r)[PPT], int64_t row) {
        const u32x4 *x = reinterpret_cast<const u32x4 *>(X + row * ldx);
#pragma unroll
        for (int i = 0; i < PPT; ++i)
            if (tid + 256 * i < nvec) r[i] = __builtin_nontemporal_load(x + tid + 256 * i);
    };
    const T *s = reinterpret_cast<const T *>(srow);
    int64_t row = blockIdx.x;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
        if (row + d * G < R) fetch(ring[d], row + d * G);
    while (true) {
#pragma unroll
        for (int d = 0; d < DEPTH; ++d) {
            if (row >= R) return;
            lds_barrier();                              // the previous row's gathers are done
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                if (tid + 256 * i < nvec) srow[tid + 256 * i] = ring[d][i];
            lds_barrier();
            if (row + DEPTH * G < R) fetch(ring[d], row + DEPTH * G);
            if constexpr (PG) {
                // the permutation entries of a group are loaded two groups
                // ahead of its gather (an L2 round trip per group otherwise)
                const uint32_t kmax = (uint32_t)K - 1u;
                uint4 pa[2], pb[2];
                auto pload = [&](int k, int64_t c) {
                    if (c * 8 < K) {
                        pa[k] = reinterpret_cast<const uint4 *>(perm + c * 8)[0];
                        pb[k] = reinterpret_cast<const uint4 *>(perm + c * 8)[1];
                    }
                };
                auto gather = [&](int k, int64_t c) {   // whole quads stay together
                    const uint32_t j[8] = {pa[k].x, pa[k].y, pa[k].z, pa[k].w, pb[k].x, pb[k].y, pb[k].z, pb[k].w};
                    float v[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[i] = load1<T>(s + (j[i] < kmax ? j[i] : kmax));
                    emit(P, row, c >> 2, (int)(c & 3), v);
                };
                int64_t cg = tid;
                pload(0, cg);
                pload(1, cg + 256);
                while (cg * 8 < K) {
                    gather(0, cg);
                    pload(0, cg + 512);
                    cg += 256;
                    if (cg * 8 >= K) break;
                    gather(1, cg);
                    pload(1, cg + 512);
                    cg += 256;
                }
            } else {
                for (int64_t cg = tid; cg * 8 < K; cg += 256) {   // whole quads stay together
                    const uint4 pi = *reinterpret_cast<const uint4 *>(sperm + cg * 8);
                    const uint32_t w[4] = {pi.x, pi.y, pi.z, pi.w};
                    float v[8];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[2 * i] = load1<T>(s + (w[i] & 0xFFFFu));
                        v[2 * i + 1] = load1<T>(s + (w[i] >> 16));
                    }
                    emit(P, row, cg >> 2, (int)(cg & 3), v);
                }
            }
            row += G;
        }
    }
}

// Rows up to kStageLdsLong bytes of LDS (permutation + row) still stream
// through the register ring: one workgroup per CU for the longest rows (the
// 28672-column down-projection input in bf16 needs 112 KiB), rather than
// gathering every element from global memory.
constexpr int64_t kStageLdsLong = 144 * 1024;

template <typename T, int PPT, bool PG>
hipError_t launch_gather_pf(const T *X, int64_t ldx, const int32_t *perm, const Planes &P, int64_t R,
                            int64_t lds_bytes, hipStream_t st) {
    // The gathers, quantisation and packing of a row are the larger cost, so
    // occupancy wins over depth: as many workgroups as LDS allows (up to 8 per
    // CU), each streaming its rows two ahead. (512 workgroups four rows deep
    // measured 24 % slower for 4096 x 4096.)
    constexpr int DEPTH = 2;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_quant_gather_pf<T, PPT, DEPTH, PG>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStageLdsLong);
    if (e != hipSuccess) return e;
    const int64_t per_cu = (160 * 1024) / lds_bytes;
    int64_t blocks = 256 * (per_cu < 8 ? (per_cu < 1 ? 1 : per_cu) : 8);
    blocks = blocks < R ? blocks : R;
    hipLaunchKernelGGL((k_quant_gather_pf<T, PPT, DEPTH, PG>), dim3((unsigned)blocks), dim3(256), (size_t)lds_bytes, st,
                       X, R, ldx, perm, P);
    return hipGetLastError();
}

template <typename T>
hipError_t run_quantize(const T *X, int64_t ldx, const int32_t *perm, const Planes &P, int64_t R,
                        hipStream_t st) {
    if (R == 0) return hipSuccess;
    if (!perm) {
        const int64_t total = R * (P.K / 8);
        int64_t blocks = ceil_div(total, 256);
        if (blocks > 65536) blocks = 65536;
        const bool vec = reinterpret_cast<uintptr_t>(X) % 16 == 0 && (ldx * (int64_t)sizeof(T)) % 16 == 0;
        if (vec) hipLaunchKernelGGL((k_quant_direct<T, true>), dim3((unsigned)blocks), dim3(256), 0, st, X, R, ldx, P);
        else hipLaunchKernelGGL((k_quant_direct<T, false>), dim3((unsigned)blocks), dim3(256), 0, st, X, R, ldx, P);
        return hipGetLastError();
    }
    const int64_t lds_bytes = ((2 * P.K + 15) / 16) * 16 + P.K * (int64_t)sizeof(T);
    const bool vec = reinterpret_cast<uintptr_t>(X) % 16 == 0 && (ldx * (int64_t)sizeof(T)) % 16 == 0;
    const int64_t ppt = ceil_div(P.K * (int64_t)sizeof(T) / 16, 256);
    // rows so long that the permutation and the row leave room for one
    // workgroup per CU: the permutation is read from L2 instead, and the
    // row alone fits two
    const int64_t row_bytes = P.K * (int64_t)sizeof(T);
    if (vec && P.K <= 65536 && ppt <= 16 && 2 * lds_bytes > 160 * 1024 && 2 * row_bytes <= 160 * 1024 &&
        reinterpret_cast<uintptr_t>(perm) % 16 == 0) {
        if (ppt <= 8) return launch_gather_pf<T, 8, true>(X, ldx, perm, P, R, row_bytes, st);
        return launch_gather_pf<T, 16, true>(X, ldx, perm, P, R, row_bytes, st);
    }
    if (vec && lds_bytes <= kStageLdsLong && P.K <= 65536 && ppt <= 16) {
        if (ppt <= 1) return launch_gather_pf<T, 1, false>(X, ldx, perm, P, R, lds_bytes, st);
        if (ppt <= 2) return launch_gather_pf<T, 2, false>(X, ldx, perm, P, R, lds_bytes, st);
        if (ppt <= 4) return launch_gather_pf<T, 4, false>(X, ldx, perm, P, R, lds_bytes, st);
        if (ppt <= 8) return launch_gather_pf<T, 8, false>(X, ldx, perm, P, R, lds_bytes, st);
        return launch_gather_pf<T, 16, false>(X, ldx, perm, P, R, lds_bytes, st);
    }
    if (lds_bytes <= kStageLds && P.K <= 65536) {
        int64_t blocks = R < 512 ? R : 512;   // each workgroup stages the permutation once
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_quant_gather_lds<T>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStageLds);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((k_quant_gather_lds<T>), dim3((unsigned)blocks), dim3(256), (size_t)lds_bytes, st, X, R,
                           ldx, perm, P);
        return hipGetLastError();
    }
    const int64_t gx = ceil_div(P.K / 8, 256);
    int64_t gy = ceil_div(4096, gx);
    if (gy > R) gy = R;
    if (gy > 65535) gy = 65535;
    const int64_t rpb = ceil_div(R, gy);
    gy = ceil_div(R, rpb);
    hipLaunchKernelGGL((k_quant_gather<T>), dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st, X, R, ldx,
                       perm, rpb, P);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void *X, mxs_dtype dt, int64_t ldx, const int32_t *perm,
                           const mxs_qmat &o, hipStream_t st) {
    Planes P{o.K, o.n8, o.n6, o.n4, o.q8, o.ld8, o.q6, o.ld6, o.q4, o.ld4, o.sc, o.lds};
    if (dt == MXS_BF16) return run_quantize<uint16_t>(static_cast<const uint16_t *>(X), ldx, perm, P, o.rows, st);
    return run_quantize<float>(static_cast<const float *>(X), ldx, perm, P, o.rows, st);
}

}  // namespace mxs
