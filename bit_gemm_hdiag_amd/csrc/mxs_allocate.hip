// mxs_allocate.hip -- budgeted 8/6/4-bit map and block-uniform permutation.
//
// gist.science/nl "Technische Samenvatting" §2.3: the columns of a layer are
// sorted by sensitivity; the first 32 n8 get 8 bits, the next 32 n6 6 bits,
// the rest 4 bits; the map rides on MXINT's block structure, so the columns
// are regrouped (8-bit ones in ascending index, then 6-bit, then 4-bit) and
// every 32-column block of the new order holds one width.
//
// Rank of column k = #{ j : key_j > key_k or (key_j == key_k and j < k) },
// with key the total order of the fp64 score bit pattern. It is an exact
// integer count, computed by a tiled all-pairs kernel (K <= 131072: at most
// 1.7e10 compares over the whole GPU; 8.2e8 at K = 28672, 1.7e7 at 4096)
// whose partial counts are added with integer atomics (order-independent). The
// perm output buffer holds the ranks until the last kernel overwrites it.
// (A one-workgroup bitonic sort in LDS measured 54 us at K = 4096, against
// 16 us for these three launches.)
#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

constexpr int kRankThreads = 256;
constexpr int kRankPer = 1;        // columns k per thread
constexpr int kRankMaxSlice = 4096;
constexpr int kScanThreads = 1024;
constexpr int64_t kPermLdsMaxK = 32768;   // ranks staged in LDS by the fused class+perm kernel

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *p, int64_t n, int32_t v) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// Workgroup (x, y): columns k in [x * 1024, x * 1024 + 1024) (4 per thread,
// strided by 256) against keys j in slice y; partial counts are added with
// integer atomics, so the result does not depend on the order.
__global__ __launch_bounds__(kRankThreads) void k_rank(const double *__restrict__ score, int64_t K,
                                                       int32_t slice, int32_t *__restrict__ rank) {
    __shared__ uint64_t keys[kRankMaxSlice];
    const int64_t j0 = (int64_t)blockIdx.y * slice;
    const int jn = (int)(K - j0 < slice ? K - j0 : slice);
    for (int t = threadIdx.x; t < jn; t += kRankThreads) keys[t] = order_key(score[j0 + t]);
    __syncthreads();
    const int64_t kbase = (int64_t)blockIdx.x * (kRankThreads * kRankPer) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kRankPer; ++u) {
        const int64_t k = kbase + u * kRankThreads;
        if (k >= K) break;
        const uint64_t kk = order_key(score[k]);
        int32_t cnt = 0;
        if (j0 + jn <= k) {            // every j of the slice precedes k: ties count
            for (int t = 0; t < jn; ++t) cnt += keys[t] >= kk;
        } else if (j0 > k) {           // every j follows k: ties do not count
            for (int t = 0; t < jn; ++t) cnt += keys[t] > kk;
        } else {
            for (int t = 0; t < jn; ++t) cnt += (keys[t] > kk) || (keys[t] == kk && j0 + t < k);
        }
            if (cnt) atomicAdd(rank + k, cnt);
    }
}

__global__ __launch_bounds__(256) void k_class(const int32_t *__restrict__ rank, int64_t K,
                                               int32_t c8, int32_t c6, uint8_t *__restrict__ bits) {
    int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    const int32_t r = rank[k];
    bits[k] = (uint8_t)(r < c8 ? 8 : (r < c8 + c6 ? 6 : 4));
}

// One workgroup: stable partition of 0..K-1 by class 8, 6, 4.
__global__ __launch_bounds__(kScanThreads) void k_perm(const uint8_t *__restrict__ bits, int64_t K,
                                                       int32_t base6, int32_t base4,
                                                       int32_t *__restrict__ perm) {
    __shared__ int32_t cnt[3][kScanThreads];
    const int t = threadIdx.x;
    const int64_t per = (K + kScanThreads - 1) / kScanThreads;
    const int64_t k0 = t * per;
    const int64_t k1 = k0 + per < K ? k0 + per : K;
    int32_t c[3] = {0, 0, 0};
    for (int64_t k = k0; k < k1; ++k) {
        const uint8_t b = bits[k];
        c[b == 8 ? 0 : (b == 6 ? 1 : 2)]++;
    }
    for (int i = 0; i < 3; ++i) cnt[i][t] = c[i];
    __syncthreads();
    // inclusive Hillis-Steele scan of the three counters
    for (int off = 1; off < kScanThreads; off <<= 1) {
        int32_t v[3];
        for (int i = 0; i < 3; ++i) v[i] = t >= off ? cnt[i][t - off] : 0;
        __syncthreads();
        for (int i = 0; i < 3; ++i) cnt[i][t] += v[i];
        __syncthreads();
    }
    int32_t pos[3];
    pos[0] = cnt[0][t] - c[0];
    pos[1] = base6 + cnt[1][t] - c[1];
    pos[2] = base4 + cnt[2][t] - c[2];
    for (int64_t k = k0; k < k1; ++k) {
        const uint8_t b = bits[k];
        const int i = b == 8 ? 0 : (b == 6 ? 1 : 2);
        const int32_t at = pos[i]++;
        if (at < K) perm[at] = (int32_t)k;   // always true when ranks are a permutation
    }
}

// One workgroup, K <= kPermLdsMaxK: ranks (held in the perm buffer) are read
// into LDS, turned into the bit map, and the stable partition 8 -> 6 -> 4
// overwrites the perm buffer.
__global__ __launch_bounds__(kScanThreads) void k_class_perm(int32_t *__restrict__ perm, int64_t K, int32_t c8,
                                                             int32_t c6, uint8_t *__restrict__ bits) {
    extern __shared__ int32_t s_rank[];
    __shared__ int32_t cnt[3][kScanThreads];
    const int t = threadIdx.x;
    for (int64_t k = t; k < K; k += kScanThreads) s_rank[k] = perm[k];
    __syncthreads();
    const int64_t per = (K + kScanThreads - 1) / kScanThreads;
    const int64_t k0 = t * per;
    const int64_t k1 = k0 + per < K ? k0 + per : K;
    int32_t c[3] = {0, 0, 0};
    for (int64_t k = k0; k < k1; ++k) {
        const int32_t r = s_rank[k];
        const int i = r < c8 ? 0 : (r < c8 + c6 ? 1 : 2);
        bits[k] = (uint8_t)(i == 0 ? 8 : (i == 1 ? 6 : 4));
        c[i]++;
    }
    for (int i = 0; i < 3; ++i) cnt[i][t] = c[i];
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        int32_t v[3];
        for (int i = 0; i < 3; ++i) v[i] = t >= off ? cnt[i][t - off] : 0;
        __syncthreads();
        for (int i = 0; i < 3; ++i) cnt[i][t] += v[i];
        __syncthreads();
    }
    int32_t pos[3];
    pos[0] = cnt[0][t] - c[0];
    pos[1] = c8 + cnt[1][t] - c[1];
    pos[2] = c8 + c6 + cnt[2][t] - c[2];
    for (int64_t k = k0; k < k1; ++k) {
        const int32_t r = s_rank[k];
        const int i = r < c8 ? 0 : (r < c8 + c6 ? 1 : 2);
        const int32_t at = pos[i]++;
        if (at < K) perm[at] = (int32_t)k;   // always true when ranks are a permutation
    }
}

}  // namespace

hipError_t launch_allocate(const double *score, int64_t K, int32_t c8, int32_t c6,
                           uint8_t *bits, int32_t *perm, hipStream_t st) {
    const unsigned gk = (unsigned)ceil_div(K, 256);
    hipLaunchKernelGGL(k_fill_i32, dim3(gk), dim3(256), 0, st, perm, K, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // slices small enough for ~1000+ workgroups, large enough to bound the atomics
    const int64_t colblocks = ceil_div(K, kRankThreads * kRankPer);
    int64_t slice = K * colblocks / 1024;
    slice = slice < 64 ? 64 : (slice > kRankMaxSlice ? kRankMaxSlice : slice);
    hipLaunchKernelGGL(k_rank, dim3((unsigned)colblocks, (unsigned)ceil_div(K, slice)), dim3(kRankThreads), 0, st,
                       score, K, (int32_t)slice, perm);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (K <= kPermLdsMaxK) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_class_perm),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kPermLdsMaxK * 4));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_class_perm, dim3(1), dim3(kScanThreads), (size_t)(K * 4), st, perm, K, c8, c6, bits);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_class, dim3(gk), dim3(256), 0, st, perm, K, c8, c6, bits);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_perm, dim3(1), dim3(kScanThreads), 0, st, bits, K, c8, c8 + c6, perm);
    return hipGetLastError();
}

}  // namespace mxs
