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
// 11.5 us for these three launches; they take 20 us at K = 8192 and 88 us at
// K = 28672, and about 11 us of launch latency at any K.)
#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

constexpr int kRankThreads = 256;
constexpr int kRankMaxSlice = 4096;
constexpr int kScanThreads = 1024;
constexpr int64_t kPermLdsMaxK = 32768;   // ranks staged in LDS by the fused class+perm kernel

__global__ __launch_bounds__(256) void k_fill_i32(int32_t *p, int64_t n, int32_t v) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// Workgroup (x, y): columns k in [x * 256 PER, (x + 1) * 256 PER) (PER per
// thread, strided by 256) against keys j in slice y, staged in LDS. Each LDS
// read (two keys) serves the thread's PER columns, so with PER = 4 the loop
// issues one LDS instruction per eight comparisons. A slice wholly before or
// after the workgroup's columns decides ties the same way for all of them;
// only a slice that overlaps them compares indices. Partial counts are added
// with integer atomics, so the result does not depend on the order.
template <int kRankPer>
__global__ __launch_bounds__(kRankThreads) void k_rank(const double *__restrict__ score, int64_t K,
                                                       int32_t slice, int32_t *__restrict__ rank) {
    __shared__ __attribute__((aligned(16))) uint64_t keys[kRankMaxSlice];
    const int64_t j0 = (int64_t)blockIdx.y * slice;
    const int jn = (int)(K - j0 < slice ? K - j0 : slice);
    for (int t = threadIdx.x; t < jn; t += kRankThreads) keys[t] = order_key(score[j0 + t]);
    __syncthreads();
    const int64_t kb0 = (int64_t)blockIdx.x * (kRankThreads * kRankPer);
    uint64_t kk[kRankPer];
    int32_t cnt[kRankPer];
#pragma unroll
    for (int u = 0; u < kRankPer; ++u) {
        const int64_t k = kb0 + threadIdx.x + u * kRankThreads;
        kk[u] = k < K ? order_key(score[k]) : 0;
        cnt[u] = 0;
    }
    const int np = jn >> 1;
    if (j0 + jn <= kb0) {                                   // every j precedes every k: ties count
        for (int t = 0; t < np; ++t) {
            const uint64_t a = keys[2 * t], b = keys[2 * t + 1];
#pragma unroll
            for (int u = 0; u < kRankPer; ++u) cnt[u] += (int32_t)(a >= kk[u]) + (int32_t)(b >= kk[u]);
        }
        if (jn & 1) {
#pragma unroll
            for (int u = 0; u < kRankPer; ++u) cnt[u] += keys[jn - 1] >= kk[u];
        }
    } else if (j0 >= kb0 + kRankThreads * kRankPer) {       // every j follows every k: ties do not count
        for (int t = 0; t < np; ++t) {
            const uint64_t a = keys[2 * t], b = keys[2 * t + 1];
#pragma unroll
            for (int u = 0; u < kRankPer; ++u) cnt[u] += (int32_t)(a > kk[u]) + (int32_t)(b > kk[u]);
        }
        if (jn & 1) {
#pragma unroll
            for (int u = 0; u < kRankPer; ++u) cnt[u] += keys[jn - 1] > kk[u];
        }
    } else {
        for (int t = 0; t < jn; ++t) {
            const uint64_t a = keys[t];
#pragma unroll
            for (int u = 0; u < kRankPer; ++u) {
                const int64_t k = kb0 + threadIdx.x + u * kRankThreads;
                cnt[u] += (a > kk[u]) || (a == kk[u] && j0 + t < k);
            }
        }
    }
#pragma unroll
    for (int u = 0; u < kRankPer; ++u) {
        const int64_t k = kb0 + threadIdx.x + u * kRankThreads;
        if (k < K && cnt[u]) atomicAdd(rank + k, cnt[u]);
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
// overwrites the perm buffer. Wave w owns one contiguous segment of columns
// (a multiple of 64). A first walk counts the segment's 8- and 6-bit columns
// with ballots; a column's place is then its class's base, plus the columns
// of that class in the segments before (the wave counts) and in the
// segment before it (running ballot counts and the prefix of the lanes below).
__global__ __launch_bounds__(kScanThreads) void k_class_perm(int32_t *__restrict__ perm, int32_t K, int32_t c8,
                                                             int32_t c6, uint8_t *__restrict__ bits) {
    constexpr int NW = kScanThreads / 64;
    extern __shared__ int32_t s_rank[];
    __shared__ int32_t wcnt[2][NW];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    for (int k = t; k < K; k += kScanThreads) s_rank[k] = perm[k];
    __syncthreads();
    const int seg = (K + NW * 64 - 1) / (NW * 64) * 64;
    const int k0 = w * seg < K ? w * seg : K;
    const int k1 = k0 + seg < K ? k0 + seg : K;
    const int32_t c86 = c8 + c6;
    int32_t n8 = 0, n6 = 0;
    for (int kb = k0; kb < k1; kb += 64) {
        const int k = kb + lane;
        const int32_t r = k < k1 ? s_rank[k] : INT32_MAX;   // past the end: no class
        n8 += __popcll(__ballot(r < c8));
        n6 += __popcll(__ballot(r >= c8 && r < c86));
    }
    if (lane == 0) {
        wcnt[0][w] = n8;
        wcnt[1][w] = n6;
    }
    __syncthreads();
    int32_t p8 = 0, p6 = 0;
    for (int v = 0; v < w; ++v) {
        p8 += wcnt[0][v];
        p6 += wcnt[1][v];
    }
    int32_t p4 = c86 + (k0 - p8 - p6);   // 4-bit columns before the segment
    p6 += c8;
    const uint64_t below = (1ull << lane) - 1ull;
    for (int kb = k0; kb < k1; kb += 64) {
        const int k = kb + lane;
        const bool in = k < k1;
        const int32_t r = in ? s_rank[k] : INT32_MAX;
        const bool is8 = r < c8, is6 = !is8 && r < c86;
        const uint64_t m8 = __ballot(is8), m6 = __ballot(is6), m4 = __ballot(in && !is8 && !is6);
        if (in) {
            const int32_t at = is8 ? p8 + __popcll(m8 & below)
                                   : (is6 ? p6 + __popcll(m6 & below) : p4 + __popcll(m4 & below));
            bits[k] = (uint8_t)(is8 ? 8 : (is6 ? 6 : 4));
            if (at < K) perm[at] = k;   // always true when ranks are a permutation
        }
        p8 += __popcll(m8);
        p6 += __popcll(m6);
        p4 += __popcll(m4);
    }
}

}  // namespace

hipError_t launch_allocate(const double *score, int64_t K, int32_t c8, int32_t c6,
                           uint8_t *bits, int32_t *perm, hipStream_t st) {
    const unsigned gk = (unsigned)ceil_div(K, 256);
    hipLaunchKernelGGL(k_fill_i32, dim3(gk), dim3(256), 0, st, perm, K, 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Up to K = 4096 one column per thread (more threads, the latency of a
    // short launch dominates); above, four per thread and slices sized for
    // ~4096 workgroups (measured at K = 28672: 96 us against 261 us for one
    // column per thread and ~1000 workgroups; the atomics grow with the
    // number of slices, K per slice)
    if (K <= 4096) {
        const int64_t colblocks = ceil_div(K, kRankThreads);
        int64_t slice = K * colblocks / 1024;
        slice = slice < 64 ? 64 : (slice > kRankMaxSlice ? kRankMaxSlice : slice);
        hipLaunchKernelGGL((k_rank<1>), dim3((unsigned)colblocks, (unsigned)ceil_div(K, slice)), dim3(kRankThreads),
                           0, st, score, K, (int32_t)slice, perm);
    } else {
        const int64_t colblocks = ceil_div(K, kRankThreads * 4);
        int64_t slice = K * colblocks / 4096;
        slice = slice < 64 ? 64 : (slice > kRankMaxSlice ? kRankMaxSlice : slice);
        hipLaunchKernelGGL((k_rank<4>), dim3((unsigned)colblocks, (unsigned)ceil_div(K, slice)), dim3(kRankThreads),
                           0, st, score, K, (int32_t)slice, perm);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (K <= kPermLdsMaxK) {
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_class_perm),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)(kPermLdsMaxK * 4));
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_class_perm, dim3(1), dim3(kScanThreads), (size_t)(K * 4), st, perm, (int32_t)K, c8,
                           c6, bits);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_class, dim3(gk), dim3(256), 0, st, perm, K, c8, c6, bits);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_perm, dim3(1), dim3(kScanThreads), 0, st, bits, K, c8, c8 + c6, perm);
    return hipGetLastError();
}

}  // namespace mxs
