// mxs_layerwise.hip -- layer sensitivity and the layer-wise budget.
//
// gist.science/nl "Technische Samenvatting" §2.1 ("Laaggewijze
// sensitiviteit": a layer's sensitivity is the L2 error at the model output
// when that layer alone is quantized) and §2.3 (one 8-bit block of the 32
// most sensitive columns per layer; the number of 6-bit columns of a layer is
// proportional to its sensitivity, scaled by one global parameter R so that
// the average width meets the target B).
//
// Without a trained model the model-output error is replaced by the layer's
// own output error on calibration tokens,
//   S = sum_{t,n} (sum_k X[t,k] W[n,k] - Yq[t,n])^2,
// with Yq the product of the quantized operands (mxs_mixed_gemm). The dense
// product runs on the fp32 matrix cores (v_mfma_f32_32x32x2_f32) over
// 64 x 64 output tiles; each tile's squared differences are summed in fp64 in
// a fixed order and the tile sums are added in tile order, so the result is
// deterministic. This is a calibration-time call, not part of inference.
//
// The budget: every layer gets n8 = 1 and n6 = min(nb - 1, floor(R S + 1/2)),
// with R the largest value whose average width over all weights (rows x K per
// layer, mantissa bits) does not exceed B. The average only changes where
// R S = j - 1/2, so R is found by bisection over those breakpoints: taken in
// ascending order, equal ones together, each accepted while its extra bits
// fit; the first that does not fit ends the search.
#include <algorithm>
#include <cmath>
#include <vector>

#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

constexpr int kET = 64;        // output tile (rows of X and of W)
constexpr int kEK = 32;        // K per stage
constexpr int kEP = kEK + 4;   // LDS row pitch in floats (16-byte aligned, spreads banks)

typedef float v16f_e __attribute__((ext_vector_type(16)));

// eight consecutive elements of a row as fp32 (bf16 widens exactly)
template <typename T>
__device__ __forceinline__ void load8f(const T *p, float v[8]);

template <>
__device__ __forceinline__ void load8f<float>(const float *p, float v[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load8f<uint16_t>(const uint16_t *p, float v[8]) {
    const uint4 q = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

// One workgroup: a 64 x 64 tile of X W^T (four waves, one 32 x 32 MFMA tile
// each), then the tile's sum of (Y - Yq)^2 in fp64 into part[tile].
// Lane l of a wave supplies row l % 32 of each operand; in MFMA step s it
// contributes k = s (lanes 0..31) and k = 16 + s (lanes 32..63) of the stage.
// Rows past M or N load zeros and are left out of the sum.
// The tile's sum of squared differences from its 16 products per lane
// (result register 4 q + r of lane l: row 8 q + 4 h + r, column l % 32).
// All 16 Yq values are requested before any is used (rows and columns past
// the matrix read its last row / column and are left out of the sum).
__device__ __forceinline__ void tile_err(const float (&acc)[16], int64_t M, int64_t N, const float *__restrict__ Yq,
                                         int64_t ldy, double *red, double *__restrict__ part) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5, wm = wave >> 1, wn = wave & 1;
    const int64_t tm = (int64_t)blockIdx.y * kET, tn = (int64_t)blockIdx.x * kET;
    double s = 0.0;
    const int64_t col = tn + 32 * wn + l32, cc = col < N ? col : N - 1;
    float yq[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t row = tm + 32 * wm + 8 * (i >> 2) + 4 * h + (i & 3);
        yq[i] = Yq[(row < M ? row : M - 1) * ldy + cc];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t row = tm + 32 * wm + 8 * (i >> 2) + 4 * h + (i & 3);
        const double d = (double)acc[i] - (double)yq[i];
        s += (row < M && col < N) ? d * d : 0.0;
    }
    red[tid] = s;
    __syncthreads();
    if (tid == 0) {
        double t = 0.0;
        for (int i = 0; i < 256; ++i) t += red[i];
        part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = t;
    }
}

// Grid (tiles of W rows, tiles of X rows, K splits). Split z forms the
// products over k in [z kper, min(K, (z + 1) kper)) (kper a multiple of
// kEK). With one split the workgroup finishes the tile (tile_err); with
// several it stores its 16 partial products per lane to py, tile-major
// ([split][tile][thread][16]), and k_outerr_fin adds the splits in order.
template <typename T>
__global__ __launch_bounds__(256) void k_outerr(const T *__restrict__ X, int64_t M, int64_t ldx,
                                                const T *__restrict__ W, int64_t N, int64_t ldw, int64_t K,
                                                int64_t kper, const float *__restrict__ Yq, int64_t ldy,
                                                float *__restrict__ py, double *__restrict__ part) {
    __shared__ __attribute__((aligned(16))) float sx[kET * kEP];
    __shared__ __attribute__((aligned(16))) float sw[kET * kEP];
    __shared__ double red[256];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, h = lane >> 5, wm = wave >> 1, wn = wave & 1;
    const int64_t tm = (int64_t)blockIdx.y * kET, tn = (int64_t)blockIdx.x * kET;
    const int lr = tid >> 2, lc = (tid & 3) * 8;          // load role: row, first column
    const bool xin = tm + lr < M, win = tn + lr < N;
    const int64_t klo = (int64_t)blockIdx.z * kper;
    const int64_t kn = K - klo < kper ? K - klo : kper;   // may be <= 0 for a trailing split
    const T *xp = X + (xin ? tm + lr : 0) * ldx + klo + lc;
    const T *wp = W + (win ? tn + lr : 0) * ldw + klo + lc;

    float xr[8], wr[8];
    if (kn > 0) {
        load8f<T>(xp, xr);
        load8f<T>(wp, wr);
    }
    v16f_e acc = {};
    for (int64_t k0 = 0; k0 < kn; k0 += kEK) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sx[lr * kEP + lc + i] = xin ? xr[i] : 0.f;
            sw[lr * kEP + lc + i] = win ? wr[i] : 0.f;
        }
        __syncthreads();
        if (k0 + kEK < kn) {
            load8f<T>(xp + k0 + kEK, xr);
            load8f<T>(wp + k0 + kEK, wr);
        }
        const float *ap = sx + (32 * wm + l32) * kEP + 16 * h;
        const float *bp = sw + (32 * wn + l32) * kEP + 16 * h;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 a = reinterpret_cast<const float4 *>(ap)[q], b = reinterpret_cast<const float4 *>(bp)[q];
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
        }
        __syncthreads();
    }

    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = acc[i];
    if (py) {
        const int64_t tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
        float4 *dst = reinterpret_cast<float4 *>(
            py + (((int64_t)blockIdx.z * gridDim.y * gridDim.x + tile) * 256 + tid) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) dst[q] = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        return;
    }
    tile_err(a, M, N, Yq, ldy, red, part);
}

// Adds the ns splits' partial products of each tile in split order, then
// finishes the tile as a single-split k_outerr does. Grid (tiles of W rows,
// tiles of X rows).
__global__ __launch_bounds__(256) void k_outerr_fin(const float *__restrict__ py, int64_t ns, int64_t M, int64_t N,
                                                    const float *__restrict__ Yq, int64_t ldy,
                                                    double *__restrict__ part) {
    __shared__ double red[256];
    const int64_t tiles = (int64_t)gridDim.y * gridDim.x, tile = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = 0.f;
    for (int64_t z = 0; z < ns; ++z) {
        const float4 *src = reinterpret_cast<const float4 *>(py + ((z * tiles + tile) * 256 + threadIdx.x) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = src[q];
            a[4 * q] += v.x;
            a[4 * q + 1] += v.y;
            a[4 * q + 2] += v.z;
            a[4 * q + 3] += v.w;
        }
    }
    tile_err(a, M, N, Yq, ldy, red, part);
}

// err = sum of part[0 .. n) in a fixed order: thread i adds part[i + 256 j]
// for increasing j, then thread 0 adds the 256 thread sums in order.
__global__ __launch_bounds__(256) void k_outerr_sum(const double *__restrict__ part, int64_t n,
                                                    double *__restrict__ err) {
    __shared__ double red[256];
    double s = 0.0;
    for (int64_t i = threadIdx.x; i < n; i += 256) s += part[i];
    red[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < 256; ++i) t += red[i];
        *err = t;
    }
}

}  // namespace

// K splits of the output-error product: with fewer than four 64 x 64 tiles
// per compute unit, up to 4 splits per tile fill the chip (the 1024-row k and
// v projections have 64 tiles at 256 tokens, q and o 512).
int64_t outerr_splits(int64_t tiles) {
    if (tiles <= 0 || tiles >= 1024) return 1;
    const int64_t s = ceil_div((int64_t)1024, tiles);
    return s < 4 ? s : 4;
}

size_t output_error_workspace(int64_t M, int64_t N) {
    const int64_t tiles = ceil_div(M, kET) * ceil_div(N, kET);
    const int64_t ns = outerr_splits(tiles);
    const size_t parts = (size_t)(tiles > 0 ? tiles : 1) * sizeof(double);
    // partial products start at the first 16-byte boundary after the tile sums
    return ns > 1 ? parts + 16 + (size_t)(ns * tiles) * kET * kET * sizeof(float) : parts;
}

hipError_t launch_output_error(const void *X, const void *W, mxs_dtype dtype, int64_t M, int64_t N, int64_t K,
                               int64_t ldx, int64_t ldw, const float *Yq, int64_t ldy, double *err, void *ws,
                               hipStream_t st) {
    double *part = static_cast<double *>(ws);
    const int64_t tx = ceil_div(N, kET), ty = ceil_div(M, kET);
    if (tx > 0 && ty > 0) {
        const int64_t ns = outerr_splits(tx * ty);
        // partial products at the first 16-byte boundary after the tile sums
        float *py = ns > 1 ? reinterpret_cast<float *>((reinterpret_cast<uintptr_t>(part + tx * ty) + 15) &
                                                      ~(uintptr_t)15)
                           : nullptr;
        const int64_t kper = ceil_div(ceil_div(K, (int64_t)kEK), ns) * kEK;
        const dim3 grid((unsigned)tx, (unsigned)ty, (unsigned)ns);
        if (dtype == MXS_BF16)
            hipLaunchKernelGGL((k_outerr<uint16_t>), grid, dim3(256), 0, st, static_cast<const uint16_t *>(X), M, ldx,
                               static_cast<const uint16_t *>(W), N, ldw, K, kper, Yq, ldy, py, part);
        else
            hipLaunchKernelGGL((k_outerr<float>), grid, dim3(256), 0, st, static_cast<const float *>(X), M, ldx,
                               static_cast<const float *>(W), N, ldw, K, kper, Yq, ldy, py, part);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (ns > 1) {
            hipLaunchKernelGGL(k_outerr_fin, dim3((unsigned)tx, (unsigned)ty), dim3(256), 0, st, py, ns, M, N, Yq,
                               ldy, part);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL(k_outerr_sum, dim3(1), dim3(256), 0, st, part, (tx > 0 && ty > 0) ? tx * ty : (int64_t)0, err);
    return hipGetLastError();
}

// Layer budget (host). Returns 0, or 1 when B cannot pay for the 8-bit
// blocks. Arguments are validated by the caller.
int layer_budget(int32_t L, const double *S, const int64_t *rows, const int64_t *K, double B, int32_t *nblk,
                 double *R_out) {
    struct Break {
        double key;   // (j - 1/2) / S_l
        int32_t layer, j;
    };
    double total = 0.0;
    int64_t used = 0;   // mantissa bits above 4 per weight, summed
    std::vector<Break> br;
    for (int32_t l = 0; l < L; ++l) {
        total += (double)rows[l] * (double)K[l];
        used += 4 * 32 * rows[l];
        const int32_t nb = (int32_t)(K[l] / 32);
        nblk[3 * l] = 1;
        nblk[3 * l + 1] = 0;
        nblk[3 * l + 2] = nb - 1;
        if (S[l] > 0.0)
            for (int32_t j = 1; j < nb; ++j) br.push_back(Break{((double)j - 0.5) / S[l], l, j});
    }
    const int64_t allowed = (int64_t)std::floor((B - 4.0) * total);
    if (used > allowed) return 1;
    std::sort(br.begin(), br.end(), [](const Break &a, const Break &b) {
        if (a.key != b.key) return a.key < b.key;
        if (a.layer != b.layer) return a.layer < b.layer;
        return a.j < b.j;
    });
    double R = 0.0;
    for (size_t i = 0; i < br.size();) {
        size_t e = i;
        int64_t add = 0;
        for (; e < br.size() && br[e].key == br[i].key; ++e) add += 2 * 32 * rows[br[e].layer];
        if (used + add > allowed) break;
        used += add;
        R = br[i].key;
        for (size_t q = i; q < e; ++q) {
            nblk[3 * br[q].layer + 1] = br[q].j;
            nblk[3 * br[q].layer + 2] = (int32_t)(K[br[q].layer] / 32) - 1 - br[q].j;
        }
        i = e;
    }
    if (R_out) *R_out = R;
    return 0;
}

}  // namespace mxs
