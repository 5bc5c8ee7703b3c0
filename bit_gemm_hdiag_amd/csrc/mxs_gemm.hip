// mxs_gemm.hip -- block-scaled mixed 4/6/8-bit MXINT GEMM on gfx950.
//
//   Y[t, n] = sum_b 2^(sa[t,b] + sw[n,b]) * sum_{j in b} ca[t, j] cw[n, j]
//
// gist.science/nl "Technische Samenvatting" §1 and §5 and the romaanj.github.io
// review ("Comparison"): the MX block scales are applied inside the product,
// with no dequantisation pass. A (tokens) and W (weights) share the channel
// permutation, so block b of both operands has the same width m.
//
// The one dense contraction of the method runs on the int8 matrix cores:
// v_mfma_i32_32x32x32_i8 takes exactly one 32-deep MXINT block, so each MFMA
// yields the exact integer block sums I_b of a 32x32 output tile. Codes enter
// the MFMA as bytes: 8-bit codes as is, 6-bit codes shifted left by 2 and
// 4-bit codes by 4 (the field lands in the top bits of the byte, which is a
// free sign extension); the shift is folded back into the block scale.
// Every block term I_b * 2^(sa+sw) is exact in fp32 (|I_b| < 2^24, power-of-
// two scale); only the fp32 accumulation across blocks rounds.
//
// Layout of the 32x32x32 i8 MFMA on a 64-lane wavefront: lane l supplies row
// (l mod 32) of A and column (l mod 32) of B, 16 bytes each from k-half
// l / 32; result register 4q + r of lane l is row 8q + 4(l / 32) + r, column
// l mod 32. A and B use the same byte-to-k assignment, so any fixed
// reordering of the k positions inside a block (as the 4-bit unpack does)
// leaves the block sum unchanged.
#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

struct QView {
    const int8_t *q8; int64_t ld8;
    const uint8_t *q6; int64_t ld6;
    const uint8_t *q4; int64_t ld4;
    const uint8_t *sc; int64_t lds;
};

// 16 codes (k-half h of block `blk`, width class m) of one row as MFMA bytes.
// 8-bit: codes; 6-bit: codes * 4; 4-bit: codes * 16 (k order within the
// half: 0,2,4,6,1,3,5,7, 8,10,..., the same for both operands).
__device__ __forceinline__ v4i operand8(const QView &Q, int64_t row, int64_t b8, int h) {
    return *reinterpret_cast<const v4i *>(Q.q8 + row * Q.ld8 + 32 * b8 + 16 * h);
}
__device__ __forceinline__ uint32_t six_to_bytes(uint32_t g) {
    return ((g << 2) & 0xFCu) | ((g << 4) & 0xFC00u) | ((g << 6) & 0xFC0000u) | ((g << 8) & 0xFC000000u);
}
__device__ __forceinline__ v4i operand6(const QView &Q, int64_t row, int64_t b6, int h) {
    const uint32_t *p = reinterpret_cast<const uint32_t *>(Q.q6 + row * Q.ld6 + 24 * b6 + 12 * h);
    const uint32_t w0 = p[0], w1 = p[1], w2 = p[2];
    v4i r;
    r[0] = (int)six_to_bytes(w0);
    r[1] = (int)six_to_bytes(__builtin_amdgcn_alignbit(w1, w0, 24));
    r[2] = (int)six_to_bytes(__builtin_amdgcn_alignbit(w2, w1, 16));
    r[3] = (int)six_to_bytes(w2 >> 8);
    return r;
}
__device__ __forceinline__ v4i operand4(const QView &Q, int64_t row, int64_t b4, int h) {
    const uint2 x = *reinterpret_cast<const uint2 *>(Q.q4 + row * Q.ld4 + 16 * b4 + 8 * h);
    v4i r;
    r[0] = (int)((x.x << 4) & 0xF0F0F0F0u);
    r[1] = (int)(x.x & 0xF0F0F0F0u);
    r[2] = (int)((x.y << 4) & 0xF0F0F0F0u);
    r[3] = (int)(x.y & 0xF0F0F0F0u);
    return r;
}

// ---------------------------------------------------------------------------
// Universal kernel: every shape, per-block scale epilogue.
// Workgroup = 4 waves as 2 (rows) x 2 (cols); a wave owns a 32 x 64 output
// tile (two MFMA tiles sharing the A fragment); the workgroup 64 x 128.
constexpr int kBM = 64, kBN = 128;

__global__ __launch_bounds__(256) void k_gemm_blockwise(QView A, QView W, int64_t M, int64_t N,
                                                        int32_t n8, int32_t n6, int32_t n4,
                                                        float *__restrict__ Y, int64_t ldy) {
    __shared__ float s_sa[kBM];
    __shared__ float s_sw[kBN];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
    // rows past the edge read the last row (results discarded)
    const int64_t ra = min(m0 + wm * 32 + l32, M - 1);
    const int64_t rw0 = min(n0 + wn * 64 + l32, N - 1);
    const int64_t rw1 = min(n0 + wn * 64 + 32 + l32, N - 1);
    const int64_t sra = min(m0 + tid, M - 1);
    const int64_t srw = min(n0 + (tid & 127), N - 1);

    float acc0[16], acc1[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) { acc0[i] = 0.f; acc1[i] = 0.f; }
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    const int64_t nb = (int64_t)n8 + n6 + n4;

    for (int64_t b = 0; b < nb; ++b) {
        const int cls = b < n8 ? 8 : (b < (int64_t)n8 + n6 ? 6 : 4);
        const float fold = cls == 8 ? 1.0f : (cls == 6 ? 0.25f : 0.0625f);
        if (tid < kBM) s_sa[tid] = e8m0_to_f32(A.sc[sra * A.lds + b]) * fold;
        if (tid < kBN) s_sw[tid] = e8m0_to_f32(W.sc[srw * W.lds + b]) * fold;
        v4i a, w0, w1;
        if (cls == 8) {
            a = operand8(A, ra, b, h); w0 = operand8(W, rw0, b, h); w1 = operand8(W, rw1, b, h);
        } else if (cls == 6) {
            const int64_t b6 = b - n8;
            a = operand6(A, ra, b6, h); w0 = operand6(W, rw0, b6, h); w1 = operand6(W, rw1, b6, h);
        } else {
            const int64_t b4 = b - n8 - n6;
            a = operand4(A, ra, b4, h); w0 = operand4(W, rw0, b4, h); w1 = operand4(W, rw1, b4, h);
        }
        __syncthreads();
        const v16i i0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, w0, zero, 0, 0, 0);
        const v16i i1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, w1, zero, 0, 0, 0);
        const float sw0 = s_sw[wn * 64 + l32], sw1 = s_sw[wn * 64 + 32 + l32];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float sa = s_sa[wm * 32 + 8 * q + 4 * h + r];
                acc0[4 * q + r] = __builtin_fmaf((float)i0[4 * q + r], sa * sw0, acc0[4 * q + r]);
                acc1[4 * q + r] = __builtin_fmaf((float)i1[4 * q + r], sa * sw1, acc1[4 * q + r]);
            }
        }
        __syncthreads();
    }
    const int64_t c0 = n0 + wn * 64 + l32, c1 = c0 + 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = m0 + wm * 32 + 8 * q + 4 * h + r;
            if (t < M) {
                if (c0 < N) Y[t * ldy + c0] = acc0[4 * q + r];
                if (c1 < N) Y[t * ldy + c1] = acc1[4 * q + r];
            }
        }
    }
}

QView view_of(const mxs_qmat &q) {
    return QView{q.q8, q.ld8, q.q6, q.ld6, q.q4, q.ld4, q.sc, q.lds};
}

}  // namespace

size_t gemm_workspace(const mxs_qmat &, const mxs_qmat &) { return 0; }

hipError_t launch_mixed_gemm(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy,
                             void *, size_t, hipStream_t st) {
    const int64_t M = A.rows, N = W.rows;
    if (M == 0 || N == 0) return hipSuccess;
    const dim3 grid((unsigned)ceil_div(N, kBN), (unsigned)ceil_div(M, kBM));
    hipLaunchKernelGGL(k_gemm_blockwise, grid, dim3(256), 0, st, view_of(A), view_of(W), M, N,
                       A.n8, A.n6, A.n4, Y, ldy);
    return hipGetLastError();
}

}  // namespace mxs
