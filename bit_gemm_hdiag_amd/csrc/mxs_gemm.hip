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
// the MFMA as bytes: 8-bit codes as is, 6-bit codes times 4 and 4-bit codes
// times 16 (the field lands in the top bits of the byte, which is a free sign
// extension); the factor is folded back into the block scale. Every block
// term I_b * 2^(sa+sw) is exact in fp32 (|I_b| < 2^24, power-of-two scale);
// only the fp32 accumulation across blocks rounds. This is mxs_mixed_gemm.
//
// mxs_mixed_gemm_mx runs the same product's prefill (64 or more tokens) on
// the block-scaled micro-float matrix cores instead, which apply the E8M0
// scales in hardware (see the section "Prefill variant on the block-scaled
// matrix cores"); below 64 tokens both use the kernels of mxs_mixed_gemm.
//
// Layout of the 32x32x32 i8 MFMA on a 64-lane wavefront: lane l supplies row
// (l mod 32) of A and column (l mod 32) of B, 16 bytes each from k-half
// l / 32; result register 4q + r of lane l is row 8q + 4(l / 32) + r, column
// l mod 32. A and B use the same byte-to-k assignment, so any fixed
// reordering of the k positions inside a block (as the 4-bit unpack does)
// leaves the block sum unchanged.
#include <cstring>

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

// ---------------------------------------------------------------------------
// Prefill path (M >= kPrefillMinRows): operand preparation + grouped GEMM.
//
// The per-block epilogue above costs 3 VALU operations per output and block,
// six times the MFMA time of the block. The prefill path removes it in two
// ways, both exact.
//
// Narrow blocks (4-bit codes): exponent alignment over windows of kG
// consecutive blocks. If a row's nonzero blocks in a window have scale
// exponents within F = 4 of each other (the headroom an int8 byte has over a
// 4-bit code), code c of block b is stored as c << (s_b - base) with base =
// max s_b - F; aligned A and W rows make the int32 MFMA sum over the window
// exact, times 2^(base_a + base_w): one epilogue per window. Other rows keep
// c << F with scale 2^(s_b - F) and the wave takes one epilogue per block for
// that window. Window sums stay below 2^24 (16 * 32 * 127^2), so the int32 ->
// fp32 conversion is exact and only the fp32 accumulation across windows
// rounds.
//
// Wide blocks (the 8- and 6-bit classes, whose codes leave an int8 byte no or
// two bits of headroom, so their windows practically never align): each
// element is stored as the bf16 value c * 2^s, which is exact (|c| <= 127 has
// at most 7 significant bits, bf16 keeps 8, and its exponent range is fp32's),
// and the bf16 matrix cores (v_mfma_f32_32x32x16_bf16) accumulate the exact
// products straight into the fp32 sums: no epilogue at all. The wide run is
// rounded up to a multiple of five blocks with the first 4-bit blocks (also
// exact in bf16), so that the GEMM's five-slot stage ring leaves the wide
// loop at slot 0; all blocks are wide when fewer 4-bit blocks remain.
//
// Prepared operand (workspace), per matrix with R rows padded to Rp; a row is
// a sequence of 32-byte units: units 2b and 2b + 1 hold wide block b < hw
// (bf16 elements 0..15 and 16..31), unit b + hw holds narrow block b >= hw,
// and the row is padded with zero units to Kp bytes (a multiple of 128):
//   codes [Rp, Kp]        W row-major, A (activations) in fragment order
//                         (afrag_off: 1 KiB per 32 rows and unit)
//   cs    f32 [Kp/32, Rp] narrow units: code scale of (row, block), negative
//                         when the row's window is not aligned, -Inf for a
//                         NaN/Inf block; wide units: 1 (never read)
// Padding rows hold zero units; padding units zero codes and scale +1. A
// NaN/Inf wide block is stored as bf16 NaN (the product is NaN for its whole
// row or column, as the definition gives).
constexpr int kG = 16;              // blocks per alignment window
constexpr int kPrefillMinRows = 64; // smaller M uses the per-block kernel

__device__ __forceinline__ int sext(uint32_t v, int bits) {
    return (int)(v << (32 - bits)) >> (32 - bits);
}

// The packed bytes of one row's block (8, 6 or 4 bits: 32, 24 or 16 bytes)
// as little-endian words, and their codes; split so that a thread can issue
// the loads of several rows before it unpacks any of them.
__device__ __forceinline__ void load_block_raw(const QView &Q, int64_t r, int64_t b, int cls, int32_t n8,
                                               int32_t n6, uint32_t w[8]) {
    if (cls == 8) {
        const uint4 *p = reinterpret_cast<const uint4 *>(Q.q8 + r * Q.ld8 + 32 * b);
        const uint4 x = p[0], y = p[1];
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w; w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
    } else if (cls == 6) {
        const uint32_t *p = reinterpret_cast<const uint32_t *>(Q.q6 + r * Q.ld6 + 24 * (b - n8));
#pragma unroll
        for (int i = 0; i < 6; ++i) w[i] = p[i];
        w[6] = 0; w[7] = 0;
    } else {
        const uint2 *p = reinterpret_cast<const uint2 *>(Q.q4 + r * Q.ld4 + 16 * (b - n8 - n6));
        const uint2 x = p[0], y = p[1];
        w[0] = x.x; w[1] = x.y; w[2] = y.x; w[3] = y.y; w[4] = 0; w[5] = 0; w[6] = 0; w[7] = 0;
    }
}

__device__ __forceinline__ void unpack_raw(const uint32_t w[8], int cls, int c[32]) {
    if (cls == 8) {
#pragma unroll
        for (int i = 0; i < 32; ++i) c[i] = sext((w[i >> 2] >> (8 * (i & 3))) & 255u, 8);
    } else if (cls == 6) {
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int bit = 24 * g;
            const uint32_t grp = __builtin_amdgcn_alignbit(w[(bit >> 5) + 1], w[bit >> 5], bit & 31);
#pragma unroll
            for (int j = 0; j < 4; ++j) c[4 * g + j] = sext((grp >> (6 * j)) & 63u, 6);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) c[i] = sext((w[i >> 3] >> (4 * (i & 7))) & 15u, 4);
    }
}

// One workgroup prepares a 64-row x 16-block window of one matrix: thread t
// takes block t % 16 of rows t / 16 + 16 i (reads and code writes run along
// the row), the window reduction is a 16-lane butterfly, and the scales are
// transposed through LDS so that they are written 64 rows at a time.
struct PrepJob {
    QView Q;
    int64_t R, Rp;
    int8_t *codes;
    float *cs;
    int64_t tiles_r;      // Rp / 64
    int32_t frag;         // codes in fragment order (afrag_off) rather than row-major
};

// Fragment order of the activation operand: for each group of 32 rows and
// each block, 1 KiB holding k-half 0 of the 32 rows (16 bytes each) and then
// k-half 1, so that the 64 lanes of a 32x32x32 MFMA fetch their A fragment
// of that block with one contiguous 16-byte load each (lane l: row l mod 32,
// k-half l / 32, bytes 16 l).
__host__ __device__ inline int64_t afrag_off(int64_t row, int64_t b, int h, int64_t nbp) {
    return (((row >> 5) * nbp + b) << 10) + ((int64_t)h << 9) + ((row & 31) << 4);
}

// Four segments of blocks: 8-bit, 6-bit and 4-bit wide blocks, then the
// narrow 4-bit blocks. The preparation works in windows that start at the
// first block of each segment: window j of segment [lo, hi) covers blocks
// lo + kG j .. min(hi, lo + kG (j + 1)) - 1; only the narrow segment's
// windows are alignment windows.
constexpr int kWideStep = 5;   // the wide run is a multiple of this many blocks
struct Segs {
    int32_t lo[4], hi[4], cls[4];
    int32_t win_base[5];   // prefix count of windows per segment
    int32_t hw;            // wide blocks (units 0 .. 2 hw - 1)
    int32_t nq;            // units of a row before padding: 2 hw + (nb - hw)
};

__host__ __device__ inline Segs make_segs(int32_t n8, int32_t n6, int32_t n4) {
    Segs S;
    const int32_t nb = n8 + n6 + n4, h1 = n8 + n6;
    const int32_t up = (h1 + kWideStep - 1) / kWideStep * kWideStep;
    S.hw = up < nb ? up : nb;
    S.nq = nb + S.hw;
    const int32_t n[4] = {n8, n6, S.hw - h1, nb - S.hw};
    int32_t lo = 0, wb = 0;
    for (int i = 0; i < 4; ++i) {
        S.lo[i] = lo;
        S.hi[i] = lo + n[i];
        S.cls[i] = i == 0 ? 8 : (i == 1 ? 6 : 4);
        S.win_base[i] = wb;
        wb += (n[i] + kG - 1) / kG;
        lo += n[i];
    }
    S.win_base[4] = wb;
    return S;
}

// bf16 bits of c * 2^s for an integer code |c| <= 127 (exact: see above)
__device__ __forceinline__ uint32_t bf16_of_code(int c, int s) {
    return __float_as_uint(__builtin_ldexpf((float)c, s)) >> 16;
}

// One workgroup prepares a 64-row x (one window) tile of one matrix: thread t
// takes block t % 16 of the window for rows t / 16 + 16 i (reads and code
// writes run along the row); it issues the loads of its four rows before it
// unpacks the first. A wide window writes bf16 values (64 bytes per row and
// block). A narrow window reduces its scale exponents with a 16-lane
// butterfly and transposes the scales through LDS (rows padded to 68 floats,
// so the 64 lanes of a store hit 64 distinct banks) to write them 64 rows at
// a time. Padding windows cover units nq .. Kp/32 - 1, 16 per window.
constexpr int kPrepCsPitch = 68;
__global__ __launch_bounds__(256) void k_gemm_prep(PrepJob ja, PrepJob jw, int64_t ntiles_a, int64_t Kp, Segs S) {
    __shared__ __attribute__((aligned(16))) float s_cs[kG][kPrepCsPitch];
    const bool is_a = blockIdx.x < ntiles_a;
    const PrepJob &J = is_a ? ja : jw;
    const int64_t tile = is_a ? blockIdx.x : blockIdx.x - ntiles_a;
    const int64_t rt = tile % J.tiles_r, win = tile / J.tiles_r;   // win < windows + pad windows
    const int tid = threadIdx.x, blk = tid & 15;
    const int64_t nup = Kp / 32;
    const bool pad = win >= S.win_base[4];
    int sg = 3;
    int64_t b, u;   // block (real windows) and unit of this thread's column
    bool real_blk;
    if (!pad) {
        sg = win < S.win_base[1] ? 0 : (win < S.win_base[2] ? 1 : (win < S.win_base[3] ? 2 : 3));
        b = S.lo[sg] + (win - S.win_base[sg]) * kG + blk;
        real_blk = b < S.hi[sg];
        u = sg < 3 ? 2 * b : b + S.hw;
    } else {
        b = -1;
        u = S.nq + (win - S.win_base[4]) * kG + blk;
        real_blk = false;
    }
    const bool wide = !pad && sg < 3;
    const int cls = S.cls[sg];
    uint32_t raw[4][8], sbyte[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = rt * 64 + (tid >> 4) + 16 * i;
        if (real_blk && r < J.R) {
            load_block_raw(J.Q, r, b, cls, S.hi[0], S.hi[1] - S.hi[0], raw[i]);
            sbyte[i] = J.Q.sc[r * J.Q.lds + b];
        }
    }
    if (wide) {   // uniform over the workgroup
        {   // the units' scale entries (never read) hold 1, so that every byte of the operand is set
            const int64_t u0 = 2 * (b - blk), uu = u0 + (tid >> 3);
            if (uu < 2 * (int64_t)S.hi[sg]) {
                float4 *dst = reinterpret_cast<float4 *>(J.cs + uu * J.Rp + rt * 64 + 8 * (tid & 7));
                dst[0] = make_float4(1.f, 1.f, 1.f, 1.f);
                dst[1] = make_float4(1.f, 1.f, 1.f, 1.f);
            }
        }
        if (!real_blk) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = rt * 64 + (tid >> 4) + 16 * i;
            uint32_t w[16];
            if (r < J.R) {
                int c[32];
                unpack_raw(raw[i], cls, c);
                const uint32_t byte = sbyte[i];
                const int s = (int)byte - 127;
#pragma unroll
                for (int k = 0; k < 16; ++k)
                    w[k] = byte == 0xFFu ? 0x7FC07FC0u : (bf16_of_code(c[2 * k], s) | (bf16_of_code(c[2 * k + 1], s) << 16));
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) w[k] = 0;
            }
            if (J.frag) {
#pragma unroll
                for (int q = 0; q < 4; ++q)   // elements 8q .. 8q + 7: unit u + q / 2, k-half q % 2
                    *reinterpret_cast<uint4 *>(J.codes + afrag_off(r, u + (q >> 1), q & 1, nup)) =
                        make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
            } else {
                uint4 *dst = reinterpret_cast<uint4 *>(J.codes + r * Kp + 32 * u);
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[q] = make_uint4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
            }
        }
        return;
    }
    constexpr int F = 4;   // narrow blocks: 4-bit codes in int8 bytes
    const bool in_range = u < nup;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int lr = (tid >> 4) + 16 * i;
        const int64_t r = rt * 64 + lr;
        const bool real = real_blk && r < J.R;
        int c[32];
        int s = 0;
        bool bad = false, nz = false;
        if (real) {
            unpack_raw(raw[i], cls, c);
            const uint32_t byte = sbyte[i];
            bad = byte == 0xFFu;
            s = (int)byte - 127;
#pragma unroll
            for (int k = 0; k < 32; ++k) nz |= c[k] != 0;
            if (bad) nz = false;
        } else {
#pragma unroll
            for (int k = 0; k < 32; ++k) c[k] = 0;
        }
        int smax = nz ? s : -100000, smin = nz ? s : 100000, anybad = bad;
#pragma unroll
        for (int off = 1; off < kG; off <<= 1) {
            smax = max(smax, __shfl_xor(smax, off));
            smin = min(smin, __shfl_xor(smin, off));
            anybad |= __shfl_xor(anybad, off);
        }
        const bool allzero = smax == -100000;
        const bool aligned = !anybad && (allzero || smax - smin <= F);
        const int base = allzero ? 0 : smax - F;
        const int shift = aligned ? (nz ? s - base : 0) : F;
        float scale;
        if (!real) scale = 1.0f;
        else if (bad) scale = -__builtin_inff();
        else scale = aligned ? __builtin_ldexpf(1.0f, base) : -__builtin_ldexpf(1.0f, s - F);
        uint32_t w[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t v = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) v |= (((uint32_t)c[4 * k + j] << shift) & 255u) << (8 * j);
            w[k] = v;
        }
        if (in_range && (real_blk || pad)) {
            if (J.frag) {
                int8_t *dst = J.codes + afrag_off(r, u, 0, nup);
                *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
                *reinterpret_cast<uint4 *>(dst + 512) = make_uint4(w[4], w[5], w[6], w[7]);
            } else {
                uint4 *dst = reinterpret_cast<uint4 *>(J.codes + r * Kp + 32 * u);
                dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
                dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
            }
        }
        s_cs[blk][lr] = scale;
    }
    __syncthreads();
    {
        const int bb = tid >> 4, part = tid & 15;
        const int64_t ou = u - blk + bb;   // unit of this transposed slice
        const bool ok = pad ? ou < nup : b - blk + bb < S.hi[3];
        if (ok) {
            const float4 v = *reinterpret_cast<const float4 *>(&s_cs[bb][4 * part]);
            *reinterpret_cast<float4 *>(J.cs + ou * J.Rp + rt * 64 + 4 * part) = v;
        }
    }
}

// Activation operand straight from X (the fused entry point): the same
// prepared layout as k_gemm_prep writes from planes, computed from the
// unquantized rows. A workgroup walks rows; each row and the permutation
// (16-bit) are staged in LDS; wave w takes windows w, w + 4, ... of the row:
// lane (block t / 4 of the window, quarter t % 4) gathers its 8 values,
// quantizes them at the block's width (the quantizer of mxs_quantize: scale
// from the quad's largest magnitude, codes rounded half to even and clamped
// symmetrically); a wide window stores the codes as bf16 values and a narrow
// window's alignment (16-lane-group reduction of the blocks' scale exponents)
// shifts them, exactly as k_gemm_prep does. Rows R .. Rp - 1 get zero units,
// padding units zero codes and scale 1.
// Rows are streamed one ahead: each thread holds its PPT 16-byte pieces of
// the workgroup's next row in registers while the current row is quantized
// (16-byte aligned rows; others are staged element by element).
template <typename T, int PPT>
__global__ __launch_bounds__(256) void k_quant_prep(const T *__restrict__ X, int64_t R, int64_t ldx,
                                                    const int32_t *__restrict__ perm, int64_t K, int64_t Rp,
                                                    int64_t Kp, Segs S, int8_t *__restrict__ codes,
                                                    float *__restrict__ cs) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint16_t *sperm = reinterpret_cast<uint16_t *>(lds);
    T *srow = reinterpret_cast<T *>(lds + ((2 * K + 15) / 16) * 16);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int blk = lane >> 2, q = lane & 3;
    if (perm) {
        stage_perm(perm, K, sperm, tid);
    } else {
        for (int64_t j = tid; j < K; j += 256) sperm[j] = (uint16_t)j;
    }
    const int64_t nup = Kp / 32;
    const int64_t nwin = S.win_base[4] + (nup - S.nq + kG - 1) / kG;
    const int64_t nvec = K * (int64_t)sizeof(T) / 16;
    const bool vec = reinterpret_cast<uintptr_t>(X) % 16 == 0 && (ldx * (int64_t)sizeof(T)) % 16 == 0;
    const int64_t G = gridDim.x;
    // Row order by XCD: workgroups are dealt to the eight XCDs in turn, so
    // workgroup w works as v = (w mod 8) G / 8 + w / 8 and each XCD walks a
    // contiguous run of rows. The 8 rows that share a 128-byte line of the
    // fragment-ordered codes (and the 32 that share a line of scales) are
    // then written through one L2 instead of eight.
    const int64_t v0 = (G & 7) ? (int64_t)blockIdx.x : (int64_t)(blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
    u32x4 ring[PPT];
    auto fetch = [&](int64_t row) {
        if (vec && row < R) {
            const u32x4 *x = reinterpret_cast<const u32x4 *>(X + row * ldx);
#pragma unroll
            for (int i = 0; i < PPT; ++i)
                if (tid + 256 * i < nvec) ring[i] = __builtin_nontemporal_load(x + tid + 256 * i);
        }
    };
    fetch(v0);
    for (int64_t row = v0; row < Rp; row += G) {
        const bool real_row = row < R;
        __syncthreads();                       // the previous row's gathers are done (and sperm is staged)
        if (real_row) {
            if (vec) {
#pragma unroll
                for (int i = 0; i < PPT; ++i)
                    if (tid + 256 * i < nvec) reinterpret_cast<u32x4 *>(srow)[tid + 256 * i] = ring[i];
            } else {
                const T *x = X + row * ldx;
                for (int64_t j = tid; j < K; j += 256) srow[j] = x[j];
            }
        }
        __syncthreads();
        fetch(row + G);                        // in flight while this row is quantized
        for (int64_t win = wave; win < nwin; win += 4) {
            const bool pad = win >= S.win_base[4];
            int sg = 3;
            int64_t b, u;
            bool real_blk;
            if (!pad) {
                sg = win < S.win_base[1] ? 0 : (win < S.win_base[2] ? 1 : (win < S.win_base[3] ? 2 : 3));
                b = S.lo[sg] + (win - S.win_base[sg]) * kG + blk;
                real_blk = b < S.hi[sg];
                u = sg < 3 ? 2 * b : b + S.hw;
            } else {   // padding units nq .. Kp/32 - 1
                b = 0;
                u = S.nq + (win - S.win_base[4]) * kG + blk;
                real_blk = false;
            }
            const int cls = S.cls[sg];
            const bool real = real_blk && real_row;
            float v[8];
            if (real) {
                const uint4 pi = *reinterpret_cast<const uint4 *>(sperm + 32 * b + 8 * q);
                const uint32_t w[4] = {pi.x, pi.y, pi.z, pi.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = load1<T>(srow + (w[i] & 0xFFFFu));
                    v[2 * i + 1] = load1<T>(srow + (w[i] >> 16));
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = 0.f;
            }
            // codes of the quarter as bytes (the quantizer of mxs_quantize)
            uint32_t a = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t m = __float_as_uint(v[i]) & 0x7fffffffu;
                a = a > m ? a : m;
            }
            a = quad_max_u32(a);
            const BlockScale bs = block_scale(a, cls);
            const float magic = 12582912.0f, cm = cmax_of(cls);
            uint32_t cb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                cb[i] = __float_as_uint(__builtin_amdgcn_fmed3f(__builtin_fmaf(v[i], bs.inv, magic), magic - cm, magic + cm));
            uint32_t lo = __builtin_amdgcn_perm(cb[1], cb[0], 0x0C0C0400u) | __builtin_amdgcn_perm(cb[3], cb[2], 0x04000C0Cu);
            uint32_t hi = __builtin_amdgcn_perm(cb[5], cb[4], 0x0C0C0400u) | __builtin_amdgcn_perm(cb[7], cb[6], 0x04000C0Cu);
            const bool bad = real && bs.bad;
            const int s = (int)bs.byte - 127;
            if (!pad && sg < 3) {   // wide window (uniform over the wave): bf16 c * 2^s
                if (real_blk) {
                    uint32_t w[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c0 = (int)(__uint_as_float(cb[2 * i]) - magic);
                        const int c1 = (int)(__uint_as_float(cb[2 * i + 1]) - magic);
                        w[i] = !real ? 0u : (bad ? 0x7FC07FC0u : (bf16_of_code(c0, s) | (bf16_of_code(c1, s) << 16)));
                    }
                    *reinterpret_cast<uint4 *>(codes + afrag_off(row, u + (q >> 1), q & 1, nup)) =
                        make_uint4(w[0], w[1], w[2], w[3]);
                    if (q < 2) cs[(u + q) * Rp + row] = 1.0f;   // never read
                }
                continue;
            }
            constexpr int F = 4;
            if (bad) lo = hi = 0;
            const uint32_t anynz = quad_max_u32((lo | hi) != 0 ? 1u : 0u);   // whole quad, unconditionally
            const bool nz = real && !bad && anynz != 0;
            // window reduction over the 16 blocks (lanes 4 apart), one packed
            // word per step: high half max(s), low half max(-s) = -min(s); a
            // non-finite block enters as +32767 in both halves, which makes
            // the window unaligned; blocks without nonzero codes as -32768
            const int hi16 = nz ? s : (bad ? 32767 : -32768);
            const int lo16 = nz ? -s : (bad ? 32767 : -32768);
            uint32_t red = ((uint32_t)hi16 << 16) | ((uint32_t)lo16 & 0xFFFFu);
#pragma unroll
            for (int off = 4; off < 64; off <<= 1) {
                const uint32_t o = (uint32_t)__shfl_xor((int)red, off);
                typedef short v2s __attribute__((ext_vector_type(2)));
                const v2s m = __builtin_elementwise_max(__builtin_bit_cast(v2s, red), __builtin_bit_cast(v2s, o));
                red = __builtin_bit_cast(uint32_t, m);
            }
            const int smax = (int)(int16_t)(red >> 16), smin = -(int)(int16_t)(red & 0xFFFFu);
            const bool allzero = smax == -32768;
            const bool aligned = allzero || smax - smin <= F;
            const int base = allzero ? 0 : smax - F;
            const int shift = aligned ? (nz ? s - base : 0) : F;
            float scale;
            if (!real) scale = 1.0f;
            else if (bad) scale = -__builtin_inff();
            else scale = aligned ? __builtin_ldexpf(1.0f, base) : -__builtin_ldexpf(1.0f, s - F);
            // per-byte left shift (bits pushed into the next byte are masked off)
            const uint32_t keep = 0x01010101u * ((0xFFu << shift) & 0xFFu);
            lo = (lo << shift) & keep;
            hi = (hi << shift) & keep;
            if (u < nup && (real_blk || pad)) {
                *reinterpret_cast<uint2 *>(codes + afrag_off(row, u, q >> 1, nup) + 8 * (q & 1)) = make_uint2(lo, hi);
                if (q == 0) cs[u * Rp + row] = scale;
            }
        }
    }
}

// Grouped int8 GEMM over prepared operands (the prefill kernel of
// mxs_mixed_gemm and mxs_mixed_gemm_fused).
//
// Workgroup: 8 waves (8 x 1), tile 256 (A rows) x 128 (W rows); wave w owns
// A rows 32 w .. 32 w + 31 against all 128 W rows, i.e. 1 x 4 MFMA tiles
// (64 int32 + 64 fp32 accumulators per lane, two waves per SIMD). Every A
// fragment therefore belongs to one wave: it is fetched from the
// fragment-ordered operand (afrag_off) with one 16-byte load per lane and
// block, four stages ahead, into a register ring that follows the LDS ring's
// slots. W codes and both operands' scales move from global memory straight
// into LDS (global_load_lds_dwordx4), which no register holds in flight.
// (An earlier version also streamed A through LDS by DMA; the DMA path, not
// the matrix cores, then bounded it, and moving A to registers took two
// thirds of the bytes off that path.)
//
// Stage = kDSB = 2 blocks (64 bytes of every W row) plus the scales of both
// operands, 11 KiB; a ring of five stage slots. Iteration s: wait for this
// wave's loads of stage s (the loads of stages s+1 .. s+3 stay in flight),
// barrier (every wave's loads of stage s have landed and every wave is done
// with stage s-1), issue stage s+4 into the slot of stage s-1, compute s.
// A DMA instruction writes 64 consecutive 16-byte LDS slots, lane by lane;
// lanes pick their global chunk so that row r keeps chunk c at slot
// c ^ ((r >> 2) & 3) of its 64 bytes: the 16 lanes of one LDS read pass
// (16 consecutive rows, same chunk) then hit 16 distinct 16-byte bank groups.
//
// A block whose integer sums end (the last block of its window, or any
// block of a window whose rows are not all aligned) needs an epilogue.
// Inside a stage it is left pending: the next block runs it (by then the
// block's MFMAs have finished, so the vector ALU does not wait for them),
// tile by tile, each tile followed by a restart MFMA that zeroes its integer
// sums in place (the matrix core has slack, the vector ALU has none), then
// the new block's MFMAs accumulate as usual. The last block of a stage runs
// its epilogue at once: the next step's DMA refills the slot of the stage
// before the one it computes, so scales cannot be read across that step.
// After the loop no DMA follows, so a pending epilogue of the final stage
// runs there.
constexpr int kGBM = 256, kGBN = 128;        // workgroup tile
constexpr int kDSB = 2;                      // blocks per stage
constexpr int kDRow = kDSB * 32;             // 64 bytes per row per stage

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void *)p);
}

// One 16-byte-per-lane DMA into LDS at lds + 16 * lane. Issued from inline
// assembly so that the compiler does not order the slot reads behind every
// outstanding DMA (its wait model cannot separate the ring slots here); the
// kernel waits for its own DMAs explicitly (vmcnt) before a barrier. The
// instruction writes no VGPR; M0 carries the wave-uniform LDS base.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds)
                 : "memory", "m0");
}

constexpr int kAW = kGBN * kDRow;            // 8 KiB: W codes of a stage
constexpr int kACA = kDSB * kGBM * 4;        // 2 KiB: A scales
constexpr int kACW = kDSB * kGBN * 4;        // 1 KiB: W scales
constexpr int kASlot = kAW + kACA + kACW;

__shared__ __attribute__((aligned(16))) int8_t g_aslot0[kASlot];
__shared__ __attribute__((aligned(16))) int8_t g_aslot1[kASlot];
__shared__ __attribute__((aligned(16))) int8_t g_aslot2[kASlot];
__shared__ __attribute__((aligned(16))) int8_t g_aslot3[kASlot];
__shared__ __attribute__((aligned(16))) int8_t g_aslot4[kASlot];

template <int SL>
__device__ __forceinline__ int8_t *aslot() {
    return SL == 0 ? g_aslot0 : (SL == 1 ? g_aslot1 : (SL == 2 ? g_aslot2 : (SL == 3 ? g_aslot3 : g_aslot4)));
}

struct A2RLanes {
    const int8_t *w;          // this lane's W chunk at stage 0
    const float *c;           // scales (waves 0..2)
    int64_t cstep;            // scale address step per stage
    int ow, oc;               // wave-uniform LDS offsets inside a slot
    const v4i *a;             // this lane's A fragment of block 0
};

template <int SL>
__device__ __forceinline__ void a2r_issue(const A2RLanes &D, int st, int nstage, bool has_c, v4i (&ar)[5][kDSB]) {
    const int s = st < nstage ? st : nstage - 1;      // past the end: reload the last stage
    const uint32_t slot = lds_addr(aslot<SL>());
    dma16(D.w + (int64_t)s * kDRow, slot + D.ow);
    if (has_c) dma16(D.c + s * D.cstep, slot + D.oc);
#pragma unroll
    for (int blk = 0; blk < kDSB; ++blk) ar[SL][blk] = D.a[(int64_t)(s * kDSB + blk) * 64];
}

// Split over K (SplitK, blockIdx.y = split): split k takes stages
// s[k] .. s[k+1] - 1 and writes its fp32 tile sums to part[k][M][N]; a second
// kernel adds the splits in order. Boundaries inside the wide run are
// multiples of the ring's five slots, those after it multiples of a 16-unit
// window (8 stages), so every split enters the narrow loop at slot 0 and no
// window straddles two splits.
struct SplitK {
    int32_t n;        // splits (1: no split, the tile sums go to Y)
    int32_t s[9];     // stage bounds, s[0] = 0, s[n] = all stages
};
constexpr int kMaxSplitK = 8;

__global__ __launch_bounds__(512, 1) void k_gemm_a2r(
    const int8_t *__restrict__ Af, const float *__restrict__ csA, const int8_t *__restrict__ Wq,
    const float *__restrict__ csW, int64_t M, int64_t N, int64_t Mp, int64_t Np, int64_t Kp,
    int32_t nb, Segs S, float *__restrict__ Y, int64_t ldy, int32_t gm, SplitK SK, float *__restrict__ part) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;

    // tile order: each XCD (workgroups are dealt round-robin to the 8 XCDs)
    // takes a contiguous run of tiles; runs sweep groups of gm row-tiles
    const int64_t tilesM = Mp / kGBM, tilesN = Np / kGBN, ntiles = tilesM * tilesN;
    int64_t t = blockIdx.x;
    if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
    const int64_t per_group = gm * tilesN;
    const int64_t gid = t / per_group, first_m = gid * gm;
    const int64_t gsz = tilesM - first_m < gm ? tilesM - first_m : gm;
    const int64_t tm = first_m + (t % per_group) % gsz, tn = (t % per_group) / gsz;
    const int64_t m0 = tm * kGBM, n0 = tn * kGBN;
    const int64_t nbp = Kp / 32;
    const int hw = __builtin_amdgcn_readfirstlane(S.hw);   // wide blocks = wide stages
    // this split's stages s0 .. nstage - 1 and units .. ub - 1; the wide loop
    // ends at wend, where the narrow loop starts
    const int s0 = __builtin_amdgcn_readfirstlane(SK.s[blockIdx.y]);
    const int nstage = __builtin_amdgcn_readfirstlane(SK.s[blockIdx.y + 1]);
    const int ub = min(nb, kDSB * nstage);
    const int wend = min(max(hw, s0), nstage);

    // DMA roles: W rows 16 wave .. +15; waves 0, 1: A scales of block 0 / 1;
    // wave 2: W scales
    A2RLanes D;
    {
        const int rsub = lane >> 2, sl = lane & 3;
        const int rw = 16 * wave + rsub;
        D.w = Wq + (n0 + rw) * Kp + ((sl ^ ((rw >> 2) & 3)) << 4);
        D.ow = 16 * wave * kDRow;
        if (wave < 2) {
            D.c = csA + (int64_t)wave * Mp + m0 + 4 * lane;
            D.cstep = kDSB * Mp;
            D.oc = kAW + wave * (kGBM * 4);
        } else {
            D.c = csW + (int64_t)(lane >> 5) * Np + n0 + 4 * (lane & 31);
            D.cstep = kDSB * Np;
            D.oc = kAW + kACA;
        }
        D.a = reinterpret_cast<const v4i *>(Af + afrag_off(m0 + 32 * wave, 0, 0, nbp)) + lane;
    }
    const bool has_c = wave < 3;

    // LDS offset of this lane's W fragment j of block blk: fbW[j] ^ (blk << 5)
    int fbW[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rw = j * 32 + l32;
        fbW[j] = rw * kDRow + ((h ^ ((rw >> 2) & 3)) << 4);
    }

    v16f acc[4];
    v16i I[4];
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
    // a zero B operand the compiler cannot see through, for the restart
    // MFMAs; the four tiles' restarts share their A operand too, so each uses
    // its own B lane-broadcast pattern (blgp = j; a zero B stays zero under
    // any of them): otherwise they would be merged into one MFMA plus vector
    // copies of its result
    v4i zb;
    {
        int z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        zb = v4i{z, z, z, z};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        I[j] = zero;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
    }
    v4i ar[5][kDSB];

    bool aligned = true, pend = false;
    const float *pCA = nullptr, *pCW = nullptr;
    auto epi_all = [&](const v4i &fa) {   // epilogue of the pending block, tile by tile, each with its restart
        f32x4_t sa[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sa[q] = *reinterpret_cast<const f32x4_t *>(pCA + 8 * q + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float cw = __builtin_fabsf(pCW[j * 32 + l32]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[j][4 * q + e] =
                        __builtin_fmaf((float)I[j][4 * q + e], __builtin_fabsf(sa[q][e]) * cw, acc[j][4 * q + e]);
            switch (j) {   // blgp must be a constant
            case 0: I[0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, zb, zero, 0, 0, 0); break;
            case 1: I[1] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, zb, zero, 0, 0, 1); break;
            case 2: I[2] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, zb, zero, 0, 0, 2); break;
            default: I[3] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, zb, zero, 0, 0, 3); break;
            }
        }
    };
    auto compute = [&](int st, const int8_t *sbase, const v4i (&fa)[kDSB]) {
        const float *sCA = reinterpret_cast<const float *>(sbase + kAW);
        const float *sCW = sCA + kDSB * kGBM;
        v4i fw[4], nw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) nw[j] = *reinterpret_cast<const v4i *>(sbase + fbW[j]);
#pragma unroll
        for (int blk = 0; blk < kDSB; ++blk) {
            const int b = st * kDSB + blk;
#pragma unroll
            for (int j = 0; j < 4; ++j) fw[j] = nw[j];
            if (blk + 1 < kDSB) {
#pragma unroll
                for (int j = 0; j < 4; ++j) nw[j] = *reinterpret_cast<const v4i *>(sbase + (fbW[j] ^ ((blk + 1) << 5)));
            }
            if (b >= ub) break;
            const int off = b - 2 * hw;   // narrow windows start after the wide units
            const bool first = (off % kG) == 0;
            const bool last = (off % kG) == kG - 1 || b == ub - 1;
            if (first) {
                const float va = sCA[blk * kGBM + 32 * wave + l32];
                const float vw0 = sCW[blk * kGBN + lane], vw1 = sCW[blk * kGBN + 64 + lane];
                aligned = __all(va > 0.f && vw0 > 0.f && vw1 > 0.f);
            }
            if (pend) epi_all(fa[blk]);
#pragma unroll
            for (int j = 0; j < 4; ++j) I[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[blk], fw[j], I[j], 0, 0, 0);
            pend = last || !aligned;
            if (pend) {
                pCA = sCA + blk * kGBM + 32 * wave;
                pCW = sCW + blk * kGBN;
                if (blk == kDSB - 1) {
                    epi_all(fa[blk]);
                    pend = false;
                }
            }
        }
    };

    // a wide stage: one wide block (two units) of bf16 values, two bf16 MFMAs
    // per tile straight into the fp32 sums
    auto compute_wide = [&](const int8_t *sbase, const v4i (&fa)[kDSB]) {
        v4i fw[4];
#pragma unroll
        for (int u = 0; u < kDSB; ++u) {
#pragma unroll
            for (int j = 0; j < 4; ++j) fw[j] = *reinterpret_cast<const v4i *>(sbase + (fbW[j] ^ (u << 5)));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, fa[u]),
                                                                 __builtin_bit_cast(v8bf, fw[j]), acc[j], 0, 0, 0);
        }
    };

    // own loads of stage s done once at most three later stages are in flight
    // (per stage: one W DMA, two A fragments, and a scale DMA on waves 0..2)
#define MXS_WAIT_ISSUE(s_, NXT)                                                               \
    do {                                                                                      \
        if (has_c) __builtin_amdgcn_s_waitcnt(0x0F70 | 12); /* vmcnt(12) */                   \
        else __builtin_amdgcn_s_waitcnt(0x0F70 | 9);        /* vmcnt(9) */                    \
        lds_barrier();                                                                        \
        a2r_issue<NXT>(D, (s_) + 4, nstage, has_c, ar);                                       \
    } while (0)
    // the wide stages 0 .. hw - 1 come first; hw is a multiple of five (the
    // ring's length) unless every stage is wide, so the narrow loop always
    // starts at slot 0 (entering it at other slots makes the register
    // allocator spill)
#define MXS_WSTEP(s_, CUR, NXT)                                                               \
    do {                                                                                      \
        if ((s_) >= wend) goto narrow;                                                        \
        MXS_WAIT_ISSUE(s_, NXT);                                                              \
        compute_wide(aslot<CUR>(), ar[CUR]);                                                  \
    } while (0)
#define MXS_ASTEP(s_, CUR, NXT)                                                               \
    do {                                                                                      \
        if ((s_) >= nstage) goto done;                                                        \
        MXS_WAIT_ISSUE(s_, NXT);                                                              \
        compute((s_), aslot<CUR>(), ar[CUR]);                                                 \
    } while (0)

    a2r_issue<0>(D, s0, nstage, has_c, ar);
    a2r_issue<1>(D, s0 + 1, nstage, has_c, ar);
    a2r_issue<2>(D, s0 + 2, nstage, has_c, ar);
    a2r_issue<3>(D, s0 + 3, nstage, has_c, ar);
    for (int s = s0;; s += 5) {
        MXS_WSTEP(s, 0, 4);
        MXS_WSTEP(s + 1, 1, 0);
        MXS_WSTEP(s + 2, 2, 1);
        MXS_WSTEP(s + 3, 3, 2);
        MXS_WSTEP(s + 4, 4, 3);
    }
narrow:
    for (int s = wend;; s += 5) {
        MXS_ASTEP(s, 0, 4);
        MXS_ASTEP(s + 1, 1, 0);
        MXS_ASTEP(s + 2, 2, 1);
        MXS_ASTEP(s + 3, 3, 2);
        MXS_ASTEP(s + 4, 4, 3);
    }
done:
#undef MXS_ASTEP
#undef MXS_WSTEP
#undef MXS_WAIT_ISSUE
    if (pend) {
        f32x4_t sa[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) sa[q] = *reinterpret_cast<const f32x4_t *>(pCA + 8 * q + 4 * h);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float cw = __builtin_fabsf(pCW[j * 32 + l32]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    acc[j][4 * q + e] =
                        __builtin_fmaf((float)I[j][4 * q + e], __builtin_fabsf(sa[q][e]) * cw, acc[j][4 * q + e]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA outstanding at exit
    float *out = Y;
    int64_t ldo = ldy;
    if (SK.n > 1) {   // this split's sums into part[split][M][N]
        out = part + (int64_t)blockIdx.y * M * N;
        ldo = N;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + j * 32 + l32;
        if (col >= N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + 32 * wave + 8 * q + 4 * h + r;
                if (row < M) out[row * ldo + col] = acc[j][4 * q + r];
            }
    }
}

// ---------------------------------------------------------------------------
// Helpers of the block-scaled prefill variant below.
// s_waitcnt immediate that waits until at most n vector memory loads are
// outstanding (expcnt and lgkmcnt left at their maxima)
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// loads from an LDS byte address
typedef __attribute__((address_space(3))) const v4i lds_v4i_t;
__device__ __forceinline__ v4i lds_v4(uint32_t a) { return *reinterpret_cast<lds_v4i_t *>((uintptr_t)a); }
typedef __attribute__((address_space(3))) const int lds_i32_t;
__device__ __forceinline__ int lds_i32(uint32_t a) { return *reinterpret_cast<lds_i32_t *>((uintptr_t)a); }

// ---------------------------------------------------------------------------
// Prefill variant on the block-scaled matrix cores (mxs_mixed_gemm_mx).
//
// gfx950's v_mfma_scale_f32_32x32x64_f8f6f4 multiplies two 64-deep slabs of
// OCP micro-float elements and applies one E8M0 scale per 32 elements of
// every row and column inside the instruction (the MX format's own block
// scale), accumulating in fp32. MXINT codes are small integers, so they map
// onto fp6 E2M3 elements exactly (E2M3 holds every multiple of 1/2 up to
// 7.5) and the MXINT scale byte is the E8M0 scale as is:
//   4-bit c in [-7, 7]:    one element, c;                 scale byte s
//   6-bit c in [-31, 31]:  c = 8 hi + lo, hi in [-4, 4], lo in [-4, 3];
//                          two elements, scale bytes s + 3 and s
//   8-bit c in [-127,127]: c = 32 (hi/2) + 2 (lo/2), hi in [-8, 7],
//                          lo in [0, 15]; two elements, bytes s + 5, s + 1
// A 6- or 8-bit block pair then takes four MFMAs (hi*hi, hi*lo, lo*hi,
// lo*lo), a 4-bit pair one. Every product and every 64-term sum is exact
// inside the instruction; only the fp32 accumulation rounds, once per MFMA.
// An E8M0 byte of 0xFF (a NaN or Inf block) makes the instruction return
// NaN for the whole row or column, as the definition does. No per-block
// epilogue remains: the vector ALU only moves fragments.
//
// MFMA operand layout (fp6, 32x32x64): lane l supplies row l mod 32 and the
// 32 elements of k-half l / 32 (one MXINT block) as 6 little-endian packed
// 6-bit fields, and the scale byte of that (row, block) in bits 0..7 of its
// scale operand. Result register 4q + r of lane l is row 8q + 4(l / 32) + r,
// column l mod 32.
//
// Prepared operand (workspace), per matrix, rows in groups of 64, K in
// stages. A stage is two MFMA steps of 64 elements: the hi and lo digit
// steps of one 6/8-bit block pair, or two 4-bit block pairs. Stages: the
// 8-bit pairs, the 6-bit pairs, then the 4-bit pairs two at a time (an odd
// block or pair is completed with zero codes). Each (group, stage) is one
// 6400-byte record laid out exactly as the GEMM wants it in LDS:
//   chunk 3j + h (1 KiB, j = step, h = k-half): bytes 0..15 of the 24-byte
//                fragment of each of the 64 rows, 16 bytes per row;
//   chunk 3j + 2: bytes 16..23 of the fragments, 8 bytes per row, the 64
//                rows of k-half 0 and then those of k-half 1;
//   bytes 6144..6399: four scale bytes per row, byte 2j + h.
// Rows past the matrix hold zero codes and zero scale bytes.
constexpr int kXBM = 256, kXBN = 256;    // workgroup tile (A rows x W rows)
constexpr int kXCode = 6144;             // code bytes of a (group, stage) record
constexpr int kXRec = kXCode + 256;      // record bytes
constexpr int kXGA = kXBM / 64, kXGW = kXBN / 64;
constexpr int kXGroups = kXGA + kXGW;
// LDS image of one stage of the workgroup tile: the code parts of the eight
// group records (A groups 0..3, W groups 0..3), then the A scale parts and
// the W scale parts
constexpr int kXScA = kXGroups * kXCode;        // 49152
constexpr int kXScW = kXScA + kXGA * 256;       // 50176
constexpr int kXSink = kXScW + kXGW * 256;      // 51200: 1 KiB that absorbs the two padding loads
constexpr int kXSlot = kXSink + 1024;           // 52224
constexpr int kXRing = 3;                       // stage slots
constexpr int kXLoads = 13;                     // loads per wave and stage
static_assert(6 * kXGroups + 2 == 4 * kXLoads - 2, "50 loads per stage over four waves, plus two into the sink");

struct XPlan {
    int32_t p8, p6, p4;   // block pairs per width class
    int32_t nd;           // digit stages (8- and 6-bit pairs)
    int32_t ns;           // stages
};

__host__ __device__ inline XPlan make_xplan(int32_t n8, int32_t n6, int32_t n4) {
    XPlan P;
    P.p8 = (n8 + 1) / 2;
    P.p6 = (n6 + 1) / 2;
    P.p4 = (n4 + 1) / 2;
    P.nd = P.p8 + P.p6;
    P.ns = P.nd + (P.p4 + 1) / 2;
    return P;
}

// E2M3 encoding, four elements per 32-bit word. Each width class turns its
// code into a 4-bit table index per byte, and a 16-entry byte table (two
// v_perm lookups and a select on index bit 3) gives the E2M3 codes:
//   4-bit code c:            index = nibble ^ 8 (= c + 8),   value c
//   6-bit c, lo digit:       index = ((c & 7) + 4) & 7,       value index - 4
//   6-bit c, hi digit:       index = ((c ^ 0x20) + 4) >> 3,   value index - 4
//   8-bit c, lo digit:       index = c & 15,                  value index / 2
//   8-bit c, hi digit:       index = (c ^ 0x80) >> 4,         value (index - 8) / 2
// (6-bit c taken as its 6-bit field; the hi digit is floor((c + 4) / 8) and
// the lo digit c - 8 hi, in [-4, 3]; the 8-bit hi digit is floor(c / 16) and
// the lo digit c mod 16). E2M3 holds every multiple of 1/2 up to 7.5.
struct Tab16 {
    uint32_t w[4];   // entries 4 i .. 4 i + 3, one per byte
};
__constant__ Tab16 kTabE2M3[5] = {
    {{0x3A3C3E00u, 0x28303438u, 0x14100800u, 0x1E1C1A18u}},   // 4-bit codes
    {{0x28303438u, 0x14100800u, 0x00000000u, 0x00000000u}},   // 6-bit lo digits
    {{0x28303438u, 0x14100800u, 0x00000018u, 0x00000000u}},   // 6-bit hi digits
    {{0x0C080400u, 0x16141210u, 0x1B1A1918u, 0x1F1E1D1Cu}},   // 8-bit lo digits
    {{0x32343638u, 0x24282C30u, 0x0C080400u, 0x16141210u}},   // 8-bit hi digits
};

__device__ __forceinline__ uint32_t lookup16(uint32_t k, const Tab16 &T) {
    const uint32_t sel = k & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(T.w[1], T.w[0], sel);
    const uint32_t hi = __builtin_amdgcn_perm(T.w[3], T.w[2], sel);
    const uint32_t m = ((k >> 3) & 0x01010101u) * 0xFFu;
    return (hi & m) | (lo & ~m);
}

// four 6-bit codes held one per byte -> 24 contiguous bits
__device__ __forceinline__ uint32_t pack4x6(uint32_t x) {
    const uint32_t u = (x & 0x003F003Fu) | ((x >> 2) & 0x0FC00FC0u);
    return (u & 0xFFFu) | ((u >> 4) & 0xFFF000u);
}

// four 6-bit fields (24 bits) -> one per byte
__device__ __forceinline__ uint32_t spread6(uint32_t g) {
    return (g & 0x3Fu) | ((g << 2) & 0x3F00u) | ((g << 4) & 0x3F0000u) | ((g << 6) & 0x3F000000u);
}

// One workgroup writes one (group, stage) record: thread t takes row t mod 64
// and slot q = t / 64 (step j = q / 2, k-half h = q mod 2), i.e. one block of
// 32 elements. (Staging the stage's 64 rows through LDS with coalesced
// loads first measured slower.)
__global__ __launch_bounds__(256) void k_mx_prep(QView A, QView W, int64_t M, int64_t N, int64_t groups_a,
                                                 int32_t n8, int32_t n6, int32_t n4, XPlan P,
                                                 int8_t *__restrict__ outA, int8_t *__restrict__ outW) {
    // records in (matrix, group, stage) order; workgroups are dealt
    // round-robin to the 8 XCDs, so XCD x takes the x-th eighth of the
    // records: consecutive stages of a group (the same rows, adjacent bytes
    // of each 128-byte line) then share one L2
    int64_t t = blockIdx.x;
    if (gridDim.x % 8 == 0) t = (t % 8) * (gridDim.x / 8) + t / 8;
    const bool is_a = t < groups_a * P.ns;
    const int64_t id = is_a ? t : t - groups_a * P.ns;
    const int64_t g = id / P.ns;
    const int32_t s = (int32_t)(id % P.ns);
    const QView &Q = is_a ? A : W;
    const int64_t R = is_a ? M : N;
    int8_t *rec = (is_a ? outA : outW) + (g * P.ns + s) * kXRec;
    const int rho = threadIdx.x & 63, q = threadIdx.x >> 6, j = q >> 1, h = q & 1;

    int cls, bl;
    int32_t nseg, base;
    if (s < P.p8) {
        cls = 8; bl = 2 * s + h; nseg = n8; base = 0;
    } else if (s < P.nd) {
        cls = 6; bl = 2 * (s - P.p8) + h; nseg = n6; base = n8;
    } else {
        cls = 4; bl = 2 * (2 * (s - P.nd) + j) + h; nseg = n4; base = n8 + n6;
    }
    const int64_t r = g * 64 + rho;
    const bool real = bl < nseg && r < R;
    uint32_t w[6] = {0, 0, 0, 0, 0, 0};
    uint32_t sb = 0;
    if (real) {
        const int64_t b = base + bl;
        const uint32_t byte = Q.sc[r * Q.lds + b];
        const uint32_t add = cls == 4 ? 0u : (cls == 6 ? (j == 0 ? 3u : 0u) : (j == 0 ? 5u : 1u));
        sb = byte == 0xFFu ? 0xFFu : byte + add;
        uint32_t k[8];   // table indices, four elements per word, element order
        int tab;
        if (cls == 4) {
            const uint2 *p = reinterpret_cast<const uint2 *>(Q.q4 + r * Q.ld4 + 16 * (b - n8 - n6));
            const uint2 x0 = p[0], x1 = p[1];
            const uint32_t x[4] = {x0.x, x0.y, x1.x, x1.y};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t ev = (x[d] & 0x0F0F0F0Fu) ^ 0x08080808u, od = ((x[d] >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
                k[2 * d] = __builtin_amdgcn_perm(od, ev, 0x05010400u);
                k[2 * d + 1] = __builtin_amdgcn_perm(od, ev, 0x07030602u);
            }
            tab = 0;
        } else if (cls == 6) {
            const uint32_t *p = reinterpret_cast<const uint32_t *>(Q.q6 + r * Q.ld6 + 24 * (b - n8));
            uint32_t x[7];
#pragma unroll
            for (int d = 0; d < 6; ++d) x[d] = p[d];
            x[6] = 0;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const int bit = 24 * t;
                const uint32_t f = spread6(__builtin_amdgcn_alignbit(x[(bit >> 5) + 1], x[bit >> 5], bit & 31));
                k[t] = j == 0 ? (((f ^ 0x20202020u) + 0x04040404u) >> 3) & 0x0F0F0F0Fu
                              : ((f & 0x07070707u) + 0x04040404u) & 0x07070707u;
            }
            tab = j == 0 ? 2 : 1;
        } else {
            const uint4 *p = reinterpret_cast<const uint4 *>(Q.q8 + r * Q.ld8 + 32 * b);
            const uint4 x0 = p[0], x1 = p[1];
            const uint32_t x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
            for (int t = 0; t < 8; ++t)
                k[t] = j == 0 ? ((x[t] ^ 0x80808080u) >> 4) & 0x0F0F0F0Fu : x[t] & 0x0F0F0F0Fu;
            tab = j == 0 ? 4 : 3;
        }
        const Tab16 T = kTabE2M3[tab];
        uint32_t gq[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) gq[t] = pack4x6(lookup16(k[t], T));
        w[0] = gq[0] | (gq[1] << 24);
        w[1] = (gq[1] >> 8) | (gq[2] << 16);
        w[2] = (gq[2] >> 16) | (gq[3] << 8);
        w[3] = gq[4] | (gq[5] << 24);
        w[4] = (gq[5] >> 8) | (gq[6] << 16);
        w[5] = (gq[6] >> 16) | (gq[7] << 8);
    }
    *reinterpret_cast<uint4 *>(rec + (3 * j + h) * 1024 + rho * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2 *>(rec + (3 * j + 2) * 1024 + h * 512 + rho * 8) = make_uint2(w[4], w[5]);
    rec[kXCode + rho * 4 + q] = (int8_t)sb;
}

// A stage of the workgroup tile in LDS: the code parts of the eight group
// records (A groups 0..3, W groups 0..3), then the four A and the four W
// scale parts, and a 1 KiB sink. Ring of three stage slots (153 KiB of the
// CU's 160 KiB).
__shared__ __attribute__((aligned(16))) int8_t g_xring[kXRing * kXSlot];

// A stage is 50 loads of 1 KiB, straight from global memory into LDS: load
// L < 48 is code chunk L mod 6 of group L / 6; load 48 the scale parts of
// the four A groups (16 lanes each), load 49 those of the four W groups.
// Wave w issues loads w, w + 4, w + 8, ..., 13 per wave: loads 50 and 51
// (the last of waves 2 and 3) repeat the wave's first load into the slot's sink,
// so that every wave has the same count and no branch. Every source
// advances by one record per stage.
struct XDma {
    const int8_t *src[kXLoads];   // this lane's source at stage 0
    uint32_t lds[kXLoads];        // wave-uniform LDS offset in the slot
};

__device__ __forceinline__ void xdma_issue(const XDma &D, uint32_t slot, int st, int s_end) {
    const int s = st < s_end ? st : s_end - 1;   // past the end: reload the last stage
    const int64_t o = (int64_t)s * kXRec;
#pragma unroll
    for (int k = 0; k < kXLoads; ++k) dma16(D.src[k] + o, slot + D.lds[k]);
}

typedef int v2i __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) const v2i lds_v2i_t;
__device__ __forceinline__ v2i lds_v2(uint32_t a) { return *reinterpret_cast<lds_v2i_t *>((uintptr_t)a); }
typedef int v8i __attribute__((ext_vector_type(8)));

// Split over K for grids of fewer tiles than CUs: split k takes stages
// s[k] .. s[k+1] - 1 and writes its fp32 tile sums to part[k][M][N], which
// k_gemv_reduce adds in split order.
struct XSplit {
    int32_t n;        // splits (1: the tile sums go to Y)
    int32_t s[9];     // stage bounds, s[0] = 0, s[n] = all stages
};

// Workgroup: 4 waves (2 x 2), one per SIMD, tile 256 x 256; each wave owns
// 128 x 128 outputs as 4 x 4 MFMA tiles (256 fp32 sums per lane, held in
// the accumulation registers), i.e. two 64-row A groups and two 64-row W
// groups. Per 64-deep MFMA step a wave reads 8 fragments (12 KiB) for 16
// MFMAs, half the LDS bytes per MFMA of a 64 x 64 wave tile, and the
// workgroup fetches 512 operand rows per 65536 outputs instead of 384 per
// 32768. Both operands reach LDS by DMA.
__global__ __launch_bounds__(256, 1) void k_gemm_mx(const int8_t *__restrict__ PA, const int8_t *__restrict__ PW,
                                                    int64_t M, int64_t N, int64_t Mp, int64_t Np, XPlan P, XSplit SK,
                                                    float *__restrict__ Y, int64_t ldy, float *__restrict__ part) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, h = lane >> 5;

    // tile order: each XCD (workgroups are dealt round-robin to the 8 XCDs)
    // takes a contiguous run of tiles; runs sweep groups of 8 row-tiles
    const int64_t tilesM = Mp / kXBM, tilesN = Np / kXBN, ntiles = tilesM * tilesN;
    int64_t t = blockIdx.x;
    if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
    const int64_t per_group = 8 * tilesN;
    const int64_t gid = t / per_group, first_m = gid * 8;
    const int64_t gsz = tilesM - first_m < 8 ? tilesM - first_m : 8;
    const int64_t tm = first_m + (t % per_group) % gsz, tn = (t % per_group) / gsz;
    const int64_t m0 = tm * kXBM, n0 = tn * kXBN;
    const int ns = P.ns, nd = P.nd;
    const int s0 = __builtin_amdgcn_readfirstlane(SK.s[blockIdx.y]);
    const int s1 = __builtin_amdgcn_readfirstlane(SK.s[blockIdx.y + 1]);

    // this lane's DMA sources and the wave's LDS destinations
    XDma D;
    {
        auto rec = [&](int g) -> const int8_t * {   // group record g of the tile at stage 0
            return g < kXGA ? PA + ((m0 / 64 + g) * ns) * (int64_t)kXRec
                            : PW + ((n0 / 64 + (g - kXGA)) * ns) * (int64_t)kXRec;
        };
#pragma unroll
        for (int k = 0; k < kXLoads; ++k) {
            const int L = wave + 4 * k;
            if (L < 6 * kXGroups) {
                D.src[k] = rec(L / 6) + (L % 6) * 1024 + lane * 16;
                D.lds[k] = (uint32_t)((L / 6) * kXCode + (L % 6) * 1024);
            } else if (L == 6 * kXGroups) {
                D.src[k] = rec(lane >> 4) + kXCode + (lane & 15) * 16;
                D.lds[k] = kXScA;
            } else if (L == 6 * kXGroups + 1) {
                D.src[k] = rec(kXGA + ((lane >> 4) & 3)) + kXCode + (lane & 15) * 16;
                D.lds[k] = kXScW;
            } else {   // loads 50, 51: a copy of load 0 of this wave into the sink
                D.src[k] = D.src[0];
                D.lds[k] = kXSink;
            }
        }
    }

    // LDS byte offsets (inside a slot) of this lane's pieces of fragment 0,
    // step 0 (16-byte piece, 8-byte piece, scale dword). A fragment f (0..3)
    // is group 2 wm + f / 2, rows 32 (f % 2) .. + 31 of it; W likewise with
    // wn; step j adds 3072 bytes to the code pieces.
    const uint32_t ca = (uint32_t)(2 * wm * kXCode), cw = (uint32_t)((kXGA + 2 * wn) * kXCode);
    const uint32_t sa0 = (uint32_t)(kXScA + wm * 512), sw0 = (uint32_t)(kXScW + wn * 512);
    const uint32_t lq = (uint32_t)(h * 1024 + l32 * 16), ld = (uint32_t)(2048 + h * 512 + l32 * 8),
                   ls = (uint32_t)(l32 * 4);
    auto foff_q = [](int f) { return (uint32_t)((f >> 1) * kXCode + (f & 1) * 512); };
    auto foff_d = [](int f) { return (uint32_t)((f >> 1) * kXCode + (f & 1) * 256); };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jw = 0; jw < 4; ++jw)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jw][e] = 0.f;

    // the fragments and scale bytes of one MFMA step (A rows, W rows)
    struct Frags {
        v8i a[4], w[4];
        int sa[4], sw[4];
    };
    // fragment u of a step (u < 4: A fragment u, else W fragment u - 4):
    // its 16-byte and 8-byte pieces; scale bytes: one dword per row holds
    // (step 0, k-half 0/1, step 1, k-half 0/1); the MFMA reads bits 0..7 of
    // its scale operand, so the lane shifts its byte (2 j + h) down
    auto read_frag = [&](uint32_t slot, int j, int u, Frags &F) {
        const uint32_t base = slot + (u < 4 ? ca : cw) + j * 3072;
        const int f = u & 3;
        const v4i pq = lds_v4(base + lq + foff_q(f));
        const v2i pd = lds_v2(base + ld + foff_d(f));
        const v8i x = v8i{pq[0], pq[1], pq[2], pq[3], pd[0], pd[1], 0, 0};
        if (u < 4) F.a[f] = x;
        else F.w[f] = x;
    };
    auto read_scale = [&](uint32_t slot, int u, int (&sa)[4], int (&sw)[4]) {
        if (u < 4) sa[u] = lds_i32(slot + sa0 + ls + u * 128);
        else sw[u - 4] = lds_i32(slot + sw0 + ls + (u - 4) * 128);
    };
    auto set_scales = [&](int j, const int (&sa)[4], const int (&sw)[4], Frags &F) {
        const int sh = 16 * j + 8 * h;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            F.sa[f] = (int)((uint32_t)sa[f] >> sh);
            F.sw[f] = (int)((uint32_t)sw[f] >> sh);
        }
    };
    auto mma1 = [&](const Frags &X, const Frags &Z, int k) {   // output tile k: A fragment k / 4, W fragment k % 4
        const int i = k >> 2, jw = k & 3;
        acc[i][jw] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(X.a[i], Z.w[jw], acc[i][jw], 2, 2, 0, X.sa[i],
                                                                    0, Z.sw[jw]);
    };
    auto mma = [&](const Frags &X, const Frags &Z) {   // X: A fragments, Z: W fragments
#pragma unroll
        for (int k = 0; k < 16; ++k) mma1(X, Z, k);
    };

    // Software pipeline over MFMA steps, two fragment sets (F0: step 0, F1:
    // step 1 of the current stage), with the memory instructions spread
    // between the MFMAs so that the matrix core never waits for a burst of
    // them (one wave per SIMD: no other wave fills its gaps). Stage s:
    //   phase 1: the MFMAs that need only F0 (A0 W0, or hi*hi), one F1
    //            fragment read after each of the first eight; then, on a
    //            digit stage, hi*lo and lo*hi;
    //   wait for this wave's loads of stage s+1; barrier (all of stage s+1
    //   has landed, every wave has finished reading stage s);
    //   phase 2: the MFMAs of F1 (A1 W1, or lo*lo), with the DMA of stage
    //            s+3 into the slot of stage s and the reads of stage s+1's
    //            scales and F0 between them.
    // Ring of three slots, stage k in slot k % 3. After the last stage the
    // reads of the following slot still run (in bounds, result unused), which
    // keeps the loop free of branches.
    const uint32_t ring = lds_addr(g_xring);
    auto slot_of = [&](int s) { return ring + (uint32_t)((s % kXRing) * kXSlot); };
#pragma unroll
    for (int k = 0; k < kXRing; ++k) xdma_issue(D, slot_of(s0 + k), s0 + k, s1);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kXLoads));
    lds_barrier();
    Frags F0, F1;
    int scA[4], scW[4];   // scale dwords of the current stage
#pragma unroll
    for (int u = 0; u < 8; ++u) read_scale(slot_of(s0), u, scA, scW);
#pragma unroll
    for (int u = 0; u < 8; ++u) read_frag(slot_of(s0), 0, u, F0);
    set_scales(0, scA, scW, F0);

    auto phase1 = [&](int s) {
        const uint32_t cur = slot_of(s);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            mma1(F0, F0, k);
            if (k < 8) read_frag(cur, 1, k, F1);
            __builtin_amdgcn_sched_barrier(0);
        }
        set_scales(1, scA, scW, F1);
    };
    auto phase2 = [&](int s) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kXLoads));
        lds_barrier();
        const uint32_t cur = slot_of(s), nxt = slot_of(s + 1);
        const int sd = s + kXRing < s1 ? s + kXRing : s1 - 1;   // past the end: reload the last stage
        const int64_t o = (int64_t)sd * kXRec;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            mma1(F1, F1, k);
            if (k < kXLoads) dma16(D.src[k] + o, cur + D.lds[k]);
            if (k < 8) read_scale(nxt, k, scA, scW);
            else read_frag(nxt, 0, k - 8, F0);
            __builtin_amdgcn_sched_barrier(0);
        }
        set_scales(0, scA, scW, F0);
    };
    int s = s0;
    const int dend = nd < s1 ? nd : s1;
    for (; s < dend; ++s) {   // digit stages: hi and lo steps of a 6/8-bit pair
        phase1(s);
        mma(F0, F1);
        mma(F1, F0);
        phase2(s);
    }
    for (; s < s1; ++s) {   // two 4-bit pairs
        phase1(s);
        phase2(s);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA outstanding at exit
    float *out = Y;
    int64_t ldo = ldy;
    if (SK.n > 1) {   // this split's sums into part[split][M][N]
        out = part + (int64_t)blockIdx.y * M * N;
        ldo = N;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jw = 0; jw < 4; ++jw) {
            const int64_t col = n0 + wn * 128 + jw * 32 + l32;
            if (col >= N) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = m0 + wm * 128 + i * 32 + 8 * q + 4 * h + r;
                    if (row < M) out[row * ldo + col] = acc[i][jw][4 * q + r];
                }
        }
}

// ---------------------------------------------------------------------------
// The same product on 256 x 128 workgroup tiles of eight waves (64 x 64 per
// wave), for grids of 64 to 255 tiles of 256 x 256: there the larger tile
// would leave CUs idle or need a K split and its reduction, while the
// smaller tile fills the chip in one pass. Same prepared records.
namespace ntile {
constexpr int kXBN = 128;                       // workgroup tile: 256 A rows x 128 W rows
constexpr int kXGroups = kXBM / 64 + kXBN / 64;
// LDS image of one stage of the workgroup tile: the code parts of the six
// group records (A groups 0..3, W groups 0..1), then the A scale parts, the
// W scale parts, and 1.5 KiB that only absorbs the copies that keep every
// wave's load count equal (see xdma_issue)
constexpr int kXScA = kXGroups * kXCode;        // 36864
constexpr int kXScW = kXScA + (kXBM / 64) * 256; // 37888
constexpr int kXSink = kXScW + 512;             // 38400
constexpr int kXSlot = kXSink + 1536;           // 39936
constexpr int kXLoads = 5;                      // loads per wave and stage

// the ring of four stage slots
__shared__ __attribute__((aligned(16))) int8_t g_xring[4 * kXSlot];

// A stage is 40 loads of 1 KiB, straight from global memory into LDS, five
// per wave (no branch, and the same wait count in every wave): load L =
// 5 wave + k is code chunk L mod 6 of group L / 6 for L < 36; load 36 the
// scale parts of the four A groups (16 lanes each); load 37 those of the two
// W groups (lanes 32..63 repeat lanes 0..31 into the sink); loads 38, 39
// repeat load 37 into the sink. Every source advances by one record per
// stage.
struct XDma {
    const int8_t *src[kXLoads];   // this lane's source at stage 0
    uint32_t lds[kXLoads];        // wave-uniform LDS offset in the slot
};

__device__ __forceinline__ void xdma_issue(const XDma &D, uint32_t slot, int st, int ns) {
    const int s = st < ns ? st : ns - 1;   // past the end: reload the last stage
    const int64_t o = (int64_t)s * kXRec;
#pragma unroll
    for (int k = 0; k < kXLoads; ++k) dma16(D.src[k] + o, slot + D.lds[k]);
}


// Workgroup: 8 waves (4 x 2), tile 256 x 128; each wave owns 64 x 64 outputs
// as 2 x 2 MFMA tiles, i.e. one 64-row A group and one 64-row W group. Both
// operands reach LDS by DMA, through a ring of four stage slots. The fp6
// matrix cores outrun the LDS here: a 4-bit step reads 6 KiB of fragments
// per wave for 4 MFMAs, so the 4-bit stages are bound by LDS reads and the
// 6/8-bit stages (four MFMAs per fragment set) by the matrix cores.
// (Loading A straight into registers instead, with 4 waves of 64 x 128,
// halves the LDS reads but measured slower: the vector memory path then
// carries the same bytes.)
__global__ __launch_bounds__(512, 1) void k_gemm_mx_n(const int8_t *__restrict__ PA, const int8_t *__restrict__ PW,
                                                    int64_t M, int64_t N, int64_t Mp, int64_t Np, XPlan P,
                                                    float *__restrict__ Y, int64_t ldy) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, h = lane >> 5;

    // tile order: each XCD (workgroups are dealt round-robin to the 8 XCDs)
    // takes a contiguous run of tiles; runs sweep groups of 8 row-tiles
    const int64_t tilesM = Mp / kXBM, tilesN = Np / kXBN, ntiles = tilesM * tilesN;
    int64_t t = blockIdx.x;
    if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
    const int64_t per_group = 8 * tilesN;
    const int64_t gid = t / per_group, first_m = gid * 8;
    const int64_t gsz = tilesM - first_m < 8 ? tilesM - first_m : 8;
    const int64_t tm = first_m + (t % per_group) % gsz, tn = (t % per_group) / gsz;
    const int64_t m0 = tm * kXBM, n0 = tn * kXBN;
    const int ns = P.ns, nd = P.nd;

    // this lane's DMA sources and the wave's LDS destinations
    XDma D;
    {
        auto rec = [&](int g) -> const int8_t * {   // group record g of the tile at stage 0
            return g < kXBM / 64 ? PA + ((m0 / 64 + g) * ns) * (int64_t)kXRec
                                 : PW + ((n0 / 64 + (g - kXBM / 64)) * ns) * (int64_t)kXRec;
        };
#pragma unroll
        for (int k = 0; k < kXLoads; ++k) {
            const int L = kXLoads * wave + k;
            if (L < 6 * kXGroups) {
                D.src[k] = rec(L / 6) + (L % 6) * 1024 + lane * 16;
                D.lds[k] = (uint32_t)((L / 6) * kXCode + (L % 6) * 1024);
            } else if (L == 6 * kXGroups) {
                D.src[k] = rec(lane >> 4) + kXCode + (lane & 15) * 16;
                D.lds[k] = kXScA;
            } else {
                D.src[k] = rec(kXBM / 64 + ((lane >> 4) & 1)) + kXCode + (lane & 15) * 16;
                D.lds[k] = L == 6 * kXGroups + 1 ? kXScW : kXSink + 512;
            }
        }
    }

    // LDS byte offsets (inside a slot) of this lane's pieces of fragment 0,
    // step 0 (16-byte piece, 8-byte piece, scale dword); fragment i adds 512
    // / 256 / 128 bytes, step j adds 3072 / 3072 / 0. Addresses are formed as
    // slot base + lane offset + immediate, so one register per piece kind
    // serves every slot and step.
    const uint32_t ca = (uint32_t)(wm * kXCode), cw = (uint32_t)((kXBM / 64 + wn) * kXCode);
    const uint32_t sa0 = (uint32_t)(kXScA + wm * 256), sw0 = (uint32_t)(kXScW + wn * 256);
    const uint32_t lq = (uint32_t)(h * 1024 + l32 * 16), ld = (uint32_t)(2048 + h * 512 + l32 * 8),
                   ls = (uint32_t)(l32 * 4);

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jw = 0; jw < 2; ++jw)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][jw][e] = 0.f;

    // the fragments and scale bytes of one MFMA step (A rows, W rows)
    struct Frags {
        v8i a[2], w[2];
        int sa[2], sw[2];
    };
    // scale bytes: one dword per row holds (step 0, k-half 0/1, step 1, k-half
    // 0/1); the MFMA reads bits 0..7 of its scale operand, so the lane shifts
    // its byte (2 j + h) down and leaves the others above it
    auto read_scales = [&](uint32_t slot, int (&sa)[2], int (&sw)[2]) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            sa[i] = lds_i32(slot + sa0 + ls + i * 128);
            sw[i] = lds_i32(slot + sw0 + ls + i * 128);
        }
    };
    auto read_step = [&](uint32_t slot, int j, const int (&sa)[2], const int (&sw)[2], Frags &F) {
        const uint32_t qa = slot + ca + lq, da = slot + ca + ld;
        const uint32_t qw = slot + cw + lq, dw = slot + cw + ld;
        const int sh = 16 * j + 8 * h;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const v4i pa = lds_v4(qa + i * 512 + j * 3072), pw = lds_v4(qw + i * 512 + j * 3072);
            const v2i ra = lds_v2(da + i * 256 + j * 3072), rw = lds_v2(dw + i * 256 + j * 3072);
            F.a[i] = v8i{pa[0], pa[1], pa[2], pa[3], ra[0], ra[1], 0, 0};
            F.w[i] = v8i{pw[0], pw[1], pw[2], pw[3], rw[0], rw[1], 0, 0};
            F.sa[i] = (int)((uint32_t)sa[i] >> sh);
            F.sw[i] = (int)((uint32_t)sw[i] >> sh);
        }
    };
    auto mma = [&](const Frags &X, const Frags &Z) {   // X: A fragments, Z: W fragments
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jw = 0; jw < 2; ++jw)
                acc[i][jw] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(X.a[i], Z.w[jw], acc[i][jw], 2, 2, 0,
                                                                            X.sa[i], 0, Z.sw[jw]);
    };

    // Software pipeline over MFMA steps, two fragment sets (F0: step 0, F1:
    // step 1 of the current stage). Stage s: read F1; MFMAs that need only
    // F0 and F1 (single stage: A0 W0; digit stage: hi*hi, hi*lo, lo*hi);
    // wait for this wave's loads of stage s+1; barrier (all of stage s+1 has
    // landed, every wave has finished reading stage s); issue stage s+4 into
    // the slot of stage s; read F0 of stage s+1; the last MFMAs of stage s
    // (A1 W1, or lo*lo), which overlap those reads. Ring of four slots,
    // stage k in slot k % 4. After the last stage the reads of the following
    // slot still run (in bounds, result unused), which keeps the loop free
    // of branches.
    const uint32_t ring = lds_addr(g_xring);
#pragma unroll
    for (int k = 0; k < 4; ++k) xdma_issue(D, ring + k * kXSlot, k, ns);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * kXLoads));
    lds_barrier();
    Frags F0, F1;
    int scA[2], scW[2];   // scale dwords of the current stage
    read_scales(ring, scA, scW);
    read_step(ring, 0, scA, scW, F0);
    auto next = [&](int s) {
        __builtin_amdgcn_sched_barrier(0);   // the MFMAs above issue before the wait
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kXLoads));
        lds_barrier();
        xdma_issue(D, ring + (uint32_t)((s & 3) * kXSlot), s + 4, ns);
        const uint32_t nxt = ring + (uint32_t)(((s + 1) & 3) * kXSlot);
        read_scales(nxt, scA, scW);
        read_step(nxt, 0, scA, scW, F0);
    };
    int s = 0;
    for (; s < nd; ++s) {   // digit stages: hi and lo steps of a 6/8-bit pair
        read_step(ring + (uint32_t)((s & 3) * kXSlot), 1, scA, scW, F1);
        mma(F0, F0);
        mma(F0, F1);
        mma(F1, F0);
        next(s);
        mma(F1, F1);
    }
    for (; s < ns; ++s) {   // two 4-bit pairs
        read_step(ring + (uint32_t)((s & 3) * kXSlot), 1, scA, scW, F1);
        mma(F0, F0);
        next(s);
        mma(F1, F1);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA outstanding at exit
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jw = 0; jw < 2; ++jw) {
            const int64_t col = n0 + wn * 64 + jw * 32 + l32;
            if (col >= N) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = m0 + wm * 64 + i * 32 + 8 * q + 4 * h + r;
                    if (row < M) Y[row * ldy + col] = acc[i][jw][4 * q + r];
                }
        }
}

}  // namespace ntile

// ---------------------------------------------------------------------------
// Decode path (M <= kGemvMaxRows tokens): stream W once from HBM. Up to
// kGemvVecRows tokens use the vector kernel below (k_gemv), more tokens the
// matrix-core kernel further down (k_decode).
//
// k_gemv: a wavefront owns 64 W rows and one slice of one width class (two
// chunks: 8 blocks of 8 or 6 bits, or 16 blocks of 4 bits). It issues every
// load of the slice at once: the rows' and tokens' scale bytes, then the
// codes, each row group of 8 rows with one coalesced 16-byte load per lane
// (lane e of a row reads one piece of it: a whole 4-bit block or half an
// 8- or 6-bit block), and the tokens' matching pieces. No code bytes pass
// through LDS, so occupancy is set by registers and each wave keeps 16 KiB
// of W in flight. Block dot products are exact in int32: 4-bit x 4-bit with
// v_dot8_i32_i4 on the packed nibbles, 8-bit with v_dot4_i32_i8, 6-bit after
// widening both sides to bytes (code * 4, the factor 16 folded into the
// scale); the two lanes holding the halves of an 8- or 6-bit block add their
// sums (one DPP add). Each block adds I_b * 2^(sa+sw) to an fp32 accumulator
// per row and token; the eight lanes of a row are summed in a fixed butterfly
// at the end. Slices write partial rows that a second kernel adds in slice
// order, so the result does not depend on scheduling.
constexpr int kGemvMaxRows = 32;   // decode path: up to 32 tokens
constexpr int kGemvVecRows = 8;    // up to 8 tokens on the vector ALU, above on the matrix cores
constexpr int kGemvPitch = 144;     // 8-bit and 4-bit tiles: 128 bytes + 16 (conflict-free b128 reads)
constexpr int kGemvPitch6 = 104;    // 6-bit tile: 96 bytes + 8 (conflict-free b64 reads)
constexpr int kGemvTile = 64 * kGemvPitch;

__device__ __forceinline__ uint32_t wide6(uint32_t g) {   // four 6-bit fields -> four bytes (code * 4)
    return ((g << 2) & 0xFCu) | ((g << 4) & 0xFC00u) | ((g << 6) & 0xFC0000u) | ((g << 8) & 0xFC000000u);
}

struct GemvChunk {
    int32_t cls;    // 8, 6 or 4
    int32_t gb;     // first block (global index)
    int32_t pb;     // first block within its class plane
    int32_t nblk;   // blocks in the chunk
};

// Coalesced fetch of one chunk of codes for 64 rows into registers. Lane
// roles (row within a group of 8 rows, piece of the row) are fixed; load i
// moves to the next group, so every address is a uniform base plus a 32-bit
// lane offset. Every width takes one 16-byte load per row group:
//   4-bit: 8 lanes x 16 bytes per row (lane e: block e of the chunk)
//   8-bit: 8 lanes x 16 bytes per row (lane e: half e & 1 of block e / 2)
//   6-bit: 8 lanes x 12 bytes per row (lane e: half e & 1 of block e / 2);
//          the load covers bytes 0..15 of the block for the first half and
//          bytes 8..23 for the second, so it never leaves the block, and
//          piece6 picks the three words of the half.
// Row group i lands in R[4 i .. 4 i + 3]. Pieces of rows past N or of
// blocks past the chunk re-read the first bytes of the tile's first row
// (always valid) instead of branching; they are never used.
__device__ __forceinline__ void gemv_fetch(const QView &W, int64_t row0, int32_t rows_left, const GemvChunk &c,
                                           int lane, uint32_t R[32]) {
    const int rs = lane >> 3, e = lane & 7;
    const bool c4 = c.cls == 4, c6 = c.cls == 6;
    const bool ok = (c4 ? e : e >> 1) < c.nblk;
    const int64_t ld = c4 ? W.ld4 : c6 ? W.ld6 : W.ld8;
    const uint8_t *base = (c4 ? W.q4 : c6 ? W.q6 : reinterpret_cast<const uint8_t *>(W.q8)) + row0 * ld;
    const uint32_t pos = c4 ? 16 * (c.pb + e) : c6 ? 24 * c.pb + 12 * e - 4 * (e & 1) : 32 * c.pb + 16 * e;
    const uint32_t off = (uint32_t)(rs * ld) + pos, step = (uint32_t)(8 * ld);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t o = (ok && rs + 8 * i < rows_left) ? off + i * step : 0u;
        const uint4 v = *reinterpret_cast<const uint4 *>(base + o);
        R[4 * i] = v.x; R[4 * i + 1] = v.y; R[4 * i + 2] = v.z; R[4 * i + 3] = v.w;
    }
}

// the three words of a 6-bit half block held as a 16-byte load (see gemv_fetch)
__device__ __forceinline__ void piece6(const uint32_t r[4], bool second, uint32_t w[3]) {
    w[0] = second ? r[1] : r[0];
    w[1] = second ? r[2] : r[1];
    w[2] = second ? r[3] : r[2];
}

// Registers -> LDS tile (row pitch kGemvPitch, or kGemvPitch6 for 6-bit),
// mirroring the lane roles of gemv_fetch.
__device__ __forceinline__ void gemv_stage(uint8_t *tile, int cls, int lane, const uint32_t R[32]) {
    const int rs = lane >> 3, e = lane & 7;
    if (cls == 6) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t w[3];
            piece6(&R[4 * i], e & 1, w);
            uint32_t *q = reinterpret_cast<uint32_t *>(tile + (rs + 8 * i) * kGemvPitch6 + 12 * e);
            q[0] = w[0]; q[1] = w[1]; q[2] = w[2];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<uint4 *>(tile + (rs + 8 * i) * kGemvPitch + 16 * e) =
                make_uint4(R[4 * i], R[4 * i + 1], R[4 * i + 2], R[4 * i + 3]);
    }
}

// Token pieces of one chunk: the same bytes of every token row as the lane's
// W piece, loaded the same way (see gemv_fetch). Pieces past the chunk
// re-read the row's first bytes.
template <int MT>
__device__ __forceinline__ void gemv_fetch_tok(const int8_t *__restrict__ a8, int64_t la8,
                                               const uint8_t *__restrict__ a6, int64_t la6,
                                               const uint8_t *__restrict__ a4, int64_t la4, int32_t M,
                                               const GemvChunk &c, int lane, uint32_t T[MT][4]) {
    const int e = lane & 7;
    const bool c4 = c.cls == 4, c6 = c.cls == 6;
    const bool ok = (c4 ? e : e >> 1) < c.nblk;
    const int64_t ld = c4 ? la4 : c6 ? la6 : la8;
    const uint8_t *base = c4 ? a4 : c6 ? a6 : reinterpret_cast<const uint8_t *>(a8);
    const uint32_t pos = !ok ? 0u : c4 ? 16 * (c.pb + e) : c6 ? 24 * c.pb + 12 * e - 4 * (e & 1) : 32 * c.pb + 16 * e;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t >= M) continue;
        const uint4 v = *reinterpret_cast<const uint4 *>(base + t * ld + pos);
        T[t][0] = v.x; T[t][1] = v.y; T[t][2] = v.z; T[t][3] = v.w;
    }
}

// 16 6-bit codes (three words) -> four words of bytes (code * 4)
__device__ __forceinline__ void wide6x16(const uint32_t w[3], uint32_t b[4]) {
    b[0] = wide6(w[0]);
    b[1] = wide6(__builtin_amdgcn_alignbit(w[1], w[0], 24));
    b[2] = wide6(__builtin_amdgcn_alignbit(w[2], w[1], 16));
    b[3] = wide6(w[2] >> 8);
}

// v summed over the eight lanes of its group (lane ^ 4, ^ 2, ^ 1); every
// lane of the group ends with the same value
__device__ __forceinline__ float sum8(float v) {
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));           // xor 4
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)); // xor 2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)); // xor 1
    return v;
}

// Slices of the vector kernel: each width class is cut into runs of
// kVecChunks chunks (8- and 6-bit chunks hold 4 blocks, 4-bit chunks 8), in
// the order 8-bit, 6-bit, 4-bit; slice s of a wave is blockIdx.y.
constexpr int kVecChunks = 2;
constexpr int kVecScW = 6;   // dwords of staged scale bytes per row (20 used)

struct VecSlices {
    int32_t s8, s6, s4;
};

__host__ __device__ inline VecSlices vec_slices(int32_t n8, int32_t n6, int32_t n4) {
    const int32_t p8 = 4 * kVecChunks, p4 = 8 * kVecChunks;
    return VecSlices{(n8 + p8 - 1) / p8, (n6 + p8 - 1) / p8, (n4 + p4 - 1) / p4};
}

// slice s -> width class, first block (global and within the class plane)
// and block count
__device__ __forceinline__ GemvChunk vec_slice(int32_t s, int32_t n8, int32_t n6, int32_t n4, VecSlices S) {
    GemvChunk c;
    const int32_t p8 = 4 * kVecChunks, p4 = 8 * kVecChunks;
    if (s < S.s8) {
        c.cls = 8; c.pb = s * p8; c.gb = c.pb; c.nblk = min(p8, n8 - c.pb);
    } else if (s < S.s8 + S.s6) {
        c.cls = 6; c.pb = (s - S.s8) * p8; c.gb = n8 + c.pb; c.nblk = min(p8, n6 - c.pb);
    } else {
        c.cls = 4; c.pb = (s - S.s8 - S.s6) * p4; c.gb = n8 + n6 + c.pb; c.nblk = min(p4, n4 - c.pb);
    }
    return c;
}

// chunk j of a slice
__device__ __forceinline__ GemvChunk vec_chunk(const GemvChunk &sl, int j) {
    const int32_t bpc = sl.cls == 4 ? 8 : 4;
    GemvChunk c = sl;
    c.gb += j * bpc;
    c.pb += j * bpc;
    c.nblk = min(bpc, max(0, sl.nblk - j * bpc));
    return c;
}

// One chunk against the tokens: lane (rs, e) dots its piece of rows
// rs + 8 g with the tokens' piece. 4-bit pieces are whole blocks; 8- and
// 6-bit pieces are half blocks, whose integer sums the two lanes of a pair
// add before the even lane scales the block sum. scw / sca: the slice's
// staged scale bytes (W rows, tokens), chunk block k at byte o + k.
template <int MT, int CLS>
__device__ __forceinline__ void vec_dot(const GemvChunk &c, int32_t o, int32_t M, int lane, const uint32_t R[32],
                                        const uint32_t T[MT][4], const uint8_t *scw, const uint8_t *sca,
                                        float acc[MT][8]) {
    const int rs = lane >> 3, e = lane & 7;
    const int pblk = CLS == 4 ? e : e >> 1;
    const bool on = pblk < c.nblk && (CLS == 4 || (e & 1) == 0);
    const int col = on ? o + pblk : 0;
    float sw[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) sw[g] = e8m0_to_f32(scw[(rs + 8 * g) * 4 * kVecScW + col]);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t >= M) break;
        const float sa = e8m0_to_f32(sca[t * 4 * kVecScW + col]) * (CLS == 6 ? 0.0625f : 1.0f);
        uint32_t ab[4];
        if (CLS == 6) {
            uint32_t aw[3];
            piece6(T[t], e & 1, aw);
            wide6x16(aw, ab);
        }
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            int d;
            if (CLS == 4) {
                d = __builtin_amdgcn_sdot8((int)T[t][0], (int)R[4 * g], 0, false);
                d = __builtin_amdgcn_sdot8((int)T[t][1], (int)R[4 * g + 1], d, false);
                d = __builtin_amdgcn_sdot8((int)T[t][2], (int)R[4 * g + 2], d, false);
                d = __builtin_amdgcn_sdot8((int)T[t][3], (int)R[4 * g + 3], d, false);
            } else if (CLS == 8) {
                d = __builtin_amdgcn_sdot4((int)T[t][0], (int)R[4 * g], 0, false);
                d = __builtin_amdgcn_sdot4((int)T[t][1], (int)R[4 * g + 1], d, false);
                d = __builtin_amdgcn_sdot4((int)T[t][2], (int)R[4 * g + 2], d, false);
                d = __builtin_amdgcn_sdot4((int)T[t][3], (int)R[4 * g + 3], d, false);
                d += __builtin_amdgcn_mov_dpp(d, 0xB1, 0xF, 0xF, true);
            } else {
                uint32_t wb[4], ww[3];
                piece6(&R[4 * g], e & 1, ww);
                wide6x16(ww, wb);
                d = __builtin_amdgcn_sdot4((int)ab[0], (int)wb[0], 0, false);
                d = __builtin_amdgcn_sdot4((int)ab[1], (int)wb[1], d, false);
                d = __builtin_amdgcn_sdot4((int)ab[2], (int)wb[2], d, false);
                d = __builtin_amdgcn_sdot4((int)ab[3], (int)wb[3], d, false);
                d += __builtin_amdgcn_mov_dpp(d, 0xB1, 0xF, 0xF, true);
            }
            acc[t][g] = __builtin_fmaf((float)d, on ? sa * sw[g] : 0.f, acc[t][g]);
        }
    }
}

// The body of k_gemv for one width class: every load of the slice is issued
// first (scale bytes, then the chunks' codes), then the chunks are computed
// in order as their loads land.
template <int MT, int CLS>
__device__ __forceinline__ void vec_body(const int8_t *__restrict__ a8, int64_t la8, const uint8_t *__restrict__ a6,
                                         int64_t la6, const uint8_t *__restrict__ a4, int64_t la4,
                                         const uint8_t *__restrict__ asc, int64_t las, const QView &W, int32_t M,
                                         int64_t N, int32_t nb, const GemvChunk &sl, uint32_t *scw_s,
                                         uint32_t *sca_s, float *__restrict__ out, int64_t ldo) {
    const int lane = threadIdx.x;
    const int64_t row0 = (int64_t)blockIdx.x * 64;
    const int32_t rows_left = N - row0 < 64 ? (int32_t)(N - row0) : 64;

    // scale bytes of the slice: five dwords from the dword holding block gb
    // (indices clamped to the row's last dword); lane r: W row r, lanes
    // 5 t + k: dword k of token t
    const int32_t d0 = sl.gb >> 2, dl = (nb - 1) >> 2;
    uint32_t vw[5], va = 0;
    {
        const uint32_t *sp = reinterpret_cast<const uint32_t *>(W.sc + (row0 + (lane < rows_left ? lane : 0)) * W.lds);
#pragma unroll
        for (int k = 0; k < 5; ++k) vw[k] = sp[min(d0 + k, dl)];
        const int t = lane / 5, k = lane - 5 * t;
        if (t < MT && t < M) va = reinterpret_cast<const uint32_t *>(asc + t * las)[min(d0 + k, dl)];
    }
    GemvChunk ch[kVecChunks];
    uint32_t R[kVecChunks][32], T[kVecChunks][MT][4];
#pragma unroll
    for (int j = 0; j < kVecChunks; ++j) {
        ch[j] = vec_chunk(sl, j);
        gemv_fetch(W, row0, rows_left, ch[j], lane, R[j]);
        gemv_fetch_tok<MT>(a8, la8, a6, la6, a4, la4, M, ch[j], lane, T[j]);
    }
#pragma unroll
    for (int k = 0; k < 5; ++k) scw_s[lane * kVecScW + k] = vw[k];
    if (lane < 5 * MT) sca_s[(lane / 5) * kVecScW + lane % 5] = va;
    __syncthreads();

    float acc[MT][8];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int g = 0; g < 8; ++g) acc[t][g] = 0.f;
    const uint8_t *scw = reinterpret_cast<const uint8_t *>(scw_s);
    const uint8_t *sca = reinterpret_cast<const uint8_t *>(sca_s);
#pragma unroll
    for (int j = 0; j < kVecChunks; ++j)
        vec_dot<MT, CLS>(ch[j], (sl.gb & 3) + (ch[j].gb - sl.gb), M, lane, R[j], T[j], scw, sca, acc);

    // sum each row over its eight lanes; lane (rs, e) then writes row rs + 8 e
    const int rs = lane >> 3, e = lane & 7;
    const int64_t n = row0 + rs + 8 * e;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        if (t >= M) break;
        float v = 0.f;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const float s = sum8(acc[t][g]);
            v = e == g ? s : v;
        }
        if (n < N) out[t * ldo + n] = v;
    }
}

template <int MT>
__global__ __launch_bounds__(64) void k_gemv(const int8_t *__restrict__ a8, int64_t la8,
                                             const uint8_t *__restrict__ a6, int64_t la6,
                                             const uint8_t *__restrict__ a4, int64_t la4,
                                             const uint8_t *__restrict__ asc, int64_t las, QView W, int32_t M,
                                             int64_t N, int32_t n8, int32_t n6, int32_t n4,
                                             float *__restrict__ out, int64_t ldo, int64_t slice_stride) {
    __shared__ uint32_t scw_s[64 * kVecScW];
    __shared__ uint32_t sca_s[MT * kVecScW];
    const VecSlices S = vec_slices(n8, n6, n4);
    const GemvChunk sl = vec_slice((int32_t)blockIdx.y, n8, n6, n4, S);
    const int32_t nb = n8 + n6 + n4;
    float *o = out + (int64_t)blockIdx.y * slice_stride;
    if (sl.cls == 4)
        vec_body<MT, 4>(a8, la8, a6, la6, a4, la4, asc, las, W, M, N, nb, sl, scw_s, sca_s, o, ldo);
    else if (sl.cls == 8)
        vec_body<MT, 8>(a8, la8, a6, la6, a4, la4, asc, las, W, M, N, nb, sl, scw_s, sca_s, o, ldo);
    else
        vec_body<MT, 6>(a8, la8, a6, la6, a4, la4, asc, las, W, M, N, nb, sl, scw_s, sca_s, o, ldo);
}

// ---------------------------------------------------------------------------
// One token (k_gemv_row): each W row is read by S waves of one workgroup and
// no partial rows leave the kernel. A row is walked in 16-byte pieces, in
// plane order: the two halves of each 8-bit block, the two halves of each
// 6-bit block (bytes 0..15 or 8..23 of the block, as in gemv_fetch), then
// each 4-bit block whole. Wave w of the workgroup takes rows of group w / S
// (R rows) and the pieces of split s = w % S: lane l takes pieces
// 64 J s + l + 64 j, j < J, so consecutive lanes read consecutive bytes of a
// plane row. The token's matching pieces (shared by the wave's R rows) and
// both scale bytes of every piece are loaded with the W pieces, all at once.
// Block sums are exact in int32 exactly as in vec_dot (the two lanes of a
// half-block pair add their sums; the even lane scales the block); a lane
// adds its blocks in piece order into an fp32 sum per row, the 64 lanes meet
// in a fixed butterfly, and the S splits of a row are added in split order
// through LDS.
constexpr int kRowWaves = 4;      // waves per workgroup

template <int J, int R, int S>
__global__ __launch_bounds__(64 * kRowWaves) void k_gemv_row(const int8_t *__restrict__ a8,
                                                              const uint8_t *__restrict__ a6,
                                                              const uint8_t *__restrict__ a4,
                                                              const uint8_t *__restrict__ asc, QView W, int64_t N,
                                                              int32_t n8, int32_t n6, int32_t n4,
                                                              float *__restrict__ y) {
    static_assert(kRowWaves % S == 0, "splits of a row must divide the workgroup");
    __shared__ float part[kRowWaves][R];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, sp = w % S;
    const int64_t grp = (int64_t)blockIdx.x * (kRowWaves / S) + w / S;
    const int32_t P8 = 2 * n8, P6 = P8 + 2 * n6, Pr = P6 + n4;
    // rows of the group past N re-read row N - 1 and are not written
    int64_t row[R];
#pragma unroll
    for (int r = 0; r < R; ++r) row[r] = min(grp * R + r, N - 1);

    // piece j of the lane: class (0 past the row's pieces), byte offset in
    // its plane row, global block. Pieces past the row re-read its last piece
    // (every load is unconditional, so all of them are in flight at once)
    int32_t cls[J], off[J], gb[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int32_t pu = 64 * J * sp + lane + 64 * j, p = min(pu, Pr - 1);
        if (p < P8) { cls[j] = 8; off[j] = 16 * p; gb[j] = p >> 1; }
        else if (p < P6) {
            const int32_t q = p - P8;
            cls[j] = 6; off[j] = 24 * (q >> 1) + 8 * (q & 1); gb[j] = n8 + (q >> 1);
        } else { cls[j] = 4; off[j] = 16 * (p - P6); gb[j] = n8 + n6 + (p - P6); }
        if (pu >= Pr) cls[j] = 0;
    }
    uint32_t T[J][4], R4[R][J][4], sa[J], sw[R][J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const bool c8 = gb[j] < n8, c6 = !c8 && gb[j] < n8 + n6;   // plane of the (clamped) piece
        const uint8_t *ab = c8 ? reinterpret_cast<const uint8_t *>(a8) : c6 ? a6 : a4;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint8_t *wb = c8   ? reinterpret_cast<const uint8_t *>(W.q8) + row[r] * W.ld8
                                : c6 ? W.q6 + row[r] * W.ld6
                                     : W.q4 + row[r] * W.ld4;
            const uint4 v = *reinterpret_cast<const uint4 *>(wb + off[j]);
            R4[r][j][0] = v.x; R4[r][j][1] = v.y; R4[r][j][2] = v.z; R4[r][j][3] = v.w;
            sw[r][j] = W.sc[row[r] * W.lds + gb[j]];
        }
        const uint4 v = *reinterpret_cast<const uint4 *>(ab + off[j]);
        T[j][0] = v.x; T[j][1] = v.y; T[j][2] = v.z; T[j][3] = v.w;
        sa[j] = asc[gb[j]];
    }

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
        const int c = cls[j];
        const bool second = (lane & 1) != 0;   // odd piece of an 8/6-bit pair (pieces of a split start even)
        uint32_t ab[4];
        if (c == 6) {
            uint32_t aw[3];
            piece6(T[j], second, aw);
            wide6x16(aw, ab);
        }
        const float fa = e8m0_to_f32(sa[j]) * (c == 6 ? 0.0625f : 1.0f);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int d;
            if (c == 4) {
                d = __builtin_amdgcn_sdot8((int)T[j][0], (int)R4[r][j][0], 0, false);
                d = __builtin_amdgcn_sdot8((int)T[j][1], (int)R4[r][j][1], d, false);
                d = __builtin_amdgcn_sdot8((int)T[j][2], (int)R4[r][j][2], d, false);
                d = __builtin_amdgcn_sdot8((int)T[j][3], (int)R4[r][j][3], d, false);
            } else if (c == 8) {
                d = __builtin_amdgcn_sdot4((int)T[j][0], (int)R4[r][j][0], 0, false);
                d = __builtin_amdgcn_sdot4((int)T[j][1], (int)R4[r][j][1], d, false);
                d = __builtin_amdgcn_sdot4((int)T[j][2], (int)R4[r][j][2], d, false);
                d = __builtin_amdgcn_sdot4((int)T[j][3], (int)R4[r][j][3], d, false);
                d += __builtin_amdgcn_mov_dpp(d, 0xB1, 0xF, 0xF, true);
            } else if (c == 6) {
                uint32_t wb[4], ww[3];
                piece6(R4[r][j], second, ww);
                wide6x16(ww, wb);
                d = __builtin_amdgcn_sdot4((int)ab[0], (int)wb[0], 0, false);
                d = __builtin_amdgcn_sdot4((int)ab[1], (int)wb[1], d, false);
                d = __builtin_amdgcn_sdot4((int)ab[2], (int)wb[2], d, false);
                d = __builtin_amdgcn_sdot4((int)ab[3], (int)wb[3], d, false);
                d += __builtin_amdgcn_mov_dpp(d, 0xB1, 0xF, 0xF, true);
            } else {
                d = 0;
            }
            const bool use = c == 4 || ((c == 8 || c == 6) && !second);
            acc[r] = __builtin_fmaf((float)d, use ? fa * e8m0_to_f32(sw[r][j]) : 0.f, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float v = acc[r];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
        acc[r] = v;
    }
    if constexpr (S == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            if (lane == 0 && grp * R + r < N) y[grp * R + r] = acc[r];
    } else {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) part[w][r] = acc[r];
        }
        __syncthreads();
        if (sp == 0 && lane < R && grp * R + lane < N) {
            float v = part[w][lane];
#pragma unroll
            for (int k = 1; k < S; ++k) v += part[w + k][lane];
            y[grp * R + lane] = v;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode with the matrix cores (9 to 32 tokens).
//
// One v_mfma_i32_32x32x32_i8 yields a 32 token x 32 row tile of exact block
// sums; the per-block epilogue (convert, scale, accumulate) then runs only
// over the tiles' token rows below M, so its cost grows with ceil(M / 8) and
// not with the 32-token tile. Codes enter the MFMA as bytes (8-bit as is,
// 6-bit * 4, 4-bit * 16, the factor folded into the scales); W fragments and
// token fragments are unpacked in registers in the same k order.
//
// The work is cut into the slices of the vector kernel (one width class,
// two chunks). A workgroup of four waves owns 64 W rows and four consecutive
// slices, one per wave. A wave issues every load of its slice at once (the
// W and token scale bytes, both chunks of W codes with the coalesced loads
// of k_gemv, the tokens' fragments), then stages each W chunk through its
// own LDS tile into the MFMA layout. The four waves' sums meet in LDS and are
// added in wave order; slice groups write partial rows that k_gemv_reduce
// adds in order.
constexpr int kDecScW = 6;   // dwords of staged W scale bytes per row (20 used)

struct DecWaveLds {          // one wave's LDS
    uint8_t tile[kGemvTile];          // a staged W chunk
    uint32_t wsc[64 * kDecScW];       // W scale bytes of the slice, row-major
    float asc[16 * 32];               // tokens' scales times the fold, [block][token]
};

// 16 MFMA bytes (one k-half) of a 4-bit block half held as two dwords: the
// low nibbles of each dword, then its high nibbles, each as code * 16
__device__ __forceinline__ v4i unpack4_half(uint32_t w0, uint32_t w1) {
    return v4i{(int)((w0 << 4) & 0xF0F0F0F0u), (int)(w0 & 0xF0F0F0F0u), (int)((w1 << 4) & 0xF0F0F0F0u),
               (int)(w1 & 0xF0F0F0F0u)};
}

// 16 MFMA bytes of a 6-bit block half: four 24-bit groups of 4 codes starting
// at bit 0 of w[0..2] (96 bits), each as code * 4
__device__ __forceinline__ v4i unpack6_half(const uint32_t w[3]) {
    const uint32_t g0 = w[0] & 0xFFFFFFu;
    const uint32_t g1 = __builtin_amdgcn_alignbit(w[1], w[0], 24) & 0xFFFFFFu;
    const uint32_t g2 = __builtin_amdgcn_alignbit(w[2], w[1], 16) & 0xFFFFFFu;
    const uint32_t g3 = w[2] >> 8;
    return v4i{(int)wide6(g0), (int)wide6(g1), (int)wide6(g2), (int)wide6(g3)};
}

// token fragment loads of one chunk (lane: token l % 32, k-half l / 32).
// Branch-free: lanes of tokens past M read token 0, blocks past the chunk
// read its first block and an empty chunk reads the plane's first block;
// those values meet zero token scales or are never used.
__device__ __forceinline__ void dec_fetch_a(const QView &A, int32_t M, const GemvChunk &c, int t, int h,
                                            uint32_t RA[16]) {
    const int64_t tr = t < M ? t : 0;
    const int64_t pb = c.nblk > 0 ? c.pb : 0;   // an empty chunk re-reads the plane's first block
    if (c.cls == 4) {
        const uint8_t *base = A.q4 + tr * A.ld4 + 16 * pb + 8 * h;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint2 v = *reinterpret_cast<const uint2 *>(base + 16 * (j < c.nblk ? j : 0));
            RA[2 * j] = v.x; RA[2 * j + 1] = v.y;
        }
    } else if (c.cls == 8) {
        const int8_t *base = A.q8 + tr * A.ld8 + 32 * pb + 16 * h;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 v = *reinterpret_cast<const uint4 *>(base + 32 * (j < c.nblk ? j : 0));
            RA[4 * j] = v.x; RA[4 * j + 1] = v.y; RA[4 * j + 2] = v.z; RA[4 * j + 3] = v.w;
        }
    } else {
        const uint8_t *base = A.q6 + tr * A.ld6 + 24 * pb + 12 * h;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t *q = reinterpret_cast<const uint32_t *>(base + 24 * (j < c.nblk ? j : 0));
            RA[3 * j] = q[0]; RA[3 * j + 1] = q[1]; RA[3 * j + 2] = q[2];
        }
    }
}

// One wave's slice (width CLS): loads, then per chunk stage, MFMA and the
// per-block epilogue into acc (tile i = W rows 32 i .. 32 i + 31).
template <int CLS>
__device__ __forceinline__ void dec_body(const QView &A, const QView &W, int32_t M, int64_t N, int32_t nb,
                                         const GemvChunk &sl, DecWaveLds &L, float acc[2][16]) {
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * 64;
    const int32_t rows_left = N - row0 < 64 ? (int32_t)(N - row0) : 64;
    constexpr int bpc = CLS == 4 ? 8 : 4;
    constexpr float fold = CLS == 8 ? 1.f : (CLS == 6 ? 0.25f : 0.0625f);

    // scale bytes: five W dwords from the one holding block gb (clamped to
    // the row's last dword), lane = row; token l32's bytes of blocks h + 2 i
    const int32_t d0 = sl.gb >> 2, dl = (nb - 1) >> 2;
    uint32_t vw[5], ab[8];
    {
        const uint32_t *sp = reinterpret_cast<const uint32_t *>(W.sc + (row0 + (lane < rows_left ? lane : 0)) * W.lds);
#pragma unroll
        for (int k = 0; k < 5; ++k) vw[k] = sp[min(d0 + k, dl)];
        const uint8_t *ap = A.sc + (int64_t)(l32 < M ? l32 : 0) * A.lds + sl.gb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = h + 2 * i;
            ab[i] = ap[j < sl.nblk ? j : 0];
        }
    }
    GemvChunk ch[kVecChunks];
    uint32_t R[kVecChunks][32], RA[kVecChunks][16];
#pragma unroll
    for (int j = 0; j < kVecChunks; ++j) {
        ch[j] = vec_chunk(sl, j);
        ch[j].cls = CLS;   // known at compile time: folds the width branches of the loads
        gemv_fetch(W, row0, rows_left, ch[j], lane, R[j]);
        dec_fetch_a(A, M, ch[j], l32, h, RA[j]);
    }
#pragma unroll
    for (int k = 0; k < 5; ++k) L.wsc[lane * kDecScW + k] = vw[k];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int j = h + 2 * i;
        L.asc[j * 32 + l32] = (l32 < M && j < sl.nblk) ? e8m0_to_f32(ab[i]) * fold : 0.f;
    }
    const uint8_t *wsb = reinterpret_cast<const uint8_t *>(L.wsc);
    const int qmax = (M + 7) >> 3;
    const v16i zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < kVecChunks; ++c) {
        if (ch[c].nblk == 0) break;
        __builtin_amdgcn_wave_barrier();            // the previous chunk's tile reads are done
        gemv_stage(L.tile, CLS, lane, R[c]);
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int j = 0; j < bpc; ++j) {
            if (j >= ch[c].nblk) break;
            v4i fa, fw[2];
            if (CLS == 4) {
                fa = unpack4_half(RA[c][2 * j], RA[c][2 * j + 1]);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint2 v = *reinterpret_cast<const uint2 *>(L.tile + (i * 32 + l32) * kGemvPitch + 16 * j + 8 * h);
                    fw[i] = unpack4_half(v.x, v.y);
                }
            } else if (CLS == 8) {
                fa = v4i{(int)RA[c][4 * j], (int)RA[c][4 * j + 1], (int)RA[c][4 * j + 2], (int)RA[c][4 * j + 3]};
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    fw[i] = *reinterpret_cast<const v4i *>(L.tile + (i * 32 + l32) * kGemvPitch + 32 * j + 16 * h);
            } else {
                const uint32_t wa[3] = {RA[c][3 * j], RA[c][3 * j + 1], RA[c][3 * j + 2]};
                fa = unpack6_half(wa);
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const uint32_t *q = reinterpret_cast<const uint32_t *>(L.tile + (i * 32 + l32) * kGemvPitch6 + 24 * j + 12 * h);
                    const uint32_t w[3] = {q[0], q[1], q[2]};
                    fw[i] = unpack6_half(w);
                }
            }
            v16i I[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) I[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa, fw[i], zero, 0, 0, 0);
            const int col = (sl.gb & 3) + c * bpc + j;   // the block's staged scale byte
            float sw[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) sw[i] = e8m0_to_f32(wsb[(i * 32 + l32) * 4 * kDecScW + col]) * fold;
            const float *sa_blk = L.asc + (c * bpc + j) * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (q >= qmax) break;
                const f32x4_t sa = *reinterpret_cast<const f32x4_t *>(sa_blk + 8 * q + 4 * h);
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][4 * q + r] = __builtin_fmaf((float)I[i][4 * q + r], sa[r] * sw[i], acc[i][4 * q + r]);
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_decode(QView A, QView W, int32_t M, int64_t N, int32_t n8, int32_t n6,
                                                int32_t n4, float *__restrict__ out, int64_t ldo,
                                                int64_t slice_stride) {
    __shared__ __attribute__((aligned(16))) DecWaveLds lds[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int64_t row0 = (int64_t)blockIdx.x * 64;
    const VecSlices S = vec_slices(n8, n6, n4);
    const int32_t ns = S.s8 + S.s6 + S.s4, nb = n8 + n6 + n4;
    const int32_t s = (int32_t)blockIdx.y * 4 + wave;

    float acc[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
    if (s < ns) {
        const GemvChunk sl = vec_slice(s, n8, n6, n4, S);
        if (sl.cls == 4)
            dec_body<4>(A, W, M, N, nb, sl, lds[wave], acc);
        else if (sl.cls == 8)
            dec_body<8>(A, W, M, N, nb, sl, lds[wave], acc);
        else
            dec_body<6>(A, W, M, N, nb, sl, lds[wave], acc);
    }

    // the four waves' sums of each output, added in wave order
    const int qmax = (M + 7) >> 3;
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);   // [wave][q][i][r][lane], 32 KiB
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q >= qmax) break;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(((wave * 4 + q) * 2 + i) * 4 + r) * 64 + lane] = acc[i][4 * q + r];
    }
    __syncthreads();
    // wave w finishes token group q = w (tokens 8w .. 8w+7)
    const int q = wave;
    if (q >= qmax) return;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t n = row0 + i * 32 + l32;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = red[(((0 * 4 + q) * 2 + i) * 4 + r) * 64 + lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) v = v + red[(((w * 4 + q) * 2 + i) * 4 + r) * 64 + lane];
            const int t = 8 * q + 4 * h + r;
            if (n < N && t < M) out[(int64_t)blockIdx.y * slice_stride + t * ldo + n] = v;
        }
    }
}

// Y[t, n] = sum over slices s (in order) of part[s][t][n]; loads run eight
// slices ahead of the ordered additions
__global__ __launch_bounds__(256) void k_gemv_reduce(const float *__restrict__ part, int32_t ns, int32_t M,
                                                     int64_t N, float *__restrict__ Y, int64_t ldy) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)M * N) return;
    const int64_t t = i / N, n = i - t * N, stride = (int64_t)M * N;
    float v = 0.f;
    int32_t s = 0;
    for (; s + 8 <= ns; s += 8) {
        float x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = part[(int64_t)(s + u) * stride + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) v = v + x[u];
    }
    for (; s < ns; ++s) v = v + part[(int64_t)s * stride + i];
    Y[t * ldy + n] = v;
}

// Row-tiles per group of k_gemm_a2r's tile order. When every tile runs in
// the first wave of workgroups, each XCD's run of 32 tiles then spans 4 row-
// by 8 column-tiles (8 MB of int8 operands at K = 4096 rather than 10 MB with
// 8 by 4), which measured 2-3 % faster at 2048 x 4096 x 4096; shapes with
// more tiles than CUs keep groups of 8 (4 measured 1-2 % slower there).
int32_t tile_group(int64_t ntiles) { return ntiles <= 256 ? 4 : 8; }

// Prepared operands of the int8 prefill kernel: 32-byte units (A in
// fragment order, W row-major; rows padded to the tile and to whole 128-byte
// pieces) and fp32 window scales [unit][row]. A's part comes first in the workspace;
// W's part is the same bytes whether it sits there or in a buffer filled
// once by mxs_prepare_weights.
struct PrepLayout {
    int64_t Mp, Np, Kp;
    size_t a_codes, a_cs, a_bytes;   // offsets inside A's part
    size_t w_codes, w_cs, w_bytes;   // offsets inside W's part
    size_t total;                    // both parts
    SplitK sk;                       // split of the product over K
    size_t part_bytes;               // its fp32 partial sums (after the operands)
};

// Shapes with fewer tiles than CUs split the product over K into about
// 256 / tiles parts of equal stage counts, boundaries rounded to the
// nearest allowed stage (a multiple of 5 up to the wide run's end, the wide
// run's end plus a multiple of 8 after it).
SplitK split_k(int64_t ntiles, int32_t nq, int32_t hw) {
    SplitK k;
    const int32_t nstage = (nq + kDSB - 1) / kDSB;
    int64_t want = ntiles <= 0 || ntiles >= 256 ? 1 : 256 / ntiles;   // no tiles (W only): no split
    if (want > kMaxSplitK) want = kMaxSplitK;
    k.n = 0;
    k.s[0] = 0;
    for (int64_t i = 1; i < want; ++i) {
        const int32_t t = (int32_t)((int64_t)nstage * i / want);
        int32_t b;
        // (a wide run whose length is not a multiple of 5 has no narrow
        // stages after it, so its splits never enter the narrow loop)
        if (t <= hw) b = (hw % 5 == 0) ? (t + 2) / 5 * 5 : t / 5 * 5;
        else b = hw + (t - hw + 4) / 8 * 8;
        if (b <= k.s[k.n] || b >= nstage) continue;
        k.s[++k.n] = b;
    }
    k.s[++k.n] = nstage;
    return k;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

PrepLayout prep_layout(int64_t M, int64_t N, const Segs &S) {
    PrepLayout L;
    L.Mp = ceil_div(M, kGBM) * kGBM;
    L.Np = ceil_div(N, kGBN) * kGBN;
    L.Kp = ceil_div(32 * (int64_t)S.nq, 128) * 128;   // whole 128-byte pieces (prep pads the tail)
    const int64_t nbp = L.Kp / 32;
    L.a_codes = 0;
    L.a_cs = align256((size_t)L.Mp * L.Kp);
    L.a_bytes = L.a_cs + align256((size_t)nbp * L.Mp * 4);
    L.w_codes = 0;
    L.w_cs = align256((size_t)L.Np * L.Kp);
    L.w_bytes = L.w_cs + align256((size_t)nbp * L.Np * 4);
    L.total = L.a_bytes + L.w_bytes;
    L.sk = split_k((L.Mp / kGBM) * (L.Np / kGBN), S.nq, S.hw);
    L.part_bytes = L.sk.n > 1 ? align256((size_t)L.sk.n * M * N * sizeof(float)) : 0;
    return L;
}

Segs segs_of(const mxs_qmat &Q) { return make_segs(Q.n8, Q.n6, Q.n4); }

int64_t prep_windows(const Segs &S, int64_t Kp) {
    return S.win_base[4] + ceil_div(Kp / 32 - S.nq, kG);
}

// W's prepared operand (k_gemm_prep, W job only) into wp
hipError_t launch_prep_w(const mxs_qmat &W, const PrepLayout &L, const Segs &S, uint8_t *wp, hipStream_t st) {
    PrepJob jw{view_of(W), W.rows, L.Np, reinterpret_cast<int8_t *>(wp + L.w_codes),
               reinterpret_cast<float *>(wp + L.w_cs), L.Np / 64, 0};
    const int64_t tw = jw.tiles_r * prep_windows(S, L.Kp);
    hipLaunchKernelGGL(k_gemm_prep, dim3((unsigned)tw), dim3(256), 0, st, jw, jw, (int64_t)0, L.Kp, S);
    return hipGetLastError();
}

// The int8 prefill product over prepared operands at ap (A's part) and wp
// (W's part).
hipError_t launch_a2r(const PrepLayout &L, const Segs &S, int64_t M, int64_t N, const uint8_t *ap,
                      const uint8_t *wp, float *Y, int64_t ldy, float *part, hipStream_t st) {
    const int64_t ntiles = (L.Mp / kGBM) * (L.Np / kGBN);
    hipLaunchKernelGGL(k_gemm_a2r, dim3((unsigned)ntiles, (unsigned)L.sk.n), dim3(512), 0, st,
                       reinterpret_cast<const int8_t *>(ap + L.a_codes), reinterpret_cast<const float *>(ap + L.a_cs),
                       reinterpret_cast<const int8_t *>(wp + L.w_codes), reinterpret_cast<const float *>(wp + L.w_cs),
                       M, N, L.Mp, L.Np, L.Kp, S.nq, S, Y, ldy, tile_group(ntiles), L.sk, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || L.sk.n == 1) return e;
    hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)ceil_div(M * N, 256)), dim3(256), 0, st, part,
                       (int32_t)L.sk.n, (int32_t)M, N, Y, ldy);
    return hipGetLastError();
}

bool use_prefill(const mxs_qmat &A) { return A.rows >= kPrefillMinRows; }
// The decode kernel addresses 64 W rows with 32-bit offsets, reads 4-bit
// rows in 16-byte pieces and both operands' scale bytes as aligned dwords.
bool use_gemv(const mxs_qmat &A, const mxs_qmat &W) {
    const int64_t lim = ((int64_t)1 << 32) / 64;
    auto al = [](const void *p, int64_t ld, int64_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0 && ld % a == 0; };
    return A.rows <= kGemvMaxRows && W.ld8 < lim && W.ld6 < lim && W.ld4 < lim && W.lds < lim &&
           al(A.sc, A.lds, 4) && al(W.sc, W.lds, 4) && (W.n4 == 0 || al(W.q4, W.ld4, 16));
}

template <int MT>
hipError_t launch_gemv_t(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy, void *ws, hipStream_t st) {
    const VecSlices S = vec_slices(A.n8, A.n6, A.n4);
    const int32_t ns = S.s8 + S.s6 + S.s4;
    const int64_t M = A.rows, N = W.rows;
    const dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ns);
    if (ns == 1) {
        hipLaunchKernelGGL((k_gemv<MT>), grid, dim3(64), 0, st, A.q8, A.ld8, A.q6, A.ld6, A.q4, A.ld4, A.sc, A.lds,
                           view_of(W), (int32_t)M, N, A.n8, A.n6, A.n4, Y, ldy, (int64_t)0);
        return hipGetLastError();
    }
    float *part = static_cast<float *>(ws);
    hipLaunchKernelGGL((k_gemv<MT>), grid, dim3(64), 0, st, A.q8, A.ld8, A.q6, A.ld6, A.q4, A.ld4, A.sc, A.lds,
                       view_of(W), (int32_t)M, N, A.n8, A.n6, A.n4, part, N, M * N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)ceil_div(M * N, 256)), dim3(256), 0, st, part, ns,
                       (int32_t)M, N, Y, ldy);
    return hipGetLastError();
}

// slice groups of the matrix-core decode kernel (four slices per workgroup)
int64_t decode_groups(const mxs_qmat &A) {
    const VecSlices S = vec_slices(A.n8, A.n6, A.n4);
    return ceil_div((int64_t)S.s8 + S.s6 + S.s4, 4);
}

hipError_t launch_decode(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy, void *ws, hipStream_t st) {
    const int64_t M = A.rows, N = W.rows, ng = decode_groups(A);
    const dim3 grid((unsigned)ceil_div(N, 64), (unsigned)ng);
    float *dst = ng == 1 ? Y : static_cast<float *>(ws);
    hipLaunchKernelGGL(k_decode, grid, dim3(256), 0, st, view_of(A), view_of(W), (int32_t)M, N, A.n8, A.n6, A.n4,
                       dst, ng == 1 ? ldy : N, ng == 1 ? (int64_t)0 : M * N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ng == 1) return e;
    hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)ceil_div(M * N, 256)), dim3(256), 0, st, dst, (int32_t)ng,
                       (int32_t)M, N, Y, ldy);
    return hipGetLastError();
}

// One token: J pieces per lane, R rows per wave, S waves per row
template <int J, int R, int S>
hipError_t launch_row_t(const mxs_qmat &A, const mxs_qmat &W, float *Y, hipStream_t st) {
    const int64_t N = W.rows, rows_per_wg = (int64_t)R * (kRowWaves / S);
    hipLaunchKernelGGL((k_gemv_row<J, R, S>), dim3((unsigned)ceil_div(N, rows_per_wg)), dim3(64 * kRowWaves), 0, st,
                       A.q8, A.q6, A.q4, A.sc, view_of(W), N, A.n8, A.n6, A.n4, Y);
    return hipGetLastError();
}

// pieces of one row (16-byte pieces: two per 8- or 6-bit block, one per 4-bit block)
int64_t row_pieces(const mxs_qmat &A) { return 2 * A.n8 + 2 * A.n6 + A.n4; }
constexpr int64_t kRowMaxPieces = 4 * 64 * 8;   // longer rows take the slice kernel

hipError_t launch_row(const mxs_qmat &A, const mxs_qmat &W, float *Y, hipStream_t st) {
    const int64_t P = row_pieces(A);
    // measured on the 70B MLP rows (308 pieces at K = 8192, 1076 at 28672):
    // three pieces per lane for four rows, split over two waves, and five
    // pieces for two rows over four waves, keep the most bytes in flight
    // (about 100 VGPRs, five waves per SIMD); one wave per long row (17
    // pieces) left two waves per SIMD and was 40 % slower
    if (P <= 3 * 64) return launch_row_t<3, 4, 1>(A, W, Y, st);
    if (P <= 2 * 3 * 64) return launch_row_t<3, 4, 2>(A, W, Y, st);
    if (P <= 4 * 3 * 64) return launch_row_t<3, 4, 4>(A, W, Y, st);
    if (P <= 4 * 5 * 64) return launch_row_t<5, 2, 4>(A, W, Y, st);
    return launch_row_t<8, 2, 4>(A, W, Y, st);
}

bool use_row(const mxs_qmat &A) {
    const int64_t P = row_pieces(A);
    return A.rows == 1 && P > 0 && P <= kRowMaxPieces;
}

hipError_t launch_gemv(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy, void *ws, hipStream_t st) {
    const int64_t M = A.rows;
    if (M > kGemvVecRows) return launch_decode(A, W, Y, ldy, ws, st);
    if (use_row(A)) return launch_row(A, W, Y, st);
    if (M <= 1) return launch_gemv_t<1>(A, W, Y, ldy, ws, st);
    if (M <= 2) return launch_gemv_t<2>(A, W, Y, ldy, ws, st);
    if (M <= 4) return launch_gemv_t<4>(A, W, Y, ldy, ws, st);
    return launch_gemv_t<8>(A, W, Y, ldy, ws, st);
}

// Prefill workspace: the two prepared operands, record-aligned, then the
// split sums when the product is split over K.
struct XLayout {
    int64_t Mp, Np;
    XPlan P;
    XSplit sk;
    bool narrow;   // 256 x 128 tiles (k_gemm_mx_n), no split
    size_t a_off, w_off, part_off, total;
};

// Grids of fewer than 64 tiles of 256 x 256 split the stages into about
// 256 / tiles parts of equal length (at most kMaxSplitK); grids of 64 to 255
// such tiles take the 256 x 128 kernel instead, unsplit (mx_split(256, ..)
// gives one part).
XSplit mx_split(int64_t ntiles, int32_t ns) {
    XSplit k;
    int64_t want = ntiles <= 0 || ntiles >= 256 ? 1 : 256 / ntiles;
    if (want > kMaxSplitK) want = kMaxSplitK;
    if (want > ns) want = ns > 0 ? ns : 1;
    k.n = (int32_t)want;
    for (int64_t i = 0; i <= want; ++i) k.s[i] = (int32_t)((int64_t)ns * i / want);
    return k;
}

XLayout mx_layout(const mxs_qmat &A, const mxs_qmat &W) {
    XLayout L;
    L.Mp = ceil_div(A.rows, kXBM) * kXBM;
    L.Np = ceil_div(W.rows, kXBN) * kXBN;
    L.P = make_xplan(A.n8, A.n6, A.n4);
    const int64_t t256 = (L.Mp / kXBM) * (L.Np / kXBN);
    L.narrow = t256 >= 64 && t256 < 256;
    L.sk = L.narrow ? mx_split(256, L.P.ns) : mx_split(t256, L.P.ns);
    L.a_off = 0;
    L.w_off = align256((size_t)(L.Mp / 64) * (size_t)L.P.ns * kXRec);
    L.part_off = align256(L.w_off + (size_t)(L.Np / 64) * (size_t)L.P.ns * kXRec);
    L.total = L.part_off + (L.sk.n > 1 ? (size_t)L.sk.n * (size_t)A.rows * (size_t)W.rows * sizeof(float) : 0);
    return L;
}

hipError_t launch_mx(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy, void *ws, hipStream_t st) {
    const XLayout L = mx_layout(A, W);
    int8_t *pa = static_cast<int8_t *>(ws) + L.a_off;
    int8_t *pw = static_cast<int8_t *>(ws) + L.w_off;
    float *part = reinterpret_cast<float *>(static_cast<int8_t *>(ws) + L.part_off);
    const int64_t ga = L.Mp / 64, gw = L.Np / 64;
    hipLaunchKernelGGL(k_mx_prep, dim3((unsigned)((ga + gw) * L.P.ns)), dim3(256), 0, st, view_of(A), view_of(W),
                       A.rows, W.rows, ga, A.n8, A.n6, A.n4, L.P, pa, pw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (L.narrow) {
        const int64_t ntiles = (L.Mp / kXBM) * (L.Np / ntile::kXBN);
        hipLaunchKernelGGL(ntile::k_gemm_mx_n, dim3((unsigned)ntiles), dim3(512), 0, st, pa, pw, A.rows, W.rows,
                           L.Mp, L.Np, L.P, Y, ldy);
        return hipGetLastError();
    }
    const int64_t ntiles = (L.Mp / kXBM) * (L.Np / kXBN);
    hipLaunchKernelGGL(k_gemm_mx, dim3((unsigned)ntiles, (unsigned)L.sk.n), dim3(256), 0, st, pa, pw, A.rows,
                       W.rows, L.Mp, L.Np, L.P, L.sk, Y, ldy, part);
    e = hipGetLastError();
    if (e != hipSuccess || L.sk.n <= 1) return e;
    const int64_t MN = A.rows * W.rows;
    hipLaunchKernelGGL(k_gemv_reduce, dim3((unsigned)ceil_div(MN, 256)), dim3(256), 0, st, part, L.sk.n,
                       (int32_t)A.rows, W.rows, Y, ldy);
    return hipGetLastError();
}


// Decode (up to 32 tokens) and 33..63 tokens take the same kernels in both
// entry points; they differ in the prefill kernels only.
size_t decode_workspace(const mxs_qmat &A, const mxs_qmat &W) {
    if (use_row(A)) return 0;   // one token: whole rows per wave, no partial rows
    const int64_t ns = A.rows > kGemvVecRows ? decode_groups(A) : [&] {
        const VecSlices S = vec_slices(A.n8, A.n6, A.n4);
        return (int64_t)S.s8 + S.s6 + S.s4;
    }();
    return ns > 1 ? (size_t)ns * (size_t)A.rows * (size_t)W.rows * sizeof(float) : 0;
}

hipError_t launch_small(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy, void *ws, hipStream_t st) {
    const int64_t M = A.rows, N = W.rows;
    if (use_gemv(A, W)) return launch_gemv(A, W, Y, ldy, ws, st);
    const dim3 grid((unsigned)ceil_div(N, kBN), (unsigned)ceil_div(M, kBM));
    hipLaunchKernelGGL(k_gemm_blockwise, grid, dim3(256), 0, st, view_of(A), view_of(W), M, N, A.n8, A.n6, A.n4, Y,
                       ldy);
    return hipGetLastError();
}

}  // namespace

size_t gemm_workspace(const mxs_qmat &A, const mxs_qmat &W, bool w_prepared) {
    if (W.rows == 0 || A.rows == 0) return 0;
    if (use_gemv(A, W)) return decode_workspace(A, W);
    if (!use_prefill(A)) return 0;
    const PrepLayout L = prep_layout(A.rows, W.rows, segs_of(A));
    return (w_prepared ? L.a_bytes : L.total) + L.part_bytes;
}

size_t wprep_bytes(const mxs_qmat &W) {
    if (W.rows == 0) return 0;
    return prep_layout(0, W.rows, segs_of(W)).w_bytes;
}

hipError_t launch_prepare_weights(const mxs_qmat &W, void *wprep, hipStream_t st) {
    if (W.rows == 0) return hipSuccess;
    const Segs S = segs_of(W);
    return launch_prep_w(W, prep_layout(0, W.rows, S), S, static_cast<uint8_t *>(wprep), st);
}

size_t gemm_workspace_mx(const mxs_qmat &A, const mxs_qmat &W) {
    if (W.rows == 0 || A.rows == 0) return 0;
    if (use_gemv(A, W)) return decode_workspace(A, W);
    if (!use_prefill(A)) return 0;
    return mx_layout(A, W).total;
}

hipError_t launch_mixed_gemm(const mxs_qmat &A, const mxs_qmat &W, const void *wprep, float *Y, int64_t ldy,
                             void *ws, hipStream_t st) {
    const int64_t M = A.rows, N = W.rows;
    if (M == 0 || N == 0) return hipSuccess;
    if (!use_prefill(A) || use_gemv(A, W)) return launch_small(A, W, Y, ldy, ws, st);
    const Segs S = segs_of(A);
    const PrepLayout L = prep_layout(M, N, S);
    uint8_t *ap = static_cast<uint8_t *>(ws);
    const int64_t windows = prep_windows(S, L.Kp);
    PrepJob ja{view_of(A), M, L.Mp, reinterpret_cast<int8_t *>(ap + L.a_codes), reinterpret_cast<float *>(ap + L.a_cs),
               L.Mp / 64, 1};
    const int64_t ta = ja.tiles_r * windows;
    const uint8_t *wp = static_cast<const uint8_t *>(wprep);
    if (wp) {   // W prepared already: A's operand only
        hipLaunchKernelGGL(k_gemm_prep, dim3((unsigned)ta), dim3(256), 0, st, ja, ja, ta, L.Kp, S);
    } else {    // both operands in one launch, W's part after A's
        uint8_t *wq = ap + L.a_bytes;
        PrepJob jw{view_of(W), N, L.Np, reinterpret_cast<int8_t *>(wq + L.w_codes),
                   reinterpret_cast<float *>(wq + L.w_cs), L.Np / 64, 0};
        const int64_t tw = jw.tiles_r * windows;
        hipLaunchKernelGGL(k_gemm_prep, dim3((unsigned)(ta + tw)), dim3(256), 0, st, ja, jw, ta, L.Kp, S);
        wp = wq;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    float *part = reinterpret_cast<float *>(ap + (wprep ? L.a_bytes : L.total));
    return launch_a2r(L, S, M, N, ap, wp, Y, ldy, part, st);
}


// Fused entry point: Y = mixed_gemm(quantize(X[:, perm] at W's block counts), W).
// Prefill rows whose row and permutation fit the LDS stage take
// k_quant_prep (no activation planes); other shapes quantize into planes
// held in the workspace and take the unfused kernels.
namespace {

mxs_qmat act_shape(int64_t M, const mxs_qmat &W) {
    mxs_qmat A;
    memset(&A, 0, sizeof A);
    A.rows = M;
    A.K = W.K;
    A.n8 = W.n8;
    A.n6 = W.n6;
    A.n4 = W.n4;
    return A;
}

int64_t quant_prep_lds(int64_t K, mxs_dtype dt) {
    return ((2 * K + 15) / 16) * 16 + K * (dt == MXS_BF16 ? 2 : 4);
}

bool fused_prefill(int64_t M, int64_t K, mxs_dtype dt) {
    return M >= kPrefillMinRows && K <= 65536 && quant_prep_lds(K, dt) <= kStageLds;
}

// activation planes inside the workspace (rows 16-byte aligned)
struct ActPlanes {
    size_t q8, q6, q4, sc, total;
    int64_t ld8, ld6, ld4, lds;
};

ActPlanes act_planes(const mxs_qmat &A) {
    ActPlanes P;
    P.ld8 = ceil_div(32 * (int64_t)A.n8, 16) * 16;
    P.ld6 = ceil_div(24 * (int64_t)A.n6, 16) * 16;
    P.ld4 = ceil_div(16 * (int64_t)A.n4, 16) * 16;
    P.lds = ceil_div(A.K / 32, 16) * 16;
    size_t off = 0;
    P.q8 = off; off = align256(off + (size_t)(A.rows * P.ld8));
    P.q6 = off; off = align256(off + (size_t)(A.rows * P.ld6));
    P.q4 = off; off = align256(off + (size_t)(A.rows * P.ld4));
    P.sc = off; off = align256(off + (size_t)(A.rows * P.lds));
    P.total = off;
    return P;
}

}  // namespace

template <typename T, int PPT>
hipError_t launch_quant_prep_t(const T *X, int64_t M, int64_t ldx, const int32_t *perm, int64_t K, int64_t Mp,
                               int64_t Kp, const Segs &S, int8_t *ac, float *acs, int64_t lds, hipStream_t st) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(k_quant_prep<T, PPT>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStageLds);
    if (e != hipSuccess) return e;
    // as many workgroups as LDS allows (up to 8 per CU), each streaming its
    // rows one ahead, and at least two rows per workgroup so that staging
    // the permutation is shared (measured: 4-5 % faster than one row each
    // at 2048 rows, K = 4096 and 8192; four rows each is no better)
    const int64_t per_cu = (160 * 1024) / lds;
    int64_t blocks = 256 * (per_cu < 8 ? (per_cu < 1 ? 1 : per_cu) : 8);
    const int64_t half = ceil_div(Mp, (int64_t)2);
    blocks = blocks < half ? blocks : half;
    hipLaunchKernelGGL((k_quant_prep<T, PPT>), dim3((unsigned)blocks), dim3(256), (size_t)lds, st, X, M, ldx, perm,
                       K, Mp, Kp, S, ac, acs);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_quant_prep_d(const T *X, int64_t M, int64_t ldx, const int32_t *perm, int64_t K, int64_t Mp,
                               int64_t Kp, const Segs &S, int8_t *ac, float *acs, int64_t lds, hipStream_t st) {
    const int64_t ppt = ceil_div(ceil_div(K * (int64_t)sizeof(T), (int64_t)16), (int64_t)256);
    if (ppt <= 1) return launch_quant_prep_t<T, 1>(X, M, ldx, perm, K, Mp, Kp, S, ac, acs, lds, st);
    if (ppt <= 2) return launch_quant_prep_t<T, 2>(X, M, ldx, perm, K, Mp, Kp, S, ac, acs, lds, st);
    if (ppt <= 4) return launch_quant_prep_t<T, 4>(X, M, ldx, perm, K, Mp, Kp, S, ac, acs, lds, st);
    if (ppt <= 8) return launch_quant_prep_t<T, 8>(X, M, ldx, perm, K, Mp, Kp, S, ac, acs, lds, st);
    if (ppt <= 16) return launch_quant_prep_t<T, 16>(X, M, ldx, perm, K, Mp, Kp, S, ac, acs, lds, st);
    return hipErrorInvalidValue;
}

hipError_t launch_quant_prep(const void *X, mxs_dtype dt, int64_t M, int64_t ldx, const int32_t *perm, int64_t K,
                             int64_t Mp, int64_t Kp, const Segs &S, int8_t *ac, float *acs, hipStream_t st) {
    const int64_t lds = quant_prep_lds(K, dt);
    if (dt == MXS_BF16)
        return launch_quant_prep_d(static_cast<const uint16_t *>(X), M, ldx, perm, K, Mp, Kp, S, ac, acs, lds, st);
    return launch_quant_prep_d(static_cast<const float *>(X), M, ldx, perm, K, Mp, Kp, S, ac, acs, lds, st);
}

size_t gemm_fused_workspace(int64_t M, mxs_dtype dt, const mxs_qmat &W, bool w_prepared) {
    if (M == 0 || W.rows == 0) return 0;
    const mxs_qmat A = act_shape(M, W);
    if (fused_prefill(M, W.K, dt) && !use_gemv(A, W)) {
        const PrepLayout L = prep_layout(M, W.rows, segs_of(A));
        return (w_prepared ? L.a_bytes : L.total) + L.part_bytes;
    }
    return act_planes(A).total + gemm_workspace(A, W, w_prepared);
}

hipError_t launch_mixed_gemm_fused(const void *X, mxs_dtype dt, int64_t M, int64_t ldx, const int32_t *perm,
                                   const mxs_qmat &W, const void *wprep, float *Y, int64_t ldy, void *ws,
                                   hipStream_t st) {
    const int64_t N = W.rows;
    if (M == 0 || N == 0) return hipSuccess;
    mxs_qmat A = act_shape(M, W);
    uint8_t *base = static_cast<uint8_t *>(ws);
    if (!fused_prefill(M, W.K, dt) || use_gemv(A, W)) {
        const ActPlanes P = act_planes(A);
        A.q8 = reinterpret_cast<int8_t *>(base + P.q8);
        A.ld8 = P.ld8;
        A.q6 = base + P.q6;
        A.ld6 = P.ld6;
        A.q4 = base + P.q4;
        A.ld4 = P.ld4;
        A.sc = base + P.sc;
        A.lds = P.lds;
        hipError_t e = launch_quantize(X, dt, ldx, perm, A, st);
        if (e != hipSuccess) return e;
        return launch_mixed_gemm(A, W, wprep, Y, ldy, base + P.total, st);
    }
    const Segs S = segs_of(A);
    const PrepLayout L = prep_layout(M, N, S);
    hipError_t e = launch_quant_prep(X, dt, M, ldx, perm, A.K, L.Mp, L.Kp, S,
                                     reinterpret_cast<int8_t *>(base + L.a_codes),
                                     reinterpret_cast<float *>(base + L.a_cs), st);
    if (e != hipSuccess) return e;
    const uint8_t *wp = static_cast<const uint8_t *>(wprep);
    if (!wp) {
        e = launch_prep_w(W, L, S, base + L.a_bytes, st);
        if (e != hipSuccess) return e;
        wp = base + L.a_bytes;
    }
    float *part = reinterpret_cast<float *>(base + (wprep ? L.a_bytes : L.total));
    return launch_a2r(L, S, M, N, base, wp, Y, ldy, part, st);
}

hipError_t launch_mixed_gemm_mx(const mxs_qmat &A, const mxs_qmat &W, float *Y, int64_t ldy,
                                void *ws, size_t, hipStream_t st) {
    const int64_t M = A.rows, N = W.rows;
    if (M == 0 || N == 0) return hipSuccess;
    if (!use_prefill(A) || use_gemv(A, W)) return launch_small(A, W, Y, ldy, ws, st);
    return launch_mx(A, W, Y, ldy, ws, st);
}

}  // namespace mxs
