// mxs_attention.hip -- attention of one query token over the 4-bit K/V cache.
//
// gist.science/nl "Technische Samenvatting" §4 (W4A4KV4): keys and values are
// kept as 4-bit MXINT, in the layout of mxs_quantize_kv (codes [T, H, D/2],
// element 2i in the low nibble of byte i; E8M0 scale bytes [T, H, D/32]).
// They are consumed here by scaled dot-product attention of one query token
// per head, query head h reading KV head h / (Hq / Hkv):
//   s_t = scale * q[h] . K[t, g],  p = softmax_t(s),  o[h] = sum_t p_t V[t, g].
// Codes are dequantized exactly (code * 2^(byte - 127) is exact in fp32).
//
// Layout of the work: a workgroup takes two KV heads (one when there is
// only one, or too little work), so it reads whole 128-byte lines of every
// cache row, and a run of consecutive tokens split into token parts, one
// wave per (head, part). A wave walks its part in sub-chunks of 64 tokens
// (32 for short caches) with an online softmax in log2 units (running
// maximum m and sum l per head; the output and l are rescaled by
// 2^(m_old - m_new) when some maximum grows). The next sub-chunk's loads
// are issued before the current one is computed. Both contractions run on
// the bf16 matrix cores (v_mfma_f32_16x16x32_bf16, heads padded to 16
// columns) with exact products: a code times its power-of-two scale is
// exact in bf16, and the fp32 query and softmax weights enter as the exact
// sum of three bf16 parts (one instruction per part); only the fp32
// accumulation rounds.
//   scores  S^T[t, h] = sum_d K[t, d] q[h, d]: A = K (16 tokens x 32 dims
//           per step, lane (t, c) takes 8 of its dims c D/4 .. c D/4 +
//           D/4 - 1 per step), B = the query parts (held in registers);
//   output  O^T[d, h] += sum_t V[t, d] p[t, h]: A = V (16 dims x 32 tokens,
//           lane (i, c) holds dims i D/16 .. i D/16 + D/16 - 1 of tokens
//           4c + r of two tiles), B = the parts of p, which the score step
//           leaves in exactly the lane layout B needs.
// Cache reads go through buffer descriptors that end at the part's last
// row, so rows past it read as zero (value 0; their scores are set to
// -inf). The parts of a workgroup are merged in LDS in part order, giving
// one (m, l, O) per head and workgroup; a second kernel combines the
// workgroups of a head in order, o = sum_s O_s 2^(m_s - M) / sum_s l_s
// 2^(m_s - M). Every sum has a fixed order, so the result is deterministic.
#include <cmath>

#include "mxs_device.h"
#include "mxs_internal.h"

namespace mxs {

namespace {

constexpr int kATile = 16;      // tokens per matrix tile; a sub-chunk is NTL = 2 or 4 tiles
constexpr int kAMaxG = 16;      // query heads per KV head (MFMA rows)
constexpr int kAMaxD = 256;     // head dimension
constexpr int kAWaves = 2048;   // waves the split aims at

typedef float v4f_a __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf_a __attribute__((ext_vector_type(8)));

// x = h + m + l exactly: three bf16 parts, each the nearest bf16 to what is
// left (every remainder is exact in fp32; the last one has at most 8
// significant bits)
// bf16 pair (lo, hi) of two fp32 values whose low 16 bits are zero (codes
// times a power of two), so taking the high halves is exact
__device__ __forceinline__ uint32_t bf16x2_exact(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
typedef uint32_t v4u_a __attribute__((ext_vector_type(4)));

struct Bf3 {
    __bf16 h, m, l;
};
__device__ __forceinline__ Bf3 split3(float x) {
    Bf3 t;
    t.h = (__bf16)x;
    const float r = x - (float)t.h;
    t.m = (__bf16)r;
    t.l = (__bf16)(r - (float)t.m);
    return t;
}

// sign-extended 4-bit field k of w (k compile-time)
__device__ __forceinline__ float nib(uint32_t w, int k) {
    return (float)((int32_t)(w << (28 - 4 * k)) >> 28);
}

// the 8 fields of w divided by 16 (v_cvt_off_f32_i4 reads bits 3:0 of the
// selected byte: even fields straight from w, odd ones from w >> 4; exact);
// the factor 16 goes into the other operand of the product
template <int SEL>
__device__ __forceinline__ float cvt_off_byte(uint32_t w) {
    float r;
    if constexpr (SEL == 0)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0" : "=v"(r) : "v"(w));
    else if constexpr (SEL == 1)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1" : "=v"(r) : "v"(w));
    else if constexpr (SEL == 2)
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2" : "=v"(r) : "v"(w));
    else
        asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3" : "=v"(r) : "v"(w));
    return r;
}
__device__ __forceinline__ void nib16x8(uint32_t w, float f[8]) {
    const uint32_t o = w >> 4;
    f[0] = cvt_off_byte<0>(w);
    f[1] = cvt_off_byte<0>(o);
    f[2] = cvt_off_byte<1>(w);
    f[3] = cvt_off_byte<1>(o);
    f[4] = cvt_off_byte<2>(w);
    f[5] = cvt_off_byte<2>(o);
    f[6] = cvt_off_byte<3>(w);
    f[7] = cvt_off_byte<3>(o);
}

// Buffer resource over n bytes at p (reads at offsets >= n return zero)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const uint8_t *p, int64_t n) {
    const int32_t nr = n <= 0 ? 0 : (n >= 0x7FFFFFFF ? 0x7FFFFFFF : (int32_t)n);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(p), 0, nr, 0x00020000);
}

// ND dwords of codes at byte offset off (4 ND bytes; 16-byte loads where ND
// is a multiple of 4, 8-byte where even)
template <int ND>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t w[ND]) {
    if constexpr (ND % 4 == 0) {
#pragma unroll
        for (int i = 0; i < ND / 4; ++i) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * i, 0, 0);
            w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
        }
    } else if constexpr (ND % 2 == 0) {
#pragma unroll
        for (int i = 0; i < ND / 2; ++i) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8 * i, 0, 0);
            w[2 * i] = v[0]; w[2 * i + 1] = v[1];
        }
    } else {
#pragma unroll
        for (int i = 0; i < ND; ++i) w[i] = __builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, 0);
    }
}

// ND bytes of codes at byte offset off into VW dwords
template <int ND>
__device__ __forceinline__ void load_bytes(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t w[(ND + 3) / 4]) {
    if constexpr (ND == 1) w[0] = __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
    else if constexpr (ND == 2) w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    else if constexpr (ND == 4) w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    else if constexpr (ND == 8) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        w[0] = v[0]; w[1] = v[1];
    } else {
#pragma unroll
        for (int i = 0; i < (ND + 3) / 4; ++i) w[i] = 0;
#pragma unroll
        for (int i = 0; i < ND; ++i)
            w[i >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off + i, 0, 0) << (8 * (i & 3));
    }
}

template <int ND>
struct KGeom {           // score operand: lane group c holds dims c DK .. c DK + DK - 1
    static constexpr int DK = 8 * ND;
    // scale bytes a lane keeps per token: the blocks its dims touch
    static constexpr int NB = ND % 4 == 0 ? ND / 4 : (ND <= 2 ? 1 : 3);
};
template <int ND>
struct VGeom {           // output operand: lane i holds dims i DL .. i DL + DL - 1
    static constexpr int DL = 2 * ND;
    static constexpr int NB = (16 % ND == 0) ? 1 : 2;
};

// scale of dim (base + s) from the NB scale values kept for blocks b0, b0+1, ...
template <int NB, bool ALIGNED>
__device__ __forceinline__ float pick_scale(const float sc[NB], int base, int b0, int s) {
    if constexpr (NB == 1) return sc[0];
    else if constexpr (ALIGNED) return sc[s >> 5];          // base is a multiple of 32
    else {
        const int k = ((base + s) >> 5) - b0;
        float v = sc[0];
#pragma unroll
        for (int i = 1; i < NB; ++i) v = k == i ? sc[i] : v;
        return v;
    }
}

// Raw codes and scale bytes of one sub-chunk as one lane loads them: K rows
// lt0 + 16 u + i (lane group c's dims), V rows lt0 + 16 u + 4 c + r (lane
// i's dims).
template <int ND, int NTL>
struct KChunk {
    uint32_t w[NTL][ND];
    uint32_t sb[NTL][KGeom<ND>::NB];
};
template <int ND, int NTL>
struct VChunk {
    uint32_t w[NTL][4][(ND + 3) / 4];
    uint32_t sb[NTL][4][VGeom<ND>::NB];
};

// Where one wave reads: the cache rows of its KV head from its first token
// on (codes and scale bytes), and the lane's byte offsets inside a row.
struct AttnSrc {
    const uint8_t *kc, *ks, *vc, *vs;   // row of (first token, KV head)
    uint32_t rowb, srow;                 // token stride of codes / scales
    int nt;                              // tokens of the wave
    uint32_t koff, kso, voff, vso;       // lane offsets inside a row
};

// Rows past the wave's last token read as zero (the buffer ends there), so
// the tail needs no clamping: zero codes, and the scale byte 0 gives value 0.
template <int ND, int NTL>
__device__ __forceinline__ void load_k(KChunk<ND, NTL> &ch, const AttnSrc &a, int lt0, int i) {
    constexpr int D = 32 * ND, KNB = KGeom<ND>::NB;
    const int64_t left = a.nt - 1 - lt0;       // rows still valid after lt0
    const auto rc = attn_rsrc(a.kc + (int64_t)lt0 * a.rowb, left * a.rowb + D / 2);
    const auto rs = attn_rsrc(a.ks + (int64_t)lt0 * a.srow, left * a.srow + ND);
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
        load_words<ND>(rc, __umul24(16 * u + i, a.rowb) + a.koff, ch.w[u]);
#pragma unroll
        for (int b = 0; b < KNB; ++b) {
            ch.sb[u][b] = __builtin_amdgcn_raw_buffer_load_b8(rs, __umul24(16 * u + i, a.srow) + a.kso + b, 0, 0);
        }
    }
}

template <int ND, int NTL>
__device__ __forceinline__ void load_v(VChunk<ND, NTL> &ch, const AttnSrc &a, int lt0, int c) {
    constexpr int D = 32 * ND, VNB = VGeom<ND>::NB;
    const int64_t left = a.nt - 1 - lt0;
    const auto rc = attn_rsrc(a.vc + (int64_t)lt0 * a.rowb, left * a.rowb + D / 2);
    const auto rs = attn_rsrc(a.vs + (int64_t)lt0 * a.srow, left * a.srow + ND);
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            load_bytes<ND>(rc, __umul24(16 * u + 4 * c + r, a.rowb) + a.voff, ch.w[u][r]);
#pragma unroll
            for (int b = 0; b < VNB; ++b)
                ch.sb[u][r][b] =
                    __builtin_amdgcn_raw_buffer_load_b8(rs, __umul24(16 * u + 4 * c + r, a.srow) + a.vso + b, 0, 0);
        }
}

// Scores (log2 units) of the sub-chunk: lane (i, c) gets head i's scores of
// tokens lt0 + 16 u + 4 c + r, -inf past the wave's last token. Step b of
// a tile takes the lane group's dword b of K (8 dims; code x scale is exact
// in bf16) against the three bf16 parts of the query.
template <int ND, int NTL>
__device__ __forceinline__ void attn_scores(const KChunk<ND, NTL> &ch, const v8bf_a qp[ND][3], int lt0, int nt,
                                            float scale2, int c, int kb0, float sv[NTL][4]) {
    constexpr int DK = KGeom<ND>::DK, KNB = KGeom<ND>::NB;
    float ksc[NTL][KNB];
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
        for (int b = 0; b < KNB; ++b) ksc[u][b] = e8m0_to_f32(ch.sb[u][b]);
    v4f_a sc4[NTL];
#pragma unroll
    for (int u = 0; u < NTL; ++u) sc4[u] = v4f_a{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < ND; ++b)
#pragma unroll
        for (int u = 0; u < NTL; ++u) {
            float kf[8];
            nib16x8(ch.w[u][b], kf);
#pragma unroll
            for (int n = 0; n < 8; ++n) kf[n] *= pick_scale<KNB, ND % 4 == 0>(ksc[u], c * DK, kb0, 8 * b + n);
            const v4u_a kw2 = {bf16x2_exact(kf[0], kf[1]), bf16x2_exact(kf[2], kf[3]), bf16x2_exact(kf[4], kf[5]),
                               bf16x2_exact(kf[6], kf[7])};
            const v8bf_a kv = __builtin_bit_cast(v8bf_a, kw2);
#pragma unroll
            for (int p = 0; p < 3; ++p) sc4[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qp[b][p], sc4[u], 0, 0, 0);
        }
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[u][r] = lt0 + 16 * u + 4 * c + r < nt ? sc4[u][r] * scale2 : -INFINITY;
}

// Online-softmax state of a wave: running maximum and sum (log2 units) of
// head i, and the output accumulators O^T (tile n, register rr: dim
// (4 c + rr) DL + n of head i).
template <int ND>
struct AttnState {
    v4f_a acc[ND * 2];
    float m, l;
};

// Folds the sub-chunk's scores into the running maximum and sum (sv becomes
// p = 2^(s - m)), then adds p V to the accumulators.
template <int ND, int NTL>
__device__ __forceinline__ void attn_values(AttnState<ND> &st, const VChunk<ND, NTL> &ch, float sv[NTL][4], int i,
                                            int vb0) {
    constexpr int DL = VGeom<ND>::DL, VNB = VGeom<ND>::NB, NT = 2 * ND;
    float mloc = -INFINITY;
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, sv[u][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(st.m, mloc);
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            sv[u][r] = sv[u][r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[u][r] - m_new);
            lsum += sv[u][r];
        }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    // rescale only when some head's maximum grew
    if (__ballot(m_new != st.m)) {
        const float alpha = st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - m_new);
#pragma unroll
        for (int n = 0; n < NT; ++n) st.acc[n] *= alpha;
        st.l *= alpha;
    }
    st.l += lsum;
    st.m = m_new;

    // 32 tokens per step: lane group c contributes tokens 4 c + r of tiles
    // u0 and u0 + 1 (the ones whose p it holds), V as exact bf16 values of
    // dims i DL + n (tile n), p as three bf16 parts
#pragma unroll
    for (int u0 = 0; u0 < NTL; u0 += 2) {
        v8bf_a pb[3];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const Bf3 t = split3(16.f * sv[u0 + (j >> 2)][j & 3]);   // V enters as code / 16
            pb[0][j] = t.h;
            pb[1][j] = t.m;
            pb[2][j] = t.l;
        }
        float vsc[8][VNB];
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int b = 0; b < VNB; ++b) vsc[j][b] = e8m0_to_f32(ch.sb[u0 + (j >> 2)][j & 3][b]);
        // the lane's 2 ND values of each of its 8 rows (code / 16)
        float vr[8][NT];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float f[8];
            nib16x8(ch.w[u0 + (j >> 2)][j & 3][0], f);
#pragma unroll
            for (int n = 0; n < NT && n < 8; ++n) vr[j][n] = f[n];
            if constexpr (NT > 8) {
                nib16x8(ch.w[u0 + (j >> 2)][j & 3][1], f);
#pragma unroll
                for (int n = 8; n < NT; ++n) vr[j][n] = f[n - 8];
            }
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float vf[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) vf[j] = vr[j][n] * pick_scale<VNB, false>(vsc[j], i * DL, vb0, n);
            const v4u_a vw2 = {bf16x2_exact(vf[0], vf[1]), bf16x2_exact(vf[2], vf[3]), bf16x2_exact(vf[4], vf[5]),
                               bf16x2_exact(vf[6], vf[7])};
            const v8bf_a vv = __builtin_bit_cast(v8bf_a, vw2);
#pragma unroll
            for (int p = 0; p < 3; ++p) st.acc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, pb[p], st.acc[n], 0, 0, 0);
        }
    }
}

// Waves per workgroup: eight where a wave fits in 256 VGPRs (D = 32, 64,
// 128), else four.
__host__ __device__ constexpr int attn_waves(int ND) { return ND == 1 || ND == 2 || ND == 4 ? 8 : 4; }
template <int ND>
struct AttnWg {
    static constexpr int NW = attn_waves(ND);
};

// LDS of one workgroup: per wave, (m, l) and O of every query head of its group
__host__ __device__ constexpr int attn_lds_bytes(int NW, int G, int D) { return NW * G * (D + 2) * 4; }

template <int ND, int NTL>
__global__ __launch_bounds__(64 * AttnWg<ND>::NW) void k_attn_part(
    const float *__restrict__ q, const uint8_t *__restrict__ kc, const uint8_t *__restrict__ ks,
    const uint8_t *__restrict__ vc, const uint8_t *__restrict__ vs, int64_t T, int Hkv, int G, int HW, int NQ,
    int TSw, float scale2, float *__restrict__ pm, float *__restrict__ pl, float *__restrict__ po) {
    constexpr int D = 32 * ND, DK = KGeom<ND>::DK, DL = VGeom<ND>::DL, NT = 2 * ND;
    const int NW = HW * NQ;                 // waves of this launch (blockDim.x / 64)
    extern __shared__ __attribute__((aligned(16))) float attn_lds[];
    float *sml = attn_lds;                  // [NW][G][2]: m, l
    float *so = attn_lds + NW * G * 2;      // [NW][G][D]
    const int lane = threadIdx.x & 63;
    // wave w takes KV head w % HW of the workgroup's and token part w / HW
    // (wave-uniform, so the buffer descriptors stay scalar)
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.y * HW + w % HW, part = w / HW;
    const int i = lane & 15, c = lane >> 4;
    const int64_t split = blockIdx.x, nsplit = gridDim.x;
    const int64_t t0 = (split * NQ + part) * (int64_t)TSw;
    const int nt = g < Hkv ? (int)(T - t0 < TSw ? (T - t0 > 0 ? T - t0 : 0) : TSw) : 0;

    AttnState<ND> st;
#pragma unroll
    for (int n = 0; n < NT; ++n) st.acc[n] = v4f_a{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
    if (nt > 0) {
        const int kb0 = (c * DK) >> 5, vb0 = (i * DL) >> 5;       // first scale block of the lane's dims
        AttnSrc a;
        a.kc = kc + (t0 * Hkv + g) * (D / 2);
        a.vc = vc + (t0 * Hkv + g) * (D / 2);
        a.ks = ks + (t0 * Hkv + g) * ND;
        a.vs = vs + (t0 * Hkv + g) * ND;
        a.rowb = (uint32_t)Hkv * (D / 2);
        a.srow = (uint32_t)Hkv * ND;
        a.nt = nt;
        a.koff = c * (DK / 2);
        a.kso = kb0;
        a.voff = i * ND;
        a.vso = vb0;

        // query column of head i (zero for the padding heads), dims c DK + s;
        // its loads go out first, then the first sub-chunk's, and the query
        // is split into three bf16 parts per step of 8 dims while those fly
        float qv[DK];
        {
            const float *qs = q + ((int64_t)g * G + (i < G ? i : 0)) * D + c * DK;
#pragma unroll
            for (int s = 0; s < DK; ++s) qv[s] = qs[s];
        }
        __builtin_amdgcn_sched_barrier(0);
        constexpr int SUB = kATile * NTL;                        // tokens per sub-chunk
        KChunk<ND, NTL> kch;
        VChunk<ND, NTL> vch;
        load_k<ND, NTL>(kch, a, 0, i);
        load_v<ND, NTL>(vch, a, 0, c);
        __builtin_amdgcn_sched_barrier(0);
        v8bf_a qp[ND][3];
#pragma unroll
        for (int s = 0; s < DK; ++s) {
            const Bf3 t = split3(i < G ? 16.f * qv[s] : 0.f);   // K enters as code / 16
            qp[s >> 3][0][s & 7] = t.h;
            qp[s >> 3][1][s & 7] = t.m;
            qp[s >> 3][2][s & 7] = t.l;
        }

        // software pipeline: the next sub-chunk's K loads fly while this
        // one's values are summed, its V loads while the next scores are
        // formed; one copy of each phase keeps the code small (scheduling
        // barriers keep the loads ahead of the work they overlap)
        for (int lt = 0; lt < nt; lt += SUB) {
            float sv[NTL][4];
            attn_scores<ND, NTL>(kch, qp, lt, nt, scale2, c, kb0, sv);
            load_k<ND, NTL>(kch, a, lt + SUB, i);
            __builtin_amdgcn_sched_barrier(0);
            attn_values<ND, NTL>(st, vch, sv, i, vb0);
            load_v<ND, NTL>(vch, a, lt + SUB, c);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // lane (i, c), tile n, register rr holds O[head i][dim (4 c + rr) DL + n]
    if (NQ == 1) {   // one token part per workgroup: straight to the split outputs
        if (i < G && g < Hkv) {
            const int64_t hs = ((int64_t)g * G + i) * nsplit + split;
            if (c == 0) {
                pm[hs] = st.m;
                pl[hs] = st.l;
            }
            float *op = po + hs * D;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                for (int n = 0; n < NT; ++n) op[(4 * c + rr) * DL + n] = st.acc[n][rr];
        }
        return;
    }
    if (i < G) {
        if (c == 0) {
            sml[(w * G + i) * 2] = st.m;
            sml[(w * G + i) * 2 + 1] = st.l;
        }
        float *op = so + (w * G + i) * D;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int n = 0; n < NT; ++n) op[(4 * c + rr) * DL + n] = st.acc[n][rr];
    }
    __syncthreads();

    // merge the token parts of each head in part order: M = max m_p,
    // O = sum_p O_p 2^(m_p - M), l = sum_p l_p 2^(m_p - M); part 0 always
    // has tokens, so M is finite. Thread t takes elements t, t + B, ... of
    // the (head row gh, dim d) grid, (gh, d) stepped without division
    // (HW <= 2, so the KV head of row gh is gh >= G)
    const int B = 64 * NW, Bq = B / D, Bd = B - Bq * D;
    int gh = threadIdx.x / D, d = threadIdx.x - gh * D;
    while (gh < HW * G) {
        const int gl = gh >= G ? 1 : 0, h = gh - gl * G;
        const int gg = blockIdx.y * HW + gl;
        if (gg < Hkv) {
            float M = -INFINITY;
            for (int p = 0; p < NQ; ++p) M = fmaxf(M, sml[((p * HW + gl) * G + h) * 2]);
            float o = 0.f, l = 0.f;
            for (int p = 0; p < NQ; ++p) {
                const int wp = p * HW + gl;
                const float mp = sml[(wp * G + h) * 2];
                const float f = mp == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mp - M);
                o = __builtin_fmaf(so[(wp * G + h) * D + d], f, o);
                l = __builtin_fmaf(sml[(wp * G + h) * 2 + 1], f, l);
            }
            const int64_t hs = ((int64_t)gg * G + h) * nsplit + split;
            po[hs * D + d] = o;
            if (d == 0) {
                pm[hs] = M;
                pl[hs] = l;
            }
        }
        d += Bd;
        gh += Bq;
        if (d >= D) {
            d -= D;
            ++gh;
        }
    }
}

// o[h, d] = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) (maxima in log2
// units, which the split kernel works in). One workgroup per head: thread
// (d4, ph) takes four dims d4 and the splits ph, ph + P, ... in order
// (P = 256 / (D / 4) phases, loads issued several splits ahead), then the
// phases are added in order.
__global__ __launch_bounds__(256) void k_attn_combine(const float *__restrict__ pm, const float *__restrict__ pl,
                                                      const float *__restrict__ po, int64_t nsplit, int D,
                                                      float *__restrict__ out) {
    __shared__ float red[256];
    __shared__ float4 sa[256];
    __shared__ float sl[256];
    const int64_t h = blockIdx.x;
    const int tid = threadIdx.x;
    const float *hm = pm + h * nsplit, *hl = pl + h * nsplit;
    const float4 *ho = reinterpret_cast<const float4 *>(po + h * nsplit * D);
    float m = -INFINITY;
    for (int64_t s = tid; s < nsplit; s += 256) m = fmaxf(m, hm[s]);
    red[tid] = m;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
        __syncthreads();
    }
    const float M = red[0];
    const int D4 = D / 4, P = 256 / D4, d4 = tid % D4, ph = tid / D4;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
    if (ph < P) {
#pragma unroll 4
        for (int64_t s = ph; s < nsplit; s += P) {
            const float f = __builtin_amdgcn_exp2f(hm[s] - M);
            const float4 v = ho[s * D4 + d4];
            l = __builtin_fmaf(hl[s], f, l);
            acc.x = __builtin_fmaf(v.x, f, acc.x);
            acc.y = __builtin_fmaf(v.y, f, acc.y);
            acc.z = __builtin_fmaf(v.z, f, acc.z);
            acc.w = __builtin_fmaf(v.w, f, acc.w);
        }
    }
    sa[tid] = acc;
    sl[tid] = l;
    __syncthreads();
    if (tid < D4) {
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        float L = 0.f;
        for (int q = 0; q < P; ++q) {
            const float4 v = sa[q * D4 + tid];
            a.x += v.x;
            a.y += v.y;
            a.z += v.z;
            a.w += v.w;
            L += sl[q * D4 + tid];
        }
        reinterpret_cast<float4 *>(out + h * D)[tid] = make_float4(a.x / L, a.y / L, a.z / L, a.w / L);
    }
}

// Split of the cache: sub-chunks of 64 tokens (32 when there are fewer than
// 4096 sub-chunks of 64, so that short caches still fill the chip); TSw
// tokens per wave, a multiple of the sub-chunk chosen so that about 2048
// waves run; a workgroup takes HW KV heads (two when there are
// enough waves: two heads fill a 128-byte line of every cache row) and NQ
// consecutive token parts of TSw tokens, as many as keep 256 or more
// workgroups busy, at most the waves one workgroup may hold.
struct AttnSplit {
    int NTL, HW, NQ, TSw;
    int64_t ns;
};

AttnSplit attn_split(int64_t T, int64_t Hkv, int64_t D) {
    AttnSplit s;
    s.NTL = ceil_div(T, (int64_t)4 * kATile) * Hkv >= 2 * kAWaves ? 4 : 2;
    const int64_t SUB = (int64_t)kATile * s.NTL;
    int64_t sub = ceil_div(ceil_div(T, SUB) * Hkv, (int64_t)kAWaves);
    if (sub < 1) sub = 1;
    s.TSw = (int)(sub * SUB);
    const int64_t waves = ceil_div(T, (int64_t)s.TSw) * Hkv;
    s.HW = Hkv >= 2 && waves >= 512 ? 2 : 1;
    const int nwmax = attn_waves((int)(D / 32));
    s.NQ = 1;
    while (2 * s.NQ * s.HW <= nwmax && waves >= (int64_t)256 * s.HW * 2 * s.NQ) s.NQ *= 2;
    s.ns = ceil_div(T, (int64_t)s.TSw * s.NQ);
    return s;
}

template <int ND>
hipError_t launch_part(const AttnSplit &sp, int64_t Hkv, int G, hipStream_t st, const float *q, const uint8_t *kc,
                       const uint8_t *ks, const uint8_t *vc, const uint8_t *vs, int64_t T, float scale2, float *pm,
                       float *pl, float *po) {
    const int nw = sp.HW * sp.NQ;
    if (nw > AttnWg<ND>::NW) return hipErrorInvalidValue;
    const dim3 grid((unsigned)sp.ns, (unsigned)ceil_div(Hkv, (int64_t)sp.HW));
    const size_t lds = (size_t)attn_lds_bytes(nw, G, 32 * ND);
    if (sp.NTL == 4)
        hipLaunchKernelGGL((k_attn_part<ND, 4>), grid, dim3(64 * nw), lds, st, q, kc, ks, vc, vs, T, (int)Hkv, G,
                           sp.HW, sp.NQ, sp.TSw, scale2, pm, pl, po);
    else
        hipLaunchKernelGGL((k_attn_part<ND, 2>), grid, dim3(64 * nw), lds, st, q, kc, ks, vc, vs, T, (int)Hkv, G,
                           sp.HW, sp.NQ, sp.TSw, scale2, pm, pl, po);
    return hipGetLastError();
}

}  // namespace

size_t attend_kv4_workspace(int64_t T, int64_t Hq, int64_t Hkv, int64_t D) {
    return (size_t)(attn_split(T, Hkv, D).ns * Hq * (2 + D)) * sizeof(float);
}

bool attend_kv4_supported(int64_t Hq, int64_t Hkv, int64_t D) {
    return Hq / Hkv <= kAMaxG && D <= kAMaxD;
}

hipError_t launch_attend_kv4(const float *q, const uint8_t *kc, const uint8_t *ks, const uint8_t *vc,
                             const uint8_t *vs, int64_t T, int64_t Hq, int64_t Hkv, int64_t D, float scale,
                             float *out, void *ws, hipStream_t st) {
    const AttnSplit sp = attn_split(T, Hkv, D);
    const int G = (int)(Hq / Hkv);
    // partial outputs first (16-byte aligned with the workspace), then maxima and sums
    float *po = static_cast<float *>(ws), *pm = po + sp.ns * Hq * D, *pl = pm + sp.ns * Hq;
    const float scale2 = scale * 1.44269504088896341f;   // scores in log2 units: 2^(s log2 e) = e^s
    hipError_t e;
    switch (D / 32) {
        case 1: e = launch_part<1>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        case 2: e = launch_part<2>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        case 3: e = launch_part<3>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        case 4: e = launch_part<4>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        case 5: e = launch_part<5>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        case 6: e = launch_part<6>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        case 7: e = launch_part<7>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        case 8: e = launch_part<8>(sp, Hkv, G, st, q, kc, ks, vc, vs, T, scale2, pm, pl, po); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)Hq), dim3(256), 0, st, pm, pl, po, sp.ns, (int)D, out);
    return hipGetLastError();
}

}  // namespace mxs
