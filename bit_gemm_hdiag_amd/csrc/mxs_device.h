// mxs_device.h -- device helpers shared by the gfx950 kernels of libmxsens.
//
// MXINT block arithmetic (one shared power-of-two scale per 32 values,
// gist.science/nl "Technische Samenvatting" §1 and §2.2), done on raw fp32
// bit patterns so that subnormal inputs and the exponent clamp are exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxs {

constexpr int kBlock = 32;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- loads
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// Eight consecutive elements starting at p, widened to fp32 (exact for bf16).
// VEC: p is 16-byte aligned (bf16) or 16-byte aligned (fp32, two loads).
template <typename T, bool VEC>
__device__ __forceinline__ void load8(const T *p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t, true>(const uint16_t *p, float v[8]) {
    u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    uint32_t w[4] = {u[0], u[1], u[2], u[3]};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
template <>
__device__ __forceinline__ void load8<uint16_t, false>(const uint16_t *p, float v[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = bf16_bits_to_f32(p[i]);
}
template <>
__device__ __forceinline__ void load8<float, true>(const float *p, float v[8]) {
    f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 1);
    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
}
template <>
__device__ __forceinline__ void load8<float, false>(const float *p, float v[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i];
}

template <typename T>
__device__ __forceinline__ float load1(const T *p);
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t *p) { return bf16_bits_to_f32(*p); }
template <>
__device__ __forceinline__ float load1<float>(const float *p) { return *p; }

// ---------------------------------------------------------------- lane groups
// Max over the 4 lanes of an aligned quad (one 32-value block when each lane
// holds 8 values), by DPP quad permutes.
__device__ __forceinline__ uint32_t quad_max_u32(uint32_t x) {
    uint32_t y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true); // xor 1
    x = x > y ? x : y;
    y = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);          // xor 2
    return x > y ? x : y;
}

// ---------------------------------------------------------------- block scale
// Scale of an m-bit MXINT block from the largest |value| bit pattern
// (sign cleared). s = floor(log2 amax) - (m - 2), clamped to >= -127; the
// largest finite fp32 gives s <= 125, so the upper clamp never binds.
// amax bits >= 0x7f800000 means the block holds Inf or NaN.
struct BlockScale {
    uint32_t byte;  // E8M0 byte s + 127 (0xFF: non-finite block)
    float inv;      // 2^-s (always a normal fp32)
    float scale;    // 2^s (2^-127 is the subnormal 0x00400000)
    bool bad;
};

__device__ __forceinline__ BlockScale block_scale(uint32_t amax_bits, int m) {
    BlockScale r;
    r.bad = amax_bits >= 0x7f800000u;
    // exponent field 0 (zero or subnormal amax) gives E <= -127 and s = -127
    int E = (int)(amax_bits >> 23) - 127;
    int s = E - (m - 2);
    s = s < -127 ? -127 : s;
    r.byte = r.bad ? 0xFFu : (uint32_t)(s + 127);
    int si = r.bad ? 0 : s;
    r.inv = __uint_as_float((uint32_t)(127 - si) << 23);
    r.scale = si >= -126 ? __uint_as_float((uint32_t)(127 + si) << 23) : __uint_as_float(0x00400000u);
    return r;
}

// Code of one value: round half to even, symmetric clamp to +-cmax.
// v * inv is exact unless it is below 2^-126, where it rounds to 0 either way.
__device__ __forceinline__ float code_of(float v, float inv, float cmax) {
    float t = __builtin_rintf(v * inv);
    return __builtin_amdgcn_fmed3f(t, -cmax, cmax);
}

__device__ __forceinline__ float cmax_of(int m) { return (float)((1 << (m - 1)) - 1); }

// Quantise the 8 values a lane holds (a quarter of a block; the other three
// quarters sit in the other lanes of the aligned quad). All 4 lanes of the
// quad must be active. Returns the integer codes and the block's scale.
__device__ __forceinline__ BlockScale quantize8(const float v[8], int m, int c[8]) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
        a = a > b ? a : b;
    }
    a = quad_max_u32(a);
    BlockScale bs = block_scale(a, m);
    const float cm = cmax_of(m);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = bs.bad ? 0 : (int)code_of(v[i], bs.inv, cm);
    return bs;
}

// Quantise the 8 values a lane holds and pack their codes for width m
// (4: bits 4i.., 32 bits; 6: bits 6i.., 48 bits; 8: byte i, 64 bits), the
// layout of pack4 / pack6 / pack8 below; `byte` receives the block's E8M0
// byte. All 4 lanes of the quad must be active.
// fma(v, 2^-s, 1.5 * 2^23) rounds v / 2^s to nearest even into the low
// mantissa bits (v / 2^s is exact and |v / 2^s| < 2^7, so the sum stays in
// the binade [2^23, 2^24) whose ulp is 1); the symmetric clamp is a median
// against 1.5 * 2^23 -+ cmax; the low byte of the float's bits is then the
// two's-complement code. A non-finite block's codes are 0.
__device__ __forceinline__ uint32_t nib4(uint32_t x) {   // four code bytes -> 16 bits
    const uint32_t y = (x & 0x000F000Fu) | ((x >> 4) & 0x00F000F0u);
    return (y & 0xFFu) | ((y >> 8) & 0xFF00u);
}
__device__ __forceinline__ uint32_t six4(uint32_t x) {   // four code bytes -> 24 bits
    const uint32_t u = (x & 0x003F003Fu) | ((x >> 2) & 0x0FC00FC0u);
    return (u & 0xFFFu) | ((u >> 4) & 0xFFF000u);
}
__device__ __forceinline__ uint64_t quantize_pack8(const float v[8], int m, uint32_t &byte) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t b = __float_as_uint(v[i]) & 0x7fffffffu;
        a = a > b ? a : b;
    }
    a = quad_max_u32(a);
    const BlockScale bs = block_scale(a, m);
    byte = bs.byte;
    const float magic = 12582912.0f, cm = cmax_of(m);
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        b[i] = __float_as_uint(__builtin_amdgcn_fmed3f(__builtin_fmaf(v[i], bs.inv, magic), magic - cm, magic + cm));
    const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) | __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
    const uint32_t hi = __builtin_amdgcn_perm(b[5], b[4], 0x0C0C0400u) | __builtin_amdgcn_perm(b[7], b[6], 0x04000C0Cu);
    uint64_t w;
    if (m == 8) w = lo | ((uint64_t)hi << 32);
    else if (m == 6) w = six4(lo) | ((uint64_t)six4(hi) << 24);
    else w = nib4(lo) | (nib4(hi) << 16);
    return bs.bad ? 0 : w;
}

// ---------------------------------------------------------------- packing
// 4-bit: code i in bits 4i..4i+3 (byte h = c_2h | c_2h+1 << 4).
__device__ __forceinline__ uint32_t pack4(const int c[8]) {
    uint32_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= ((uint32_t)c[i] & 15u) << (4 * i);
    return w;
}
// 6-bit: two little-endian 24-bit words c0|c1<<6|c2<<12|c3<<18 (48 bits).
__device__ __forceinline__ uint64_t pack6(const int c[8]) {
    uint64_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (uint64_t)((uint32_t)c[i] & 63u) << (6 * i);
    return w;
}
__device__ __forceinline__ uint64_t pack8(const int c[8]) {
    uint64_t w = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) w |= (uint64_t)((uint32_t)c[i] & 255u) << (8 * i);
    return w;
}

// Store the low n bytes of w (n = 4, 6 or 8) at p with the widest stores the
// address alignment allows.
__device__ __forceinline__ void store_bytes(uint8_t *p, uint64_t w, int n) {
    uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (n == 8 && (a & 7) == 0) {
        *reinterpret_cast<uint64_t *>(p) = w;
    } else if (n != 6 && (a & 3) == 0) {
        for (int i = 0; i < n; i += 4) *reinterpret_cast<uint32_t *>(p + i) = (uint32_t)(w >> (8 * i));
    } else if ((a & 1) == 0) {
        for (int i = 0; i < n; i += 2) *reinterpret_cast<uint16_t *>(p + i) = (uint16_t)(w >> (8 * i));
    } else {
        for (int i = 0; i < n; ++i) p[i] = (uint8_t)(w >> (8 * i));
    }
}

// ---------------------------------------------------------------- gathers
// LDS budget of the row-staged gathers (the permutation as 16-bit indices
// plus one source row).
constexpr int64_t kStageLds = 96 * 1024;

// sperm[j] = perm[j] as 16 bits (an index outside [0, K) is clamped). With a
// 16-byte aligned permutation each thread takes 8 consecutive indices per
// pass (two 16-byte loads, one 16-byte LDS write) and issues the loads of up
// to 8 passes before writing, so the workgroup waits for one round trip
// instead of one per pass. K is a multiple of 32.
__device__ __forceinline__ void stage_perm(const int32_t *__restrict__ perm, int64_t K, uint16_t *sperm, int tid) {
    const uint32_t k = (uint32_t)K;
    auto clamp = [k](uint32_t v) { return v < k ? v : k - 1u; };
    if (reinterpret_cast<uintptr_t>(perm) % 16 == 0) {
        constexpr int kPasses = 8;
        for (int64_t j0 = 8 * (int64_t)tid; j0 < K; j0 += 2048 * kPasses) {
            uint4 v[kPasses][2];
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int64_t j = j0 + 2048 * p;
                if (j < K) {
                    v[p][0] = reinterpret_cast<const uint4 *>(perm + j)[0];
                    v[p][1] = reinterpret_cast<const uint4 *>(perm + j)[1];
                }
            }
#pragma unroll
            for (int p = 0; p < kPasses; ++p) {
                const int64_t j = j0 + 2048 * p;
                if (j < K)
                    *reinterpret_cast<uint4 *>(sperm + j) =
                        make_uint4(clamp(v[p][0].x) | (clamp(v[p][0].y) << 16), clamp(v[p][0].z) | (clamp(v[p][0].w) << 16),
                                   clamp(v[p][1].x) | (clamp(v[p][1].y) << 16), clamp(v[p][1].z) | (clamp(v[p][1].w) << 16));
            }
        }
    } else {
        for (int64_t j = tid; j < K; j += 256) sperm[j] = (uint16_t)clamp((uint32_t)perm[j]);
    }
}


// fp32 value 2^(byte - 127) of an E8M0 scale byte (0xFF -> +Inf, which turns
// the all-zero codes of a non-finite block into NaN in any product).
// Workgroup barrier for LDS hand-offs: waits only for this wave's LDS (and
// scalar) operations, so global loads issued before it stay in flight.
// (__syncthreads() also drains outstanding global loads.)
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Order key of an fp64 score: larger key = earlier rank. Total order on the
// bit pattern: NaN above +Inf above all finite values.
__device__ __forceinline__ uint64_t order_key(double s) {
    uint64_t u = (uint64_t)__double_as_longlong(s);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

}  // namespace mxs
