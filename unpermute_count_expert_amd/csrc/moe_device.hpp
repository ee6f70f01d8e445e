// moe_device.hpp -- device-side numerics and helpers shared by the gfx950
// kernels of the MoE expert pipeline (bf16 rounding, OCP E4M3FN encoding,
// the pinned exp used by SiLU, wave helpers).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kGroup = 128;      // quantisation group / weight block edge
constexpr int kWave = 64;
constexpr int kMaxLocalExperts = 1024;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even; a NaN keeps its sign and top payload
// bits and is made quiet.  The gfx950 conversion (v_cvt_pk_bf16_f32) does
// exactly this: it matches the bit-level definition
//   NaN: (u >> 16) | 0x40,  otherwise: (u + 0x7fff + ((u >> 16) & 1)) >> 16
// on all 2^32 inputs.
typedef float moe_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 moe_bf2 __attribute__((ext_vector_type(2)));

// two values packed lo | hi << 16, one instruction
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    const moe_bf2 r = __builtin_convertvector((moe_f2){lo, hi}, moe_bf2);
    uint32_t u;
    __builtin_memcpy(&u, &r, 4);
    return u;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    return static_cast<uint16_t>(f32x2_to_bf16x2(v, 0.0f));
}

// Four fp32 -> four OCP E4M3FN codes packed little-endian in one dword,
// saturating: the hardware conversion rounds to nearest even but turns
// out-of-range values into the NaN code, so they are clamped to +-448
// first; NaN maps to 0x7F with its sign.
__device__ __forceinline__ uint32_t f32x4_to_e4m3(float a, float b, float c, float d) {
    float ca = __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
    float cb = __builtin_fminf(__builtin_fmaxf(b, -448.0f), 448.0f);
    float cc = __builtin_fminf(__builtin_fmaxf(c, -448.0f), 448.0f);
    float cd = __builtin_fminf(__builtin_fmaxf(d, -448.0f), 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cc, cd, w, true);
    uint32_t r = static_cast<uint32_t>(w);
    // NaN lanes: 0x7F | sign
    if (a != a) r = (r & 0xffffff00u) | ((__float_as_uint(a) >> 24) & 0x80u) | 0x7fu;
    if (b != b) r = (r & 0xffff00ffu) | ((((__float_as_uint(b) >> 24) & 0x80u) | 0x7fu) << 8);
    if (c != c) r = (r & 0xff00ffffu) | ((((__float_as_uint(c) >> 24) & 0x80u) | 0x7fu) << 16);
    if (d != d) r = (r & 0x00ffffffu) | ((((__float_as_uint(d) >> 24) & 0x80u) | 0x7fu) << 24);
    return r;
}

// The same encoding for values that are NaN or below 464 in magnitude, such
// as v * (448 / d) with d >= |v| (at most 448 * (1 + 2^-23)): without the
// clamp the hardware conversion gives the same codes there (checked on all
// 2^32 inputs), and the NaN repair runs only when a NaN is present.
__device__ __forceinline__ uint32_t f32x4_to_e4m3_bounded(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    uint32_t r = static_cast<uint32_t>(w);
    if (__builtin_expect((a != a) | (b != b) | (c != c) | (d != d), 0)) {
        if (a != a) r = (r & 0xffffff00u) | ((__float_as_uint(a) >> 24) & 0x80u) | 0x7fu;
        if (b != b) r = (r & 0xffff00ffu) | ((((__float_as_uint(b) >> 24) & 0x80u) | 0x7fu) << 8);
        if (c != c) r = (r & 0xff00ffffu) | ((((__float_as_uint(c) >> 24) & 0x80u) | 0x7fu) << 16);
        if (d != d) r = (r & 0x00ffffffu) | ((((__float_as_uint(d) >> 24) & 0x80u) | 0x7fu) << 24);
    }
    return r;
}

// Largest value among the 16 lanes of this lane's DPP row, returned to all
// 16, for values that are never NaN (so the hardware maximum is the plain
// larger value, as compare-select would give): lane pairs xor 1, xor 2
// (quad permutes), then the two quads of each half and the two halves (the
// half-row and row mirrors), one v_max_f32 with a DPP operand each.  The
// s_nop before each step covers the wait a DPP read of a VGPR written by the
// previous VALU instruction needs.
__device__ __forceinline__ float row16_max_nonnan(float m) {
    float r;
    asm volatile(
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
        "s_nop 1\n\t"
        "v_max_f32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf"
        : "=&v"(r)
        : "v"(m));
    return r;
}

// One 1x128 quantisation group held by 16 consecutive lanes, 8 values each
// (lane l owns group elements 8*(l mod 16) .. +7): amax over the group (the
// largest non-NaN magnitude, by compare-select, so quiet and signalling NaNs
// are both skipped), d = max(amax, 1e-10), scale = d / 448, inv = 448 / d,
// codes = e4m3(x * inv).  All 16 lanes of a group must call it together
// (the group max is a DPP maximum over the 16-lane row, no LDS involved);
// returns the scale.
__device__ __forceinline__ float quant_group16(const float (&x)[8], uint2& codes) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float a = __builtin_fabsf(x[i]);
        amax = a > amax ? a : amax;
    }
    amax = row16_max_nonnan(amax);   // the lane maxima are never NaN
    const float dd = __builtin_fmaxf(amax, 1e-10f);
    const float scale = dd / 448.0f;
    const float inv = 448.0f / dd;
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = x[i] * inv;
    // |t| <= 448 (1 + 2^-23) unless t is NaN: d >= every |x| of the group
    codes.x = f32x4_to_e4m3_bounded(t[0], t[1], t[2], t[3]);
    codes.y = f32x4_to_e4m3_bounded(t[4], t[5], t[6], t[7]);
    return scale;
}

// eight bf16 values (one 16-byte load) as fp32
__device__ __forceinline__ void bf16x8_to_f32(uint4 u, float (&v)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// Loads and stores of data that one kernel touches exactly once (rows read
// once, outputs written once): non-temporal, so the lines are not kept in
// the caches at the expense of data that is reused.
typedef int moe_i4 __attribute__((ext_vector_type(4)));
typedef int moe_i2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 load_once16(const void* p) {
    const moe_i4 q = __builtin_nontemporal_load(reinterpret_cast<const moe_i4*>(p));
    return uint4{(unsigned)q.x, (unsigned)q.y, (unsigned)q.z, (unsigned)q.w};
}
__device__ __forceinline__ void store_once16(void* p, const uint4& v) {
    __builtin_nontemporal_store(moe_i4{(int)v.x, (int)v.y, (int)v.z, (int)v.w}, reinterpret_cast<moe_i4*>(p));
}
__device__ __forceinline__ void store_once8(void* p, const uint2& v) {
    __builtin_nontemporal_store(moe_i2{(int)v.x, (int)v.y}, reinterpret_cast<moe_i2*>(p));
}

// exp for SiLU, fixed operation by operation so that it is reproducible:
// clamp to [-86, 88]; n = nearest-even(x / ln2); r = x - n*ln2 with ln2 in
// two parts (Cody-Waite); Horner over the Taylor coefficients 1/k!, k<=7;
// result p * 2^n.
__device__ __forceinline__ float exp_pinned(float x) {
    const float kLog2e = __uint_as_float(0x3fb8aa3bu);
    const float kLn2Hi = __uint_as_float(0x3f317200u);
    const float kLn2Lo = __uint_as_float(0x35bfbe8eu);
    float xc = __builtin_fminf(__builtin_fmaxf(x, -86.0f), 88.0f);
    float n = __builtin_rintf(xc * kLog2e);
    float r = __builtin_fmaf(-n, kLn2Hi, xc);
    r = __builtin_fmaf(-n, kLn2Lo, r);
    float p = __uint_as_float(0x39500d01u);                 // 1/7!
    p = __builtin_fmaf(p, r, __uint_as_float(0x3ab60b61u)); // 1/6!
    p = __builtin_fmaf(p, r, __uint_as_float(0x3c088889u)); // 1/5!
    p = __builtin_fmaf(p, r, __uint_as_float(0x3d2aaaabu)); // 1/4!
    p = __builtin_fmaf(p, r, __uint_as_float(0x3e2aaaabu)); // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_amdgcn_ldexpf(p, static_cast<int>(n));
}

// SiLU as the SiLU-mul requant defines it: g / (1 + exp(-g)) with the
// pinned exp and an IEEE division.
__device__ __forceinline__ float silu_pinned(float g) {
    const float e = exp_pinned(-g);
    return g / (1.0f + e);
}

// SiLU of a bf16 value is a function of its 16 bits: a table of the formula's
// own results for every bf16 g with 2^-12 <= |g| < 2^8 (both signs, 5120
// entries, 20 KB of LDS; entry (sign * kSiluExps + exponent - kSiluExpLo) *
// 128 + mantissa), built by the whole block; other g (zeros, tiny and huge
// values, infinities, NaN) take the formula itself, so a lookup returns the
// formula's bits for every g.
constexpr int kSiluExpLo = 127 - 12;
constexpr int kSiluExps = 20;
constexpr int kSiluHalf = kSiluExps * 128;
constexpr int kSiluEntries = 2 * kSiluHalf;

__device__ __forceinline__ void silu_table_build(float* tab) {
    for (int j = threadIdx.x; j < kSiluEntries; j += blockDim.x) {
        const bool neg = j >= kSiluHalf;
        const uint32_t hb = ((uint32_t)neg << 15) | (uint32_t)((kSiluExpLo << 7) + (neg ? j - kSiluHalf : j));
        tab[j] = silu_pinned(__uint_as_float(hb << 16));
    }
}

// silu of the bf16 value with bits hb
__device__ __forceinline__ float silu_bf16(const float* __restrict__ tab, uint32_t hb) {
    const uint32_t t = (hb & 0x7fffu) - (uint32_t)(kSiluExpLo << 7);
    if (__builtin_expect(t < (uint32_t)kSiluHalf, 1)) return tab[t + (hb >> 15) * kSiluHalf];
    return silu_pinned(__uint_as_float(hb << 16));
}

__device__ __forceinline__ int local_expert(int id, const int32_t* __restrict__ emap, int Eg, int El) {
    if (id < 0 || id >= Eg) return -1;
    int e = emap ? emap[id] : id;
    return (e >= 0 && e < El) ? e : -1;
}

// inclusive prefix sum over the 64 lanes of the wave
template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const T u = __shfl_up(v, d, kWave);
        if (lane >= d) v += u;
    }
    return v;
}

// The same for 32-bit values, without LDS: a Hillis-Steele scan inside each
// 16-lane DPP row (row shifts by 1, 2, 4 and 8; a lane whose source falls
// outside its row adds 0), then every row adds the totals of the rows before
// it (lane 15's value broadcast into rows 1 and 3, then lane 31's into rows 2
// and 3).  Every lane of the wave must call it.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

// And for 64-bit values: each step moves both 32-bit halves with the same DPP
// pattern and adds them as one 64-bit value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int64_t dpp_add64(int64_t v) {
    const uint64_t u = (uint64_t)v;
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)u, CTRL, ROW_MASK, 0xf, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(u >> 32), CTRL, ROW_MASK, 0xf, false);
    return (int64_t)(u + (((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ int64_t wave_inclusive_scan(int64_t v) {
    v = dpp_add64<0x111, 0xf>(v);   // row_shr:1
    v = dpp_add64<0x112, 0xf>(v);   // row_shr:2
    v = dpp_add64<0x114, 0xf>(v);   // row_shr:4
    v = dpp_add64<0x118, 0xf>(v);   // row_shr:8
    v = dpp_add64<0x142, 0xa>(v);   // row_bcast:15
    v = dpp_add64<0x143, 0xc>(v);   // row_bcast:31
    return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = threadIdx.x & (kWave - 1);
    return lane ? (~0ull >> (64 - lane)) : 0ull;
}

}  // namespace moe
