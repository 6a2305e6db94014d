// Device helpers shared by the activation pass and the GEMMs (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dq_internal.h"

namespace dq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));

// Formats of the scaled MFMA (cbsz / blgp field values).
constexpr int FMT_FP8 = 0;
constexpr int FMT_FP6 = 2;   // FP6 E2M3
constexpr int FMT_BF6 = 3;   // FP6 E3M2
constexpr int FMT_FP4 = 4;
constexpr int FMT_BF16 = 16;  // plain bf16 operands (the bf16-core ablation), not a scaled-MFMA format

// Scale exponent of an MX group (关键设计 4, quantizer definition, with the
// scale restricted to a power of two): the smallest e with
// amax <= q_max * 2^e.  With amax = m 2^E (1 <= m < 2) and
// q_max = c 2^Q, that is E - Q + [m > c]; zero and subnormal maxima give the
// floor -127.  Adding 2^23 - 1 - (c - 1) 2^23 to amax's bits carries into the
// exponent field exactly when the fraction exceeds c - 1, so the biased
// exponent field of the sum is E + 127 + [m > c], and e + 127 is that minus
// Q, saturated at 0 (the floor; also every subnormal and zero maximum).
//   FP4 E2M1 q_max = 1.5 2^2, FP8 E4M3 1.75 2^8, FP6 E2M3 1.875 2^2,
//   FP6 E3M2 1.75 2^4.
__device__ __forceinline__ int mx_exp_carry(float amax, uint32_t add, uint32_t q) {
    const uint32_t ef = (__float_as_uint(amax) + add) >> 23;
    return (int)__builtin_elementwise_sub_sat(ef, q) - 127;
}
__device__ __forceinline__ int mx_exp_fp4(float amax) { return mx_exp_carry(amax, 0x3fffffu, 2u); }
__device__ __forceinline__ int mx_exp_fp8(float amax) { return mx_exp_carry(amax, 0x1fffffu, 8u); }
__device__ __forceinline__ int mx_exp_fp6(float amax, bool e3m2) {
    return e3m2 ? mx_exp_carry(amax, 0x1fffffu, 4u) : mx_exp_carry(amax, 0x0fffffu, 2u);
}
// 2^e (-127 <= e <= 127) as a float operand of the scaled converts: the
// bits (e + 127) << 23, or for e = -127 the subnormal 0x00400000; every
// normal power's bits exceed 0x00400000, so that is the unsigned maximum.
__device__ __forceinline__ float pow2f(int e) {
    return __uint_as_float(max((uint32_t)(e + 127) << 23, 0x00400000u));
}

// 32 fp32 values -> 32 FP4 E2M1 codes (16 bytes, element 2i in the low
// nibble of byte i), each v / 2^e rounded to nearest even by the hardware
// converter.
__device__ __forceinline__ uint4 encode_fp4x32(const float* v, float scale) {
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        int w = i >> 2;
        switch (i & 3) {
            case 0: d[w] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d[w], v[2 * i], v[2 * i + 1], scale, 0); break;
            case 1: d[w] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d[w], v[2 * i], v[2 * i + 1], scale, 1); break;
            case 2: d[w] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d[w], v[2 * i], v[2 * i + 1], scale, 2); break;
            default: d[w] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d[w], v[2 * i], v[2 * i + 1], scale, 3); break;
        }
    }
    return make_uint4(d[0], d[1], d[2], d[3]);
}

// 32 fp32 values -> 32 FP8 E4M3 codes (two 16-byte halves), v / 2^e rounded
// to nearest even by the hardware converter.
__device__ __forceinline__ void encode_fp8x32(const float* v, float scale, uint4& lo, uint4& hi) {
    uint32_t d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v2s z = {0, 0};
        v2s a = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, v[4 * i], v[4 * i + 1], scale, false);
        v2s b = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(a, v[4 * i + 2], v[4 * i + 3], scale, true);
        d[i] = __builtin_bit_cast(uint32_t, b);
    }
    lo = make_uint4(d[0], d[1], d[2], d[3]);
    hi = make_uint4(d[4], d[5], d[6], d[7]);
}

// 32 fp32 values -> 32 FP6 codes (E2M3, or E3M2), v / 2^e rounded to nearest
// even by the hardware converter, packed six bits each in order (value i at
// bits [6 i, 6 i + 6) of d[0..5]).  The converter interleaves its two
// 16-value sources (output value 2 j from the first, 2 j + 1 from the
// second), so the even-indexed values go first and the odd ones second.
__device__ __forceinline__ void encode_fp6x32(const float* v, float scale, bool e3m2, uint32_t* d) {
    v16f ev, od;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        ev[j] = v[2 * j];
        od[j] = v[2 * j + 1];
    }
    typedef unsigned v6u __attribute__((ext_vector_type(6)));
    const v6u w = e3m2 ? __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(ev, od, scale)
                       : __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, scale);
#pragma unroll
    for (int i = 0; i < 6; ++i) d[i] = w[i];
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Slot layout: cube k owns slots [k S, k S + S); slot k S + (dt h + dh) w + dw
// holds token (kt t + dt, kh h + dh, kw w + dw) if that lies in the grid,
// else it is a pad slot (-1).  Within a cube the slots run in lexicographic
// (dt, dh, dw) order.
__device__ __forceinline__ long long slot_token(const Geom& g, long long slot) {
    long long k = slot / g.S;
    int s = (int)(slot - k * g.S);
    int dw = s % g.w;
    int dh = (s / g.w) % g.h;
    int dt = s / (g.w * g.h);
    long long kw = k % g.Wc;
    long long kh = (k / g.Wc) % g.Hc;
    long long kt = k / ((long long)g.Wc * g.Hc);
    long long ti = kt * g.t + dt, hi = kh * g.h + dh, wi = kw * g.w + dw;
    if (k >= g.K || ti >= g.T || hi >= g.H || wi >= g.W) return -1;
    return (ti * g.H + hi) * g.W + wi;
}

// Token count of cube k (clipped at the high ends of the grid).
__device__ __forceinline__ int cube_count(const Geom& g, long long k, int* ct, int* ch, int* cw) {
    long long kw = k % g.Wc;
    long long kh = (k / g.Wc) % g.Hc;
    long long kt = k / ((long long)g.Wc * g.Hc);
    *ct = (int)min((long long)g.t, g.T - kt * g.t);
    *ch = (int)min((long long)g.h, g.H - kh * g.h);
    *cw = (int)min((long long)g.w, g.W - kw * g.w);
    return *ct * *ch * *cw;
}

// 1 / cnt for a power of two cnt (1 .. 2^126), built from its exponent bits:
// exact, and a few instructions instead of an IEEE division.
__device__ __forceinline__ float inv_pow2(int cnt) {
    return __uint_as_float((uint32_t)(127 - __builtin_ctz((unsigned)cnt)) << 23);
}

// Correctly rounded s / cnt: exact for cnt = 1 and powers of two (a
// power-of-two scaling), IEEE division otherwise.
__device__ __forceinline__ float mean_div(float s, int cnt) {
    if ((cnt & (cnt - 1)) == 0) return s * inv_pow2(cnt);
    return __fdiv_rn(s, (float)cnt);
}

}  // namespace dq
