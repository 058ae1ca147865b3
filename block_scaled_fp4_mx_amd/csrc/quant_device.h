// Per-lane MX / NV quantizers shared by the standalone quantize kernels and the
// MoE gate/up epilogue.  A lane owns 8 consecutive bf16 elements (4 words); an
// MX block of 32 is 4 consecutive, 4-aligned lanes and an NV group of 16 is 2
// consecutive, 2-aligned lanes, so block maxima combine with DPP quad permutes.
// All lanes of a quad must be active.
#pragma once

#include "fp4_internal.h"

namespace fp4 {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// DPP quad permutations: lane i of each group of 4 reads lane perm[i].
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {   // (1,0,3,2)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {   // (2,3,0,1)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}

// Largest 15-bit magnitude of the two bf16 halves of a word (integer order of
// finite magnitudes is their numeric order).
__device__ __forceinline__ uint32_t mag_max2(uint32_t w) {
    return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

__device__ __forceinline__ uint32_t mag_max8(const uint32_t w[4]) {
    return max(max(mag_max2(w[0]), mag_max2(w[1])), max(mag_max2(w[2]), mag_max2(w[3])));
}

// MX block exponent byte from the block's largest magnitude bits: the biased
// exponent field e of amax gives floor(log2 amax) = e - 127 for normal amax, so
// E = e - 129 and the byte E + 127 = e - 2, clamped at 0 (zero and subnormal
// amax, whose floor(log2) is below -126, clamp to E = -127 as well).
__device__ __forceinline__ uint32_t mx_scale_byte(uint32_t amax_bits) {
    const uint32_t e = amax_bits >> 7;
    return e > 2u ? e - 2u : 0u;
}

// MX: quantize this lane's 8 elements; returns the packed codes (element i in
// bits 4i..4i+3) and the block's UE8M0 byte.  The conversion instruction
// divides by the power of two held in its scale operand's exponent field and
// rounds to nearest even onto E2M1 with saturation; an operand whose exponent
// field is the scale byte (mantissa 0) is exactly 2^E, including byte 0, which
// the instruction reads as 2^-127.
__device__ __forceinline__ uint32_t mx_quant8(const uint32_t w[4], uint32_t& sbyte) {
    uint32_t am = mag_max8(w);
    am = max(am, quad_swap1(am));
    am = max(am, quad_swap2(am));
    sbyte = mx_scale_byte(am);
    const float sc = __uint_as_float(sbyte << 23);
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[0]), sc, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[1]), sc, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[2]), sc, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(p, __builtin_bit_cast(bf16x2_t, w[3]), sc, 3);
    return p;
}

// Four fp32 pairs -> 8 E2M1 codes, round to nearest even (scale 1.0 = 2^0).
__device__ __forceinline__ uint32_t cvt8_f32(const float v[8]) {
    uint32_t p = 0;
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0], v[1], 1.0f, 0);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2], v[3], 1.0f, 1);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4], v[5], 1.0f, 2);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6], v[7], 1.0f, 3);
    return p;
}

__device__ __forceinline__ float bf16_elem(const uint32_t w[4], int i) {
    return (i & 1) ? __uint_as_float(w[i >> 1] & 0xFFFF0000u) : __uint_as_float(w[i >> 1] << 16);
}

// NV group scale byte: E4M3 of amax_g / (6 s_t), the fp64 quotient being
// correctly rounded and far enough from every E4M3 midpoint for the second
// rounding to be exact (8-bit over <= 26-bit operands).
__device__ __forceinline__ uint32_t nv_scale_byte(uint32_t amax_bits, double st) {
    if (!(st > 0.0)) return 0u;
    const double amax = (double)__uint_as_float(amax_bits << 16);
    return e4m3_rne_sat(amax / (6.0 * st));
}

// NV: quantize this lane's 8 elements given s_t; returns packed codes and the
// group's E4M3 byte.  With d = s_g s_t (exact in fp64) and r = 1/d, the fp32
// products x * r(1 - 2^-22) and x * r(1 + 2^-22) bracket the exact quotient
// x / d strictly, so where their nearest-even E2M1 codes agree that code is the
// exact one.  Where they differ the quotient lies within 2^-21 of the midpoint
// between the two candidates, and |x| is compared with midpoint * d exactly in
// fp64 (ties to the even index).
__device__ __forceinline__ uint32_t nv_quant8(const uint32_t w[4], double st, uint32_t& sg) {
    uint32_t am = mag_max8(w);
    am = max(am, quad_swap1(am));
    sg = nv_scale_byte(am, st);
    if (sg == 0u) {
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            p |= ((b >> 12) & 8u) << (4 * i);
        }
        return p;
    }
    const double d = (double)e4m3_value(sg) * st;
    const double r = 1.0 / d;
    const bool finite = r < 1.0e37;
    const float r_lo = finite ? (float)(r * (1.0 - 0x1p-22)) : 0.0f;
    const float r_hi = finite ? (float)(r * (1.0 + 0x1p-22)) : 0.0f;
    float lo[8], hi[8];
    if (sg == 0x7Eu) {
        // saturated group scale: quotients may exceed fp32 range; clamp at 8
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = bf16_elem(w, i);
            lo[i] = __builtin_amdgcn_fmed3f(__fmul_rn(x, r_lo), -8.0f, 8.0f);
            hi[i] = __builtin_amdgcn_fmed3f(__fmul_rn(x, r_hi), -8.0f, 8.0f);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = bf16_elem(w, i);
            lo[i] = __fmul_rn(x, r_lo);
            hi[i] = __fmul_rn(x, r_hi);
        }
    }
    const uint32_t plo = cvt8_f32(lo);
    const uint32_t phi = cvt8_f32(hi);
    uint32_t p = plo;
    uint32_t diff = finite ? (plo ^ phi) : 0x77777777u;
    if (diff) {
#pragma unroll 1
        for (int i = 0; i < 8; ++i) {
            if (((diff >> (4 * i)) & 7u) == 0u) continue;
            const float x = bf16_elem(w, i);
            const double ad = fabs((double)x);
            uint32_t idx = 0;
            for (uint32_t j = 0; j < 7; ++j) {
                const double t = 0.5 * ((double)e2m1_mag(j) + (double)e2m1_mag(j + 1)) * d;
                idx += ((j & 1u) ? (ad >= t) : (ad > t)) ? 1u : 0u;
            }
            const uint32_t code = ((__float_as_uint(x) >> 28) & 8u) | idx;
            p = (p & ~(0xFu << (4 * i))) | (code << (4 * i));
        }
    }
    return p;
}

}  // namespace fp4
