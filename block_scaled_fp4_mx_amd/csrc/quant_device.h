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

// MXFP8 (E4M3 elements, UE8M0 scale per 32) for the W4A8 activations: the
// block exponent is E = floor(log2 amax) - 8, 8 being E4M3's largest exponent,
// so the block maximum lands in [256, 512) and saturates at 448 when above it.
// From the amax's exponent field e: byte = E + 127 = e - 8, clamped at 0.
__device__ __forceinline__ uint32_t mxfp8_scale_byte(uint32_t amax_bits) {
    const uint32_t e = amax_bits >> 7;
    return e > 8u ? e - 8u : 0u;
}

// E4M3 magnitude byte of an exactly known fp32 value 0 <= v < 512, nearest
// even, saturating at 448 (byte 0x7E).  Below 2^-6 the grid is the subnormal
// one, multiples of 2^-9 (v * 512 is exact and rint rounds to even).  From
// 2^-6 on, rounding v's fp32 pattern to 3 mantissa bits (add half an ulp of
// the kept bits minus one, plus the kept lsb, then truncate) leaves
// exponent:mantissa in bits 30:20 with any carry moved into the exponent; the
// E4M3 byte is that field with the exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_byte_f32(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t sub = (uint32_t)__builtin_rintf(v * 512.0f);
    const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
    const uint32_t nrm = min(r - (120u << 3), 0x7Eu);
    return b < 0x3C800000u ? sub : nrm;
}

// MXFP8: quantize this lane's 8 elements (a quad of lanes is one block) to 8
// E4M3 bytes (element i in byte i) and the block's UE8M0 byte.  |x| * 2^-E is
// exact in fp32 whenever it is at least 2^-10 (a bf16 value times a power of
// two stays exact down to fp32's subnormal range); smaller ones round to 0
// either way.  The sign bit of x is copied, so -0 gives 0x80.
__device__ __forceinline__ uint2 mxfp8_quant8(const uint32_t w[4], uint32_t& sbyte) {
    uint32_t am = mag_max8(w);
    am = max(am, quad_swap1(am));
    am = max(am, quad_swap2(am));
    sbyte = mxfp8_scale_byte(am);
    const float inv = __uint_as_float((254u - sbyte) << 23);     // 2^(127 - byte) = 2^-E
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        const float v = __fmul_rn(__uint_as_float((h & 0x7FFFu) << 16), inv);
        const uint32_t byte = e4m3_byte_f32(v) | ((h >> 8) & 0x80u);
        out[i >> 2] |= byte << (8 * (i & 3));
    }
    return make_uint2(out[0], out[1]);
}

// E4M3 byte of an E2M1 code (lossless: E2M1 values are E4M3 values).  From the
// fields: index e*2 + m with e > 0 is (1 + m/2) 2^(e-1), E4M3 exponent field
// e + 6 and mantissa m << 2; index 1 is 0.5 = 2^-1 (field 6); index 0 is 0.
__device__ __forceinline__ uint32_t e2m1_to_e4m3(uint32_t c) {
    const uint32_t i = c & 7u, e = i >> 1, m = i & 1u;
    const uint32_t mag = e ? (((e + 6u) << 3) | (m << 2)) : (m ? 48u : 0u);
    return mag | ((c & 8u) << 4);
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

// ------------------------------------------------------------------ NV, one lane per 16-group
// E4M3 byte of q ~ amax_g / (6 s_t), given as q' = amax_g * inv6st with inv6st
// the fp64 rounding of 1 / (6 s_t): q' is within 3 fp64 ulp of q.  The exact q
// is either an E4M3 rounding midpoint or at least 2^-32 q away from every one
// (8-bit numerator over a 26-bit denominator against 5-bit midpoints), so the
// rounding of q' agrees with that of q except at an exact midpoint, where q'
// lies within a few ulp of it: such a q' is taken as the tie and goes to the
// even mantissa.  Rounding works on the fp64 bit pattern: above 2^-6 the byte is
// (biased exponent, top 3 mantissa bits) rebased by (1023 - 7) * 8, and a
// round-up carry into the exponent gives the next binade; below 2^-6 the unit is
// 2^-9 and n = 8 (rounded up from the top subnormal) is byte 0x08 = 2^-6.
__device__ __forceinline__ uint32_t e4m3_rne_sat_near(double q) {
    if (!(q > 0.0)) return 0u;
    if (q >= 448.0) return 0x7Eu;
    const uint64_t b = (uint64_t)__double_as_longlong(q);
    const int e = (int)(b >> 52) - 1023;
    uint64_t n, rem, half;
    bool normal = e >= -6;
    if (normal) {
        n = b >> 49;
        rem = b & ((1ull << 49) - 1);
        half = 1ull << 48;
    } else {
        const uint64_t mant = (b & ((1ull << 52) - 1)) | (1ull << 52);   // q = mant * 2^(e - 52)
        const int sh = 52 - (e + 9);                                    // q * 2^9 = mant >> sh (+ rem)
        if (sh >= 63) return 0u;                                        // q < 2^-19: far below 2^-10
        n = mant >> sh;
        rem = mant & ((1ull << sh) - 1);
        half = 1ull << (sh - 1);
    }
    const int64_t dlt = (int64_t)(rem - half);
    const bool up = dlt > 4 || (dlt >= -4 && (n & 1u));
    n += up ? 1u : 0u;
    const uint32_t byte = normal ? (uint32_t)(n - ((uint64_t)(1023 - 7) << 3)) : (uint32_t)n;
    return min(byte, 0x7Eu);
}

// Largest magnitude (bf16 bits, sign cleared) of the 16 elements held as 8
// words, with packed 16-bit integer maxima.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t amax16_bits(const uint32_t w[8]) {
    u16x2_t m = __builtin_bit_cast(u16x2_t, w[0] & 0x7FFF7FFFu);
#pragma unroll
    for (int i = 1; i < 8; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[i] & 0x7FFF7FFFu));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// Group-scale byte of a 16-group from its largest magnitude.  Fast path
// (valid when inv32 = fp32(1 / (6 s_t)) is a normal fp32 value): p = amax * inv32
// is within 2^-23 of q relative, i.e. within 2 fp32 ulp, so unless p lies within
// 4 ulp of an E4M3 rounding midpoint its rounding (done on the fp32 bit pattern,
// or on 512 p below 2^-6) is that of q.  The fast path is branch-free; a lane
// near a midpoint (or without a valid inv32) takes the fp64 path above.
__device__ __forceinline__ uint32_t nv_group_scale(uint32_t am_bits, float inv32, double inv64, bool fast) {
    const float a = __uint_as_float(am_bits << 16);
    const float p = __fmul_rn(a, inv32);
    const uint32_t b = __float_as_uint(p);
    const int32_t dn = (int32_t)(b & 0xFFFFFu) - 0x80000;
    const uint32_t byte_n = (b >> 20) + (dn > 0 ? 1u : 0u) - (120u << 3);
    const float t = __fmul_rn(p, 512.0f);               // below 2^-6: exact, t < 8, ulp(t) <= 2^-21
    const float fl = floorf(t);
    const float fr = t - fl;                              // exact
    const uint32_t byte_s = (uint32_t)fl + (fr > 0.5f ? 1u : 0u);
    const bool normal = p >= 0x1p-6f;
    const bool near = normal ? (dn <= 4 && dn >= -4) : (fabsf(fr - 0.5f) <= 0x1p-19f);
    uint32_t sg = p >= 448.0f ? 0x7Eu : min(normal ? byte_n : byte_s, 0x7Eu);
    if (am_bits == 0u || !(inv64 > 0.0)) sg = 0u;
    else if (!fast || near) sg = e4m3_rne_sat_near((double)a * inv64);
    return sg;
}

// Per-workgroup constants of one NV tensor scale s_t > 0: for every group-scale
// byte g in 1..126, the fp32 factors bracketing r = 1 / (v(g) s_t) from below
// and above: r (1 - 2^-22) and r (1 + 2^-22).  Byte 0 has {0, 0}: the products
// are signed zeros, whose codes (sign | 0) are the right ones.  When r is too
// large for fp32 products to stay finite the entry is {0, inf}: the two codes
// of any nonzero element then differ, which sends it to the exact path.
struct NvRecip {
    float lo, hi;
};

// inv_st = 1 / s_t in fp64; 1 / v(g) = 2^(7 - e) * 8 / (8 + m) for a normal byte
// (e, m) and 2^9 / m for a subnormal one, so r is a product of fp64 factors
// with a relative error near 2^-52, far inside the 2^-22 bracket.
__device__ __forceinline__ NvRecip nv_recip_entry(uint32_t g, double inv_st) {
    const uint32_t e = (g >> 3) & 15u, m = g & 7u;
    const double r = e ? ldexp(inv_st * (8.0 / (double)(8u + m)), 7 - (int)e) : inv_st * (512.0 / (double)m);
    if (!(r < 1.0e37)) return NvRecip{0.0f, __builtin_inff()};
    return NvRecip{(float)(r * (1.0 - 0x1p-22)), (float)(r * (1.0 + 0x1p-22))};
}

// Element i (0..15) of a 16-group held as 8 bf16 words, as fp32 bits.
__device__ __forceinline__ uint32_t group_elem_bits(const uint32_t w[8], uint32_t i) {
    const uint32_t j = i >> 1;
    const uint32_t a = (j & 1) ? w[1] : w[0], b = (j & 1) ? w[3] : w[2];
    const uint32_t c = (j & 1) ? w[5] : w[4], d = (j & 1) ? w[7] : w[6];
    const uint32_t lo = (j & 2) ? b : a, hi = (j & 2) ? d : c;
    const uint32_t word = (j & 4) ? hi : lo;
    return (i & 1) ? (word & 0xFFFF0000u) : (word << 16);
}

// Bit 4i set where nibble i of x is nonzero.
__device__ __forceinline__ uint32_t nibble_flags(uint32_t x) {
    x |= x >> 2;
    x |= x >> 1;
    return x & 0x11111111u;
}

// Codes of one 16-group held as 8 bf16 words (w[i] = elements 2i, 2i+1), with
// its group-scale byte; element i goes to bits 4i..4i+3 of the 64-bit result.
// The fp32 products x * lo < x / d < x * hi (d = v(g) s_t) bracket the exact
// quotient within 2^-21, so where their nearest-even E2M1 codes agree that code
// is the exact one.  Where they differ, exactly one E2M1 midpoint m lies between
// them (the two codes are neighbours) and |x| is compared with m d exactly in
// fp64 (a tie goes to the even index).  Such near-ties are common: with
// s_t = amax_t / 2688, amax_g / (6 s_t) is often within 2^-24 of an E4M3 value,
// and bf16 elements often stand in small-integer ratios to the group maximum.
// A group whose bracket is not finite (tiny d) compares with all midpoints.
__device__ __forceinline__ uint2 nv_codes16(const uint32_t w[8], uint32_t sg, double st, NvRecip rc) {
    float lo[16], hi[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float x = (i & 1) ? __uint_as_float(w[i >> 1] & 0xFFFF0000u) : __uint_as_float(w[i >> 1] << 16);
        lo[i] = __fmul_rn(x, rc.lo);
        hi[i] = __fmul_rn(x, rc.hi);
    }
    if (sg == 0x7Eu) {   // saturated group scale: quotients may exceed the fp32 range; clamp at 8
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            lo[i] = __builtin_amdgcn_fmed3f(lo[i], -8.0f, 8.0f);
            hi[i] = __builtin_amdgcn_fmed3f(hi[i], -8.0f, 8.0f);
        }
    }
    uint32_t pl[2];
    pl[0] = cvt8_f32(lo);
    pl[1] = cvt8_f32(lo + 8);
    uint64_t flags = (uint64_t)nibble_flags(pl[0] ^ cvt8_f32(hi)) | ((uint64_t)nibble_flags(pl[1] ^ cvt8_f32(hi + 8)) << 32);
    if (flags) {
        const double d = (double)e4m3_value(sg) * st;
        const bool neighbours = rc.lo != 0.0f;
        do {
            const uint32_t i = (uint32_t)__builtin_ctzll(flags) >> 2;
            flags &= flags - 1;
            const uint32_t xb = group_elem_bits(w, i);
            const double ax = fabs((double)__uint_as_float(xb));
            const uint32_t sh = 4 * (i & 7);
            uint32_t& word = (i & 8) ? pl[1] : pl[0];
            uint32_t idx;
            if (neighbours) {
                const uint32_t cl = (word >> sh) & 7u;
                const double t = 0.5 * ((double)e2m1_mag(cl) + (double)e2m1_mag(cl + 1u)) * d;
                idx = cl + ((ax > t || (ax == t && (cl & 1u))) ? 1u : 0u);
            } else {
                idx = 0;
                for (uint32_t j = 0; j < 7; ++j) {
                    const double t = 0.5 * ((double)e2m1_mag(j) + (double)e2m1_mag(j + 1)) * d;
                    idx += ((j & 1u) ? (ax >= t) : (ax > t)) ? 1u : 0u;
                }
            }
            word = (word & ~(0xFu << sh)) | ((((xb >> 28) & 8u) | idx) << sh);
        } while (flags);
    }
    return make_uint2(pl[0], pl[1]);
}

}  // namespace fp4
