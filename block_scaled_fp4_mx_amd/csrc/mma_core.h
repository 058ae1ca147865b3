// Wave-level MMA cores shared by the dense GEMM and the grouped MoE GEMMs.
//
// A wave computes a 64x64 fp32 tile as 4x4 MFMA tiles of 16x16.  Row pointers
// are per lane: a_rows[i] points at the packed codes of the A row this lane
// feeds for row-fragment i (NULL for a row outside the problem, read as zeros),
// b_rows[j] likewise for B; the matching scale rows are a_srow / b_srow.
//
// MX: v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 operands; lane l carries the
// 32 K-values (16 bytes) of MX block (kb0 + l/16) of its row and that block's
// UE8M0 byte as its scale operand.  A and B use the same lane -> K mapping, so
// the product is independent of how the instruction orders K within a lane.
// NV: each lane expands 8 codes of its row (one 16-group) to bf16 code * s_g
// (exact: <= 6 significant bits) and feeds v_mfma_f32_16x16x32_bf16.
#pragma once

#include "fp4_internal.h"

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void zero_acc(v4f acc[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
}

// MX core over k (a multiple of 32; blocks past the end read as zero).
__device__ __forceinline__ void mma_mx_64x64(v4f acc[4][4], const uint8_t* const a_rows[4],
                                             const uint8_t* const a_srow[4], const uint8_t* const b_rows[4],
                                             const uint8_t* const b_srow[4], int64_t k, int lane) {
    const int64_t kb_total = k / 32;
    const int lk = lane >> 4;
    for (int64_t kb0 = 0; kb0 < kb_total; kb0 += 4) {
        const int64_t kb = kb0 + lk;
        const bool kin = kb < kb_total;
        v8i a[4], b[4];
        int sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 v = make_uint4(0, 0, 0, 0);
            int s = 127;
            if (kin && a_rows[i]) {
                v = *reinterpret_cast<const uint4*>(a_rows[i] + kb * 16);
                s = a_srow[i][kb];
            }
            a[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sa[i] = s;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 v = make_uint4(0, 0, 0, 0);
            int s = 127;
            if (kin && b_rows[j]) {
                v = *reinterpret_cast<const uint4*>(b_rows[j] + kb * 16);
                s = b_srow[j][kb];
            }
            b[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sb[j] = s;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0, sa[i],
                                                                               0, sb[j]);
    }
}

// W4A8 core over k (a multiple of 32; blocks past the end read as zero): B is
// MXFP4 as above (lane group g: block kb0 + g and its scale); A is MXFP8, whose
// 8-register operand in the mixed-format MFMA holds, for lane group g, the
// step's K values 16g .. 16g + 15 in bytes 0-15 and 64 + 16g .. 64 + 16g + 15
// in bytes 16-31 (measured on gfx950), while the scale operand of lane group g
// is still block kb0 + g's.  E4M3 (format 0) times E2M1 (format 4).
__device__ __forceinline__ void mma_w4a8_64x64(v4f acc[4][4], const uint8_t* const a_rows[4],
                                               const uint8_t* const a_srow[4], const uint8_t* const b_rows[4],
                                               const uint8_t* const b_srow[4], int64_t k, int lane) {
    const int64_t kb_total = k / 32;
    const int lk = lane >> 4;
    for (int64_t kb0 = 0; kb0 < kb_total; kb0 += 4) {
        const int64_t kb = kb0 + lk;
        const bool kin = kb < kb_total;
        const bool lo_in = kb0 + (lk >> 1) < kb_total, hi_in = kb0 + 2 + (lk >> 1) < kb_total;
        v8i a[4], b[4];
        int sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
            int s = 127;
            if (a_rows[i]) {
                const uint8_t* p = a_rows[i] + kb0 * 32 + lk * 16;
                if (lo_in) lo = *reinterpret_cast<const uint4*>(p);
                if (hi_in) hi = *reinterpret_cast<const uint4*>(p + 64);
                if (kin) s = a_srow[i][kb];
            }
            a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            sa[i] = s;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 v = make_uint4(0, 0, 0, 0);
            int s = 127;
            if (kin && b_rows[j]) {
                v = *reinterpret_cast<const uint4*>(b_rows[j] + kb * 16);
                s = b_srow[j][kb];
            }
            b[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sb[j] = s;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b[j], acc[i][j], 0, 4, 0, sa[i],
                                                                               0, sb[j]);
    }
}

// Expand 8 codes (one 32-bit word of one 16-group) with group scale s_g to bf16.
__device__ __forceinline__ bf16x8 expand_nv8(uint32_t codes, float sg) {
    u16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t cd = (codes >> (4 * i)) & 0xFu;
        const float v = __fmul_rn(e2m1_mag(cd & 7u), sg);
        r[i] = (unsigned short)((__float_as_uint(v) >> 16) | ((cd & 8u) << 12));
    }
    return __builtin_bit_cast(bf16x8, r);
}

// NV core over k (a multiple of 16; chunks past the end read as zero).
__device__ __forceinline__ void mma_nv_64x64(v4f acc[4][4], const uint8_t* const a_rows[4],
                                             const uint8_t* const a_srow[4], const uint8_t* const b_rows[4],
                                             const uint8_t* const b_srow[4], int64_t k, int lane) {
    const int64_t ch_total = k / 8;
    const int lk = lane >> 4;
    for (int64_t c0 = 0; c0 < ch_total; c0 += 4) {
        const int64_t ch = c0 + lk;
        const bool kin = ch < ch_total;
        bf16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t w = 0;
            float s = 0.f;
            if (kin && a_rows[i]) {
                w = reinterpret_cast<const uint32_t*>(a_rows[i])[ch];
                s = e4m3_value(a_srow[i][ch >> 1]);
            }
            a[i] = expand_nv8(w, s);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t w = 0;
            float s = 0.f;
            if (kin && b_rows[j]) {
                w = reinterpret_cast<const uint32_t*>(b_rows[j])[ch];
                s = e4m3_value(b_srow[j][ch >> 1]);
            }
            b[j] = expand_nv8(w, s);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

}  // namespace fp4
