// W4A4 GEMM kernels for gfx950: C[m, n] = sum_k A_hat[m, k] B_hat[n, k].
//
// MX: both operands feed v_mfma_scale_f32_16x16x128_f8f6f4 as E2M1 with their
// UE8M0 block scales; every lane of the MFMA carries 32 consecutive K values of
// one row (one MX block) and that block's scale byte, so the matrix core applies
// the per-block scale correction that the W4A4 description calls for
// ("DeepSeek-V4.1-Flash-NVFP4" explainer, section 2).  A and B fragments are
// loaded with the same lane -> K mapping, so the product does not depend on the
// order in which the instruction walks K inside a fragment.
//
// NV: E4M3 scales on 16-element groups are not a matrix-core scale format, so
// each lane expands its 8 codes to bf16 values code * s_g (exact: at most 6
// significant bits) and uses v_mfma_f32_16x16x32_bf16; the two fp32 tensor
// scales multiply the fp32 accumulator at the end.
#include "fp4_internal.h"

namespace fp4 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 128, kBN = 128, kThreads = 256;

__device__ __forceinline__ void store_c(void* c, int c_f32, int64_t ldc, int64_t m, int64_t n,
                                        int64_t row, int64_t col, float v) {
    if (row < m && col < n) {
        if (c_f32)
            static_cast<float*>(c)[row * ldc + col] = v;
        else
            static_cast<uint16_t*>(c)[row * ldc + col] = (uint16_t)f32_to_bf16_rne(v);
    }
}

// ------------------------------------------------------------------ MX
// Block tile 128x128, four waves in a 2x2 grid, each wave 64x64 as 4x4 MFMA
// tiles of 16x16; K advances 128 values (4 MX blocks) per step.
__global__ __launch_bounds__(kThreads) void gemm_mx_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs,
    int64_t m, int64_t n, int64_t k, void* __restrict__ c, int c_f32, int64_t ldc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kBM + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * kBN + (wave & 1) * 64;
    const int64_t kb_total = k / 32;                     // MX blocks per row
    const int64_t row_bytes = k / 2;
    const int lr = lane & 15, lk = lane >> 4;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int64_t kb0 = 0; kb0 < kb_total; kb0 += 4) {
        const int64_t kb = kb0 + lk;
        const bool kin = kb < kb_total;
        v8i a[4], b[4];
        int sa[4], sb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = m0 + i * 16 + lr;
            uint4 v = make_uint4(0, 0, 0, 0);
            int s = 127;
            if (kin && r < m) {
                v = *reinterpret_cast<const uint4*>(ac + r * row_bytes + kb * 16);
                s = as[r * kb_total + kb];
            }
            a[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sa[i] = s;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = n0 + j * 16 + lr;
            uint4 v = make_uint4(0, 0, 0, 0);
            int s = 127;
            if (kin && r < n) {
                v = *reinterpret_cast<const uint4*>(bc + r * row_bytes + kb * 16);
                s = bs[r * kb_total + kb];
            }
            b[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
            sb[j] = s;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    a[i], b[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
    }
    // 16x16 accumulator layout: lane holds rows 4*(lane/16) + r, column lane % 16
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_c(c, c_f32, ldc, m, n, m0 + i * 16 + lk * 4 + r, n0 + j * 16 + lr, acc[i][j][r]);
}

// ------------------------------------------------------------------ NV
// Expand 8 codes (one 32-bit word) of one 16-group with scale s_g to bf16
// code * s_g.  The product has at most 6 significant bits, so the fp32 product
// is exact and truncating it to bf16 is exact.
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

__global__ __launch_bounds__(kThreads) void gemm_nv_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    int64_t m, int64_t n, int64_t k, void* __restrict__ c, int c_f32, int64_t ldc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kBM + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * kBN + (wave & 1) * 64;
    const int64_t k8_total = k / 8;                      // 8-element chunks per row
    const int64_t g_total = k / 16;
    const int64_t row_words = k / 8;                     // 32-bit words of codes per row
    const int lr = lane & 15, lk = lane >> 4;

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int64_t c0 = 0; c0 < k8_total; c0 += 4) {       // 32 K values per step
        const int64_t ch = c0 + lk;
        const bool kin = ch < k8_total;
        bf16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = m0 + i * 16 + lr;
            uint32_t w = 0;
            float s = 0.f;
            if (kin && r < m) {
                w = reinterpret_cast<const uint32_t*>(ac)[r * row_words + ch];
                s = e4m3_value(as[r * g_total + (ch >> 1)]);
            }
            a[i] = expand_nv8(w, s);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t r = n0 + j * 16 + lr;
            uint32_t w = 0;
            float s = 0.f;
            if (kin && r < n) {
                w = reinterpret_cast<const uint32_t*>(bc)[r * row_words + ch];
                s = e4m3_value(bs[r * g_total + (ch >> 1)]);
            }
            b[j] = expand_nv8(w, s);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    const float st = __fmul_rn(*ats, *bts);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_c(c, c_f32, ldc, m, n, m0 + i * 16 + lk * 4 + r, n0 + j * 16 + lr,
                        __fmul_rn(acc[i][j][r], st));
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s) {
    dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
    gemm_mx_kernel<<<grid, kThreads, 0, s>>>(ac, as, bc, bs, m, n, k, c, c_f32, ldc);
    return hipGetLastError();
}

hipError_t launch_gemm_nv(const uint8_t* ac, const uint8_t* as, const float* ats,
                          const uint8_t* bc, const uint8_t* bs, const float* bts,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s) {
    dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
    gemm_nv_kernel<<<grid, kThreads, 0, s>>>(ac, as, ats, bc, bs, bts, m, n, k, c, c_f32, ldc);
    return hipGetLastError();
}

}  // namespace fp4
