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
#include "mma_core.h"

namespace fp4 {
namespace {

constexpr int kBM = 128, kBN = 128, kThreads = 256;

// 16x16 accumulator layout: lane holds rows 4*(lane/16) + r, column lane % 16.
__device__ __forceinline__ void store_tile(const v4f acc[4][4], void* c, int c_f32, int64_t ldc, int64_t m,
                                           int64_t n, int64_t m0, int64_t n0, int lane, float scale) {
    const int lr = lane & 15, lk = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + i * 16 + lk * 4 + r, col = n0 + j * 16 + lr;
                if (row < m && col < n) {
                    const float v = __fmul_rn(acc[i][j][r], scale);
                    if (c_f32)
                        static_cast<float*>(c)[row * ldc + col] = v;
                    else
                        static_cast<uint16_t*>(c)[row * ldc + col] = (uint16_t)f32_to_bf16_rne(v);
                }
            }
}

// Block tile 128x128: four waves in a 2x2 grid, each a 64x64 MMA core.
template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    int64_t m, int64_t n, int64_t k, void* __restrict__ c, int c_f32, int64_t ldc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kBM + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * kBN + (wave & 1) * 64;
    const int blk = FMT == FP4_FMT_MX ? 32 : 16;
    const int lr = lane & 15;
    const uint8_t *a_rows[4], *a_srow[4], *b_rows[4], *b_srow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = m0 + i * 16 + lr;
        a_rows[i] = r < m ? ac + r * (k / 2) : nullptr;
        a_srow[i] = r < m ? as + r * (k / blk) : nullptr;
        const int64_t q = n0 + i * 16 + lr;
        b_rows[i] = q < n ? bc + q * (k / 2) : nullptr;
        b_srow[i] = q < n ? bs + q * (k / blk) : nullptr;
    }
    v4f acc[4][4];
    zero_acc(acc);
    float scale = 1.0f;
    if (FMT == FP4_FMT_MX) {
        mma_mx_64x64(acc, a_rows, a_srow, b_rows, b_srow, k, lane);
    } else {
        mma_nv_64x64(acc, a_rows, a_srow, b_rows, b_srow, k, lane);
        scale = __fmul_rn(*ats, *bts);
    }
    store_tile(acc, c, c_f32, ldc, m, n, m0, n0, lane, scale);
}

}  // namespace

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s) {
    dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
    gemm_kernel<FP4_FMT_MX><<<grid, kThreads, 0, s>>>(ac, as, nullptr, bc, bs, nullptr, m, n, k, c, c_f32, ldc);
    return hipGetLastError();
}

hipError_t launch_gemm_nv(const uint8_t* ac, const uint8_t* as, const float* ats,
                          const uint8_t* bc, const uint8_t* bs, const float* bts,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s) {
    dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
    gemm_kernel<FP4_FMT_NV><<<grid, kThreads, 0, s>>>(ac, as, ats, bc, bs, bts, m, n, k, c, c_f32, ldc);
    return hipGetLastError();
}

}  // namespace fp4
