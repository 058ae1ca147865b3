// Internal declarations shared by the library's translation units: device
// helpers for the E2M1 / E4M3 / UE8M0 encodings and the host launchers that the
// C ABI (api.cpp) dispatches to.  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4.h"

namespace fp4 {

// ------------------------------------------------------------------ device helpers
// E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 ("DeepSeek-V4.1-Flash-NVFP4"
// explainer, section 2) indexed by the low 3 bits of a code.
__device__ __forceinline__ float e2m1_mag(uint32_t idx) {
    // 2-bit exponent e, 1-bit mantissa m: e == 0 -> m * 0.5, else (1 + m/2) * 2^(e-1).
    // Built from the fields: for e > 0 the fp32 pattern is exponent (e - 1 + 127)
    // and mantissa m << 22; for e == 0 it is 0 or 0.5.
    uint32_t e = (idx >> 1) & 3u, m = idx & 1u;
    uint32_t bits = e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3F000000u : 0u);
    return __uint_as_float(bits);
}

// Round a non-negative, exactly known fp32 value v (< 2^22) to the E2M1 index
// (0..7) with round-to-nearest-even and saturation at 6.  The grid spacing is
// 0.5 below 2, 1 in [2, 4) and 2 from 4 on; scaling v by the inverse spacing
// (a power of two, exact) and adding 1.5 * 2^23 rounds to an integer with the
// hardware's nearest-even rule; the parity of that integer is the parity of
// the E2M1 index, so the tie rule is the same.
__device__ __forceinline__ uint32_t e2m1_index_rne(float v) {
    v = fminf(v, 8.0f);
    const bool lo = v < 2.0f, mid = v < 4.0f;
    const float s = lo ? 2.0f : (mid ? 1.0f : 0.5f);
    const uint32_t off = lo ? 0u : (mid ? 2u : 4u);
    const float t = __fadd_rn(__fmul_rn(v, s), 12582912.0f);
    const uint32_t q = __float_as_uint(t) - 0x4B400000u;
    return min(off + q, 7u);
}

// E4M3FN byte (0..0x7E) of a non-negative double q: nearest value, ties to even
// mantissa, saturating at 448.  The quantum is 2^-9 below 2^-6 (subnormals) and
// 2^(e-3) in [2^e, 2^(e+1)); the byte is exponent-field * 8 + mantissa, and a
// mantissa carry flows into the exponent field, so byte = base + n - 8 works
// across binades.
__device__ __forceinline__ uint32_t e4m3_rne_sat(double q) {
    if (!(q > 0.0)) return 0u;
    if (q >= 448.0) return 0x7Eu;
    int e = ((int)((__double_as_longlong(q) >> 52) & 0x7FF)) - 1023;   // q normal in fp64
    if (e < -6) {
        double n = rint(q * 512.0);          // multiples of 2^-9, exact scaling
        return (uint32_t)n;                   // n == 8 is byte 0x08 = 2^-6
    }
    double n = rint(ldexp(q, 3 - e));       // in [8, 16]
    uint32_t b = (uint32_t)((e + 7) * 8) + (uint32_t)n - 8u;
    return min(b, 0x7Eu);
}

// Exact value of a non-negative E4M3 byte (0..0x7E) as fp32.
__device__ __forceinline__ float e4m3_value(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 0) return (float)m * 0.001953125f;               // m * 2^-9
    return __uint_as_float(((e + 120u) << 23) | (m << 20));   // (1 + m/8) 2^(e-7)
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------------ host launchers
// Each returns hipSuccess or the launch error.  Shapes are validated by the caller.
hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_mx_to_mxfp8(const uint8_t* codes, int64_t rows, int64_t k, uint8_t* codes8, hipStream_t s);
hipError_t launch_quantize_nv(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* tensor_scale,
                              bool ts_is_input, uint32_t* amax_ws, hipStream_t s);
hipError_t launch_quantize_nv_noalloc(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* codes,
                                      uint8_t* scales, float* tensor_scale, bool ts_is_input, hipStream_t s);
size_t nv_scratch_bytes();
hipError_t launch_kv_append(const uint16_t* x, int64_t tokens, int64_t d, int64_t ldx, const int32_t* slots,
                            uint8_t* codes, uint8_t* scales, int64_t capacity, hipStream_t s);
hipError_t launch_fake_quant(int fmt, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, void* out,
                             int out_f32, int64_t ld_out, float* tensor_scale, bool ts_is_input, uint32_t* amax_ws,
                             hipStream_t s);
hipError_t launch_ste_backward(const void* g, int g_f32, int64_t rows, int64_t k, int64_t ldg, float* gm, int64_t ldm,
                               int accumulate, hipStream_t s);
// Bytes of the optional workspace of launch_remap / launch_dequant_fp8 (one per
// partial-maximum workgroup, at most 256); ws == nullptr takes a third launch.
size_t scale_max_workspace_bytes(int64_t rows, int64_t k);
hipError_t launch_remap(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                        uint8_t* scales_nv, float* tensor_scale, int32_t* n_inexact, uint8_t* ws, hipStream_t s);
hipError_t launch_dequant_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, uint8_t* v8,
                              uint8_t* s8, float* tensor_scale, int32_t* n_inexact, uint8_t* ws, hipStream_t s);
hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, const float* ts,
                          int64_t rows, int64_t k, void* out, int out_f32, int64_t ld_out,
                          hipStream_t s);
hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s);
hipError_t launch_gemm_nv(const uint8_t* ac, const uint8_t* as, const float* ats,
                          const uint8_t* bc, const uint8_t* bs, const float* bts,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s);

hipError_t launch_gemm_w4a8(const uint8_t* a8, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                            int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc, hipStream_t s);

struct MoeArgs {
    int fmt;
    const uint16_t* x;
    int64_t tokens, hidden, inter;
    const int32_t* ids;
    const float* weights;
    int topk, num_experts;
    const uint8_t *w13c, *w13s, *w2c, *w2s;
    const float *w13ts, *w2ts, *act_ts;
    uint16_t* out;
    void* ws;
    size_t ws_bytes;
    fp4_moe_debug dbg;
};
int64_t moe_max_tiles(int64_t tokens, int topk, int num_experts);
size_t moe_workspace_bytes(int fmt, int64_t tokens, int64_t hidden, int topk, int num_experts,
                           int64_t inter);
hipError_t launch_moe(const MoeArgs& a, hipStream_t s);

}  // namespace fp4
