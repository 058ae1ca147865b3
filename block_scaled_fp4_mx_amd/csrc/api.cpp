// C ABI of libfp4: argument validation and dispatch to the gfx950 kernels.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing; the library holds no state besides the per-thread error message.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fp4_internal.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

int ok() {
    g_last_error[0] = '\0';
    return FP4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(FP4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

#define FP4_REQUIRE(cond, status, ...) \
    do {                               \
        if (!(cond)) return fail(status, __VA_ARGS__); \
    } while (0)

#define FP4_PTR(p) FP4_REQUIRE((p) != nullptr, FP4_ERR_INVALID, "%s is NULL", #p); \
    FP4_REQUIRE(aligned16(p), FP4_ERR_ALIGN, "%s is not 16-byte aligned", #p)

// Scalars the kernels read (tensor scales, counters) need only natural alignment.
#define FP4_SCALAR_PTR(p) FP4_REQUIRE((p) != nullptr, FP4_ERR_INVALID, "%s is NULL", #p); \
    FP4_REQUIRE((reinterpret_cast<uintptr_t>(p) & 3u) == 0, FP4_ERR_ALIGN, "%s is not 4-byte aligned", #p)

int check_ld(int64_t ld, int64_t width, const char* name) {
    FP4_REQUIRE(ld >= width, FP4_ERR_INVALID, "%s (%lld) is smaller than the row width (%lld)", name,
                (long long)ld, (long long)width);
    FP4_REQUIRE(ld % 8 == 0, FP4_ERR_ALIGN, "%s (%lld) is not a multiple of 8", name, (long long)ld);
    return FP4_OK;
}

size_t nv_ws_bytes() { return 4096; }   // pass-1 partial maxima of the tensor amax (1024 words)

// The remap's and FP8 dequant's optional workspace: NULL (with 0 bytes) or at
// least fp4_scale_max_workspace_bytes(rows, k) bytes.
int check_scale_max_ws(const void* ws, size_t bytes, int64_t rows, int64_t k) {
    if (ws == nullptr) {
        FP4_REQUIRE(bytes == 0, FP4_ERR_WORKSPACE, "workspace is NULL but workspace_bytes=%zu", bytes);
        return FP4_OK;
    }
    const size_t need = fp4::scale_max_workspace_bytes(rows, k);
    FP4_REQUIRE(bytes >= need, FP4_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, bytes);
    return FP4_OK;
}

}  // namespace

extern "C" {

int fp4_abi_version(void) { return 2; }

const char* fp4_status_string(int status) {
    switch (status) {
        case FP4_OK: return "ok";
        case FP4_ERR_INVALID: return "invalid argument";
        case FP4_ERR_SHAPE: return "unsupported shape";
        case FP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
        case FP4_ERR_UNSUPPORTED: return "unsupported combination";
        case FP4_ERR_WORKSPACE: return "workspace missing or too small";
        case FP4_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* fp4_last_error(void) { return g_last_error; }

int fp4_quantize_mx(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x,
                    uint8_t* codes, uint8_t* scales, void* stream) {
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 32 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 32", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(x_bf16);
    FP4_PTR(codes);
    FP4_PTR(scales);
    if (int e = check_ld(ld_x, k, "ld_x")) return e;
    return hip_status(fp4::launch_quantize_mx(static_cast<const uint16_t*>(x_bf16), rows, k, ld_x, codes,
                                              scales, static_cast<hipStream_t>(stream)),
                      "fp4_quantize_mx launch");
}

size_t fp4_quantize_nv_workspace_bytes(int64_t rows, int64_t k) {
    (void)rows;
    (void)k;
    return nv_ws_bytes();
}

int fp4_quantize_nv(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x, uint8_t* codes,
                    uint8_t* scales, float* tensor_scale, int tensor_scale_is_input, void* workspace,
                    size_t workspace_bytes, void* stream) {
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 16 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 16", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(x_bf16);
    FP4_PTR(codes);
    FP4_PTR(scales);
    FP4_SCALAR_PTR(tensor_scale);
    if (int e = check_ld(ld_x, k, "ld_x")) return e;
    if (!tensor_scale_is_input) {
        FP4_REQUIRE(workspace != nullptr && workspace_bytes >= nv_ws_bytes(), FP4_ERR_WORKSPACE,
                    "workspace needs %zu bytes, got %zu", nv_ws_bytes(), workspace ? workspace_bytes : (size_t)0);
        FP4_REQUIRE(aligned16(workspace), FP4_ERR_ALIGN, "workspace is not 16-byte aligned");
    }
    return hip_status(fp4::launch_quantize_nv(static_cast<const uint16_t*>(x_bf16), rows, k, ld_x, codes, scales,
                                              tensor_scale, tensor_scale_is_input != 0,
                                              static_cast<uint32_t*>(workspace), static_cast<hipStream_t>(stream)),
                      "fp4_quantize_nv launch");
}

int fp4_quantize_nv_noalloc(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x, uint8_t* codes,
                            uint8_t* scales, float* tensor_scale, int tensor_scale_is_input, void* stream) {
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 16 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 16", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(x_bf16);
    FP4_PTR(codes);
    FP4_PTR(scales);
    FP4_SCALAR_PTR(tensor_scale);
    if (int e = check_ld(ld_x, k, "ld_x")) return e;
    // The partial maxima need one word per pass-1 workgroup; the grid is capped
    // so that every shape fits the static array.
    FP4_REQUIRE(nv_ws_bytes() <= fp4::nv_scratch_bytes(), FP4_ERR_WORKSPACE,
                "the NV quantize needs %zu bytes of scratch, the static array holds %zu", nv_ws_bytes(),
                fp4::nv_scratch_bytes());
    return hip_status(fp4::launch_quantize_nv_noalloc(static_cast<const uint16_t*>(x_bf16), rows, k, ld_x, codes,
                                                      scales, tensor_scale, tensor_scale_is_input != 0,
                                                      static_cast<hipStream_t>(stream)),
                      "fp4_quantize_nv_noalloc launch");
}

size_t fp4_scale_max_workspace_bytes(int64_t rows, int64_t k) {
    return rows > 0 && k >= 32 ? fp4::scale_max_workspace_bytes(rows, k) : 0;
}

int fp4_remap_mx_to_nv(const uint8_t* codes, const uint8_t* scales_e8m0, int64_t rows, int64_t k,
                       uint8_t* scales_e4m3, float* tensor_scale, int32_t* n_inexact_blocks, void* workspace,
                       size_t workspace_bytes, void* stream) {
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 32 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 32", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(codes);
    FP4_PTR(scales_e8m0);
    FP4_PTR(scales_e4m3);
    FP4_SCALAR_PTR(tensor_scale);
    FP4_SCALAR_PTR(n_inexact_blocks);
    if (const int e = check_scale_max_ws(workspace, workspace_bytes, rows, k)) return e;
    return hip_status(fp4::launch_remap(codes, scales_e8m0, rows, k, scales_e4m3, tensor_scale, n_inexact_blocks,
                                        static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream)),
                      "fp4_remap_mx_to_nv launch");
}

int fp4_dequant(fp4_format fmt, const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                int64_t rows, int64_t k, void* out, fp4_dtype out_dtype, int64_t ld_out, void* stream) {
    FP4_REQUIRE(fmt == FP4_FMT_MX || fmt == FP4_FMT_NV, FP4_ERR_INVALID, "bad format %d", (int)fmt);
    FP4_REQUIRE(out_dtype == FP4_DT_BF16 || out_dtype == FP4_DT_F32, FP4_ERR_INVALID, "bad dtype %d", (int)out_dtype);
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    const int blk = fmt == FP4_FMT_MX ? 32 : 16;
    FP4_REQUIRE(k % blk == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of %d", (long long)k, blk);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(codes);
    FP4_PTR(scales);
    FP4_PTR(out);
    if (fmt == FP4_FMT_NV) { FP4_SCALAR_PTR(tensor_scale); }
    if (int e = check_ld(ld_out, k, "ld_out")) return e;
    return hip_status(fp4::launch_dequant(fmt, codes, scales, tensor_scale, rows, k, out, out_dtype == FP4_DT_F32,
                                          ld_out, static_cast<hipStream_t>(stream)),
                      "fp4_dequant launch");
}

int fp4_gemm(fp4_format fmt, const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale, int64_t m, int64_t n,
             int64_t k, void* c, fp4_dtype c_dtype, int64_t ldc, void* stream) {
    FP4_REQUIRE(fmt == FP4_FMT_MX || fmt == FP4_FMT_NV, FP4_ERR_INVALID, "bad format %d", (int)fmt);
    FP4_REQUIRE(c_dtype == FP4_DT_BF16 || c_dtype == FP4_DT_F32, FP4_ERR_INVALID, "bad dtype %d", (int)c_dtype);
    FP4_REQUIRE(m >= 0 && n >= 0 && k >= 0, FP4_ERR_INVALID, "negative size m=%lld n=%lld k=%lld", (long long)m,
                (long long)n, (long long)k);
    const int blk = fmt == FP4_FMT_MX ? 32 : 16;
    FP4_REQUIRE(k % blk == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of %d", (long long)k, blk);
    FP4_REQUIRE(m < (int64_t)65535 * 128, FP4_ERR_SHAPE, "m=%lld too large", (long long)m);
    if (m == 0 || n == 0) return ok();
    FP4_PTR(c);
    FP4_REQUIRE(ldc >= n, FP4_ERR_INVALID, "ldc (%lld) < n (%lld)", (long long)ldc, (long long)n);
    if (k > 0) {
        FP4_PTR(a_codes);
        FP4_PTR(a_scales);
        FP4_PTR(b_codes);
        FP4_PTR(b_scales);
    }
    if (fmt == FP4_FMT_NV) {
        FP4_SCALAR_PTR(a_tensor_scale);
        FP4_SCALAR_PTR(b_tensor_scale);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = fmt == FP4_FMT_MX
                       ? fp4::launch_gemm_mx(a_codes, a_scales, b_codes, b_scales, m, n, k, c, c_dtype == FP4_DT_F32, ldc, s)
                       : fp4::launch_gemm_nv(a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, m, n,
                                             k, c, c_dtype == FP4_DT_F32, ldc, s);
    return hip_status(e, "fp4_gemm launch");
}

int fp4_kv_append_mx(const void* x_bf16, int64_t tokens, int64_t d, int64_t ld_x, const int32_t* slots,
                     uint8_t* cache_codes, uint8_t* cache_scales, int64_t capacity, void* stream) {
    FP4_REQUIRE(tokens >= 0 && d >= 0 && capacity >= 0, FP4_ERR_INVALID, "negative size tokens=%lld d=%lld capacity=%lld",
                (long long)tokens, (long long)d, (long long)capacity);
    FP4_REQUIRE(d % 32 == 0, FP4_ERR_SHAPE, "d=%lld is not a multiple of 32", (long long)d);
    if (tokens == 0 || d == 0 || capacity == 0) return ok();
    FP4_PTR(x_bf16);
    FP4_SCALAR_PTR(slots);
    FP4_PTR(cache_codes);
    FP4_PTR(cache_scales);
    if (int e = check_ld(ld_x, d, "ld_x")) return e;
    return hip_status(fp4::launch_kv_append(static_cast<const uint16_t*>(x_bf16), tokens, d, ld_x, slots, cache_codes,
                                            cache_scales, capacity, static_cast<hipStream_t>(stream)),
                      "fp4_kv_append_mx launch");
}

int fp4_fake_quant(fp4_format fmt, const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x, void* out,
                   fp4_dtype out_dtype, int64_t ld_out, float* tensor_scale, int tensor_scale_is_input, void* workspace,
                   size_t workspace_bytes, void* stream) {
    FP4_REQUIRE(fmt == FP4_FMT_MX || fmt == FP4_FMT_NV, FP4_ERR_INVALID, "bad format %d", (int)fmt);
    FP4_REQUIRE(out_dtype == FP4_DT_BF16 || out_dtype == FP4_DT_F32, FP4_ERR_INVALID, "bad dtype %d", (int)out_dtype);
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    const int blk = fmt == FP4_FMT_MX ? 32 : 16;
    FP4_REQUIRE(k % blk == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of %d", (long long)k, blk);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(x_bf16);
    FP4_PTR(out);
    if (int e = check_ld(ld_x, k, "ld_x")) return e;
    if (int e = check_ld(ld_out, k, "ld_out")) return e;
    {
        const uintptr_t xb = reinterpret_cast<uintptr_t>(x_bf16), ob = reinterpret_cast<uintptr_t>(out);
        const uintptr_t xe = xb + (uintptr_t)(((rows - 1) * ld_x + k) * 2);
        const uintptr_t oe = ob + (uintptr_t)(((rows - 1) * ld_out + k) * (out_dtype == FP4_DT_F32 ? 4 : 2));
        const bool overlap = xb < oe && ob < xe;
        const bool in_place = xb == ob && ld_x == ld_out && out_dtype == FP4_DT_BF16;
        FP4_REQUIRE(!overlap || in_place, FP4_ERR_INVALID, "out overlaps x without being x itself");
    }
    if (fmt == FP4_FMT_NV) {
        FP4_SCALAR_PTR(tensor_scale);
        if (!tensor_scale_is_input) {
            FP4_REQUIRE(workspace != nullptr && workspace_bytes >= nv_ws_bytes(), FP4_ERR_WORKSPACE,
                        "workspace needs %zu bytes, got %zu", nv_ws_bytes(), workspace ? workspace_bytes : (size_t)0);
            FP4_REQUIRE(aligned16(workspace), FP4_ERR_ALIGN, "workspace is not 16-byte aligned");
        }
    }
    return hip_status(fp4::launch_fake_quant(fmt, static_cast<const uint16_t*>(x_bf16), rows, k, ld_x, out,
                                             out_dtype == FP4_DT_F32, ld_out, tensor_scale, tensor_scale_is_input != 0,
                                             static_cast<uint32_t*>(workspace), static_cast<hipStream_t>(stream)),
                      "fp4_fake_quant launch");
}

int fp4_ste_backward(const void* grad, fp4_dtype grad_dtype, int64_t rows, int64_t k, int64_t ld_grad,
                     float* grad_master, int64_t ld_master, int accumulate, void* stream) {
    FP4_REQUIRE(grad_dtype == FP4_DT_BF16 || grad_dtype == FP4_DT_F32, FP4_ERR_INVALID, "bad dtype %d", (int)grad_dtype);
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 8 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 8", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(grad);
    FP4_PTR(grad_master);
    if (int e = check_ld(ld_grad, k, "ld_grad")) return e;
    if (int e = check_ld(ld_master, k, "ld_master")) return e;
    return hip_status(fp4::launch_ste_backward(grad, grad_dtype == FP4_DT_F32, rows, k, ld_grad, grad_master, ld_master,
                                               accumulate, static_cast<hipStream_t>(stream)),
                      "fp4_ste_backward launch");
}

int fp4_quantize_mxfp8(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x, uint8_t* codes8, uint8_t* scales,
                       void* stream) {
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 32 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 32", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(x_bf16);
    FP4_PTR(codes8);
    FP4_PTR(scales);
    if (int e = check_ld(ld_x, k, "ld_x")) return e;
    return hip_status(fp4::launch_quantize_mxfp8(static_cast<const uint16_t*>(x_bf16), rows, k, ld_x, codes8, scales,
                                                 static_cast<hipStream_t>(stream)),
                      "fp4_quantize_mxfp8 launch");
}

int fp4_mx_dequant_fp8(const uint8_t* codes, const uint8_t* scales_e8m0, int64_t rows, int64_t k,
                       uint8_t* values_e4m3, uint8_t* block_scales_e4m3, float* tensor_scale,
                       int32_t* n_inexact_blocks, void* workspace, size_t workspace_bytes, void* stream) {
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 32 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 32", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(codes);
    FP4_PTR(scales_e8m0);
    FP4_PTR(values_e4m3);
    FP4_SCALAR_PTR(tensor_scale);
    FP4_SCALAR_PTR(n_inexact_blocks);
    if (const int e = check_scale_max_ws(workspace, workspace_bytes, rows, k)) return e;
    return hip_status(fp4::launch_dequant_fp8(codes, scales_e8m0, rows, k, values_e4m3, block_scales_e4m3,
                                              tensor_scale, n_inexact_blocks, static_cast<uint8_t*>(workspace),
                                              static_cast<hipStream_t>(stream)),
                      "fp4_mx_dequant_fp8 launch");
}

int fp4_mx_to_mxfp8(const uint8_t* codes, int64_t rows, int64_t k, uint8_t* codes8, void* stream) {
    FP4_REQUIRE(rows >= 0 && k >= 0, FP4_ERR_INVALID, "negative size rows=%lld k=%lld", (long long)rows, (long long)k);
    FP4_REQUIRE(k % 32 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 32", (long long)k);
    if (rows == 0 || k == 0) return ok();
    FP4_PTR(codes);
    FP4_PTR(codes8);
    return hip_status(fp4::launch_mx_to_mxfp8(codes, rows, k, codes8, static_cast<hipStream_t>(stream)),
                      "fp4_mx_to_mxfp8 launch");
}

int fp4_gemm_w4a8(const uint8_t* a_codes8, const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                  int64_t m, int64_t n, int64_t k, void* c, fp4_dtype c_dtype, int64_t ldc, void* stream) {
    FP4_REQUIRE(c_dtype == FP4_DT_BF16 || c_dtype == FP4_DT_F32, FP4_ERR_INVALID, "bad dtype %d", (int)c_dtype);
    FP4_REQUIRE(m >= 0 && n >= 0 && k >= 0, FP4_ERR_INVALID, "negative size m=%lld n=%lld k=%lld", (long long)m,
                (long long)n, (long long)k);
    FP4_REQUIRE(k % 32 == 0, FP4_ERR_SHAPE, "k=%lld is not a multiple of 32", (long long)k);
    FP4_REQUIRE(m < (int64_t)65535 * 128, FP4_ERR_SHAPE, "m=%lld too large", (long long)m);
    if (m == 0 || n == 0) return ok();
    FP4_PTR(c);
    FP4_REQUIRE(ldc >= n, FP4_ERR_INVALID, "ldc (%lld) < n (%lld)", (long long)ldc, (long long)n);
    if (k > 0) {
        FP4_PTR(a_codes8);
        FP4_PTR(a_scales);
        FP4_PTR(b_codes);
        FP4_PTR(b_scales);
    }
    return hip_status(fp4::launch_gemm_w4a8(a_codes8, a_scales, b_codes, b_scales, m, n, k, c, c_dtype == FP4_DT_F32,
                                            ldc, static_cast<hipStream_t>(stream)),
                      "fp4_gemm_w4a8 launch");
}

size_t fp4_moe_workspace_bytes(fp4_format fmt, int64_t tokens, int64_t hidden, int topk, int num_experts,
                               int64_t inter) {
    if (tokens < 0 || hidden <= 0 || topk < 1 || num_experts < 1 || inter <= 0) return 0;
    return fp4::moe_workspace_bytes(fmt, tokens, hidden, topk, num_experts, inter);
}

int fp4_moe_grouped_gemm(fp4_format fmt, const void* x_bf16, int64_t tokens, int64_t hidden,
                         const int32_t* topk_ids, const float* topk_weights, int topk, int num_experts,
                         int64_t inter, const uint8_t* w13_codes, const uint8_t* w13_scales,
                         const float* w13_tensor_scales, const uint8_t* w2_codes, const uint8_t* w2_scales,
                         const float* w2_tensor_scales, const float* act_tensor_scales, void* out_bf16,
                         void* workspace, size_t workspace_bytes, const fp4_moe_debug* dbg, void* stream) {
    FP4_REQUIRE(fmt == FP4_FMT_MX || fmt == FP4_FMT_NV, FP4_ERR_INVALID, "bad format %d", (int)fmt);
    FP4_REQUIRE(tokens >= 0, FP4_ERR_INVALID, "negative tokens");
    FP4_REQUIRE(topk >= 1 && topk <= 16, FP4_ERR_INVALID, "topk=%d outside [1, 16]", topk);
    FP4_REQUIRE(num_experts >= 1 && num_experts <= 1024, FP4_ERR_INVALID, "num_experts=%d outside [1, 1024]", num_experts);
    FP4_REQUIRE(hidden > 0 && inter > 0, FP4_ERR_INVALID, "hidden and inter must be positive");
    FP4_REQUIRE(hidden % 128 == 0 && inter % 128 == 0, FP4_ERR_SHAPE, "hidden=%lld and inter=%lld must be multiples of 128",
                (long long)hidden, (long long)inter);
    FP4_REQUIRE(tokens * topk < (int64_t)1 << 30 && fp4::moe_max_tiles(tokens, topk, num_experts) <= 65535,
                FP4_ERR_SHAPE, "tokens*topk=%lld too large", (long long)(tokens * topk));
    {
        // The grouped GEMM tiles address each operand with 32-bit byte offsets
        // from its base: the gathered activation rows (Q(x) by token, Q(h) by
        // routed slot; NV also their fp16 expansions) and one expert's weight
        // slab.  Each must stay below 2 GiB.
        const int64_t lim = (int64_t)1 << 31, S = tokens * topk;
        const int64_t act_x = fmt == FP4_FMT_NV ? tokens * hidden * 2 : tokens * (hidden / 2);
        const int64_t act_h = fmt == FP4_FMT_NV ? S * inter * 2 : S * (inter / 2);
        FP4_REQUIRE(act_x < lim && act_h < lim && inter * hidden < lim, FP4_ERR_SHAPE,
                    "operand too large for 32-bit tile offsets: activations %lld and %lld bytes, expert slab %lld "
                    "bytes (each must be below 2^31)",
                    (long long)act_x, (long long)act_h, (long long)(inter * hidden));
    }
    if (tokens == 0) return ok();
    FP4_PTR(x_bf16);
    FP4_SCALAR_PTR(topk_ids);
    FP4_SCALAR_PTR(topk_weights);
    FP4_PTR(w13_codes);
    FP4_PTR(w13_scales);
    FP4_PTR(w2_codes);
    FP4_PTR(w2_scales);
    FP4_PTR(out_bf16);
    if (fmt == FP4_FMT_NV) {
        FP4_SCALAR_PTR(w13_tensor_scales);
        FP4_SCALAR_PTR(w2_tensor_scales);
        FP4_SCALAR_PTR(act_tensor_scales);
    }
    const size_t need = fp4::moe_workspace_bytes(fmt, tokens, hidden, topk, num_experts, inter);
    FP4_REQUIRE(workspace != nullptr && workspace_bytes >= need, FP4_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu",
                need, workspace ? workspace_bytes : (size_t)0);
    FP4_REQUIRE(aligned16(workspace), FP4_ERR_ALIGN, "workspace is not 16-byte aligned");
    fp4::MoeArgs a{};
    a.fmt = fmt;
    a.x = static_cast<const uint16_t*>(x_bf16);
    a.tokens = tokens;
    a.hidden = hidden;
    a.inter = inter;
    a.ids = topk_ids;
    a.weights = topk_weights;
    a.topk = topk;
    a.num_experts = num_experts;
    a.w13c = w13_codes;
    a.w13s = w13_scales;
    a.w2c = w2_codes;
    a.w2s = w2_scales;
    a.w13ts = w13_tensor_scales;
    a.w2ts = w2_tensor_scales;
    a.act_ts = act_tensor_scales;
    a.out = static_cast<uint16_t*>(out_bf16);
    a.ws = workspace;
    a.ws_bytes = workspace_bytes;
    if (dbg) {
        a.dbg = *dbg;
        FP4_REQUIRE(aligned16(a.dbg.gate_up) && aligned16(a.dbg.h_bf16) && aligned16(a.dbg.h_codes) &&
                        aligned16(a.dbg.h_scales) && aligned16(a.dbg.y) && aligned16(a.dbg.gate_up_in) &&
                        aligned16(a.dbg.h_codes_in) && aligned16(a.dbg.h_scales_in),
                    FP4_ERR_ALIGN, "debug buffers must be 16-byte aligned");
        FP4_REQUIRE((a.dbg.h_codes_in == nullptr) == (a.dbg.h_scales_in == nullptr), FP4_ERR_INVALID,
                    "h_codes_in and h_scales_in must be given together");
    }
    return hip_status(fp4::launch_moe(a, static_cast<hipStream_t>(stream)), "fp4_moe_grouped_gemm launch");
}

}  // extern "C"
