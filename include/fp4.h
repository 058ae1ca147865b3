/*
 * fp4.h -- C ABI of the MI355X (gfx950) block-scaled FP4 library (libfp4.so).
 *
 * Formats.  An FP4 element is E2M1: one sign bit, two exponent bits and one
 * mantissa bit, whose non-negative values are exactly {0, 0.5, 1, 1.5, 2, 3, 4, 6}
 * ("DeepSeek-V4.1-Flash-NVFP4" explainer, section 2, NVFP4 format breakdown).
 *   MXFP4: blocks of 32 consecutive elements along K share one UE8M0 scale byte
 *          b meaning 2^(b-127) (same explainer, section 3, and the "DeepSeek-V4"
 *          architecture article, section 6.3, 1x32 tiles).
 *   NVFP4: groups of 16 consecutive elements along K share one E4M3 (OCP FP8
 *          E4M3FN) scale byte, and the whole tensor shares one fp32 scale s_t
 *          (explainer section 2: group_size 16 plus a tensor-level scale).
 *
 * Memory layout (all tensors row-major, K contiguous, no padding):
 *   codes   uint8 [rows, k/2]: byte j holds element 2j in bits 3:0 and element
 *           2j+1 in bits 7:4; a code is sign*8 + index into the value table.
 *   MX      scales uint8 [rows, k/32] (UE8M0).
 *   NV      scales uint8 [rows, k/16] (E4M3FN), plus one fp32 tensor scale in
 *           device memory.
 *   bf16 inputs/outputs are IEEE bfloat16 bit patterns with a leading dimension
 *   in elements (ld_x, ldc, ld_out >= k or n).
 *
 * Conventions shared by every entry point:
 *   - Pointers are device pointers owned by the caller; the library never
 *     allocates, frees or keeps them.  Every pointer must be 16-byte aligned and
 *     every leading dimension a multiple of 8 elements, else FP4_ERR_ALIGN.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and is asynchronous: the return value reports argument and
 *     launch errors only.  Data-dependent results (the remap's inexact count,
 *     computed tensor scales) are written to device memory.
 *   - Arguments are validated before any HIP call; a failing call enqueues
 *     nothing and returns a negative fp4_status.  fp4_last_error() gives the
 *     message of the last failure on the calling thread.
 *   - Zero-sized problems return FP4_OK and enqueue nothing.
 *   - Calls that overlap in time may not share output or workspace buffers.
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP4_OK = 0,
    FP4_ERR_INVALID = -1,      /* null pointer, bad enum, negative size        */
    FP4_ERR_SHAPE = -2,        /* k not a multiple of the block/group size ... */
    FP4_ERR_ALIGN = -3,        /* pointer not 16-B aligned, ld not multiple of 8 */
    FP4_ERR_UNSUPPORTED = -4,  /* no kernel for this combination               */
    FP4_ERR_WORKSPACE = -5,    /* workspace null or smaller than required      */
    FP4_ERR_HIP = -6           /* a HIP runtime call failed                    */
} fp4_status;

typedef enum { FP4_FMT_MX = 0, FP4_FMT_NV = 1 } fp4_format;
typedef enum { FP4_DT_BF16 = 0, FP4_DT_F32 = 1 } fp4_dtype;

/* Version of this ABI (incremented on any incompatible change). */
int fp4_abi_version(void);

/* Static text for a status code. */
const char* fp4_status_string(int status);

/* Message of the last failed call on the calling thread ("" if none). */
const char* fp4_last_error(void);

/*
 * MXFP4 quantization ("DeepSeek-V4.1-Flash-NVFP4" explainer, section 3: one
 * UE8M0 scale per 32 elements; "DeepSeek-V4" article, section 6.3).
 * For each row and each block of 32 elements along k:
 *   amax = max|x|; E = floor(log2 amax) - 2 (E = -127 when amax = 0), clamped to
 *   [-127, 127]; scales = E + 127; code = round-to-nearest-even of x * 2^-E onto
 *   the E2M1 values, saturating at 6, keeping the sign bit of x (so -0.0 gives 0x8).
 * x_bf16: [rows, ld_x] bf16; codes: [rows, k/2]; scales: [rows, k/32].
 * Errors: k % 32 != 0 -> FP4_ERR_SHAPE.  Inputs must be finite.
 */
int fp4_quantize_mx(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x,
                    uint8_t* codes, uint8_t* scales, void* stream);

/*
 * NVFP4 quantization (explainer, section 2: groups of 16 with a per-group scale
 * bringing the group into [-6, 6] and a tensor-level scale; section 4: activation
 * scales are calibrated).
 *   s_t = fp32(amax_tensor / (6 * 448)) unless tensor_scale_is_input != 0, in
 *   which case *tensor_scale (device fp32) is read as the calibrated s_t;
 *   per group: s_g = E4M3 round-to-nearest-even of amax_g / (6 s_t), saturating
 *   at 448; code = E2M1 round-to-nearest-even of x / (s_g s_t), saturating at 6.
 *   Each step is a single correct rounding of the exact real quotient.  When
 *   s_t = 0 or s_g = 0 the group's codes are signed zeros and s_g = 0.
 * codes: [rows, k/2]; scales: [rows, k/16]; tensor_scale: one device float,
 * written when computed.  workspace: device memory of at least
 * fp4_quantize_nv_workspace_bytes() bytes (used for the tensor amax).
 * Errors: k % 16 != 0 -> FP4_ERR_SHAPE; workspace too small -> FP4_ERR_WORKSPACE.
 */
int fp4_quantize_nv(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x,
                    uint8_t* codes, uint8_t* scales, float* tensor_scale,
                    int tensor_scale_is_input,
                    void* workspace, size_t workspace_bytes, void* stream);
size_t fp4_quantize_nv_workspace_bytes(int64_t rows, int64_t k);

/*
 * fp4_quantize_nv for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same operation, arguments and results as fp4_quantize_nv without the
 * workspace.  The tensor-amax partial maxima go to a static device array of
 * the library (4 KiB per GPU, held until the process ends); the call allocates
 * nothing.  Every call on a GPU shares that GPU's array, so calls that overlap
 * in time on one GPU (different streams or threads) race and must be ordered
 * by the caller.  The array's size covers every shape; FP4_ERR_WORKSPACE
 * reports a library built with a smaller one.  A HIP error in looking up the
 * array's address on the current device returns FP4_ERR_HIP.
 * Errors: as fp4_quantize_nv.
 */
int fp4_quantize_nv_noalloc(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x,
                            uint8_t* codes, uint8_t* scales, float* tensor_scale,
                            int tensor_scale_is_input, void* stream);

/*
 * Lossless MXFP4 -> NVFP4 scale remap (explainer, section 1: NVFP4's finer
 * 16-element scale layout can re-express MXFP4 weights block by block without
 * loss; section 6: the conversion script's E2M1 -> E4M3 remap).
 * Codes are reused unchanged (the NVFP4 tensor is (codes, scales_e4m3, s_t)).
 *   E_max = max over blocks of (scale byte - 127); k = E_max - 8;
 *   *tensor_scale = 2^k; both 16-groups of a block with exponent E_b get the
 *   E4M3 value nearest 2^(E_b - k) (exact for E_b - k in [-9, 8]).
 *   *n_inexact_blocks = number of blocks with a nonzero code whose 2^(E_b - k)
 *   is below 2^-9 (those lose precision); 0 means the remap is lossless.
 * codes: [rows, k/2]; scales_e8m0: [rows, k/32]; scales_e4m3: [rows, k/16];
 * tensor_scale: 1 device float; n_inexact_blocks: 1 device int32.
 * workspace: optional device memory of at least
 * fp4_scale_max_workspace_bytes(rows, k) bytes (any alignment, not overlapping
 * the other arguments) for the partial maxima of E_max; the call then takes two
 * kernel launches instead of three.  NULL (with workspace_bytes 0) keeps the
 * maxima in the output array's first bytes until a third launch rewrites them.
 * Results are the same either way.  Calls sharing one workspace must be ordered
 * (one stream).
 * Errors: k % 32 != 0 -> FP4_ERR_SHAPE; workspace too small, or NULL with
 * workspace_bytes != 0 -> FP4_ERR_WORKSPACE.
 */
int fp4_remap_mx_to_nv(const uint8_t* codes, const uint8_t* scales_e8m0,
                       int64_t rows, int64_t k, uint8_t* scales_e4m3,
                       float* tensor_scale, int32_t* n_inexact_blocks,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of the optional workspace of fp4_remap_mx_to_nv and fp4_mx_dequant_fp8
 * for an MX tensor of rows x k (at most 256; 0 for an empty tensor).
 */
size_t fp4_scale_max_workspace_bytes(int64_t rows, int64_t k);

/*
 * Dequantization (explainer, section 2: the block scales multiply back in;
 * "DeepSeek-V4 FP4 QAT" article, section 4.2: FP4 data times the scale).
 *   MX: value = (-1)^s * MAG[i] * 2^(b-127), exact in fp32 and bf16.
 *   NV: fp32 value = round-to-nearest-even(MAG[i] * s_g * s_t); bf16 output is
 *       the bf16 rounding of that fp32 value.
 * out: [rows, ld_out] of out_dtype.  tensor_scale: device float (NV only).
 * Errors: k % 32 (MX) or k % 16 (NV) != 0 -> FP4_ERR_SHAPE.
 */
int fp4_dequant(fp4_format fmt, const uint8_t* codes, const uint8_t* scales,
                const float* tensor_scale, int64_t rows, int64_t k,
                void* out, fp4_dtype out_dtype, int64_t ld_out, void* stream);

/*
 * W4A4 GEMM: C[m, n] = sum_k A_hat[m, k] * B_hat[n, k] with fp32 accumulation
 * (explainer, section 2: activations and weights both 4-bit block-scaled, the
 * accumulator rescaled per block).  A_hat, B_hat are the exact dequantized
 * operands; B is given [n, k] (the nn.Linear weight layout), so C = A . B^T.
 *   MX: scaled MFMA with the UE8M0 block scales applied by the matrix core.
 *   NV: operands expanded exactly to a 16-bit float (code * s_g has at most 6
 *       significant bits: fp16 in the tiled kernels, bf16 in the fallback) and
 *       multiplied on the 16-bit MFMA; the product is scaled by
 *       (*a_tensor_scale) * (*b_tensor_scale).
 * c: [m, ldc] of c_dtype.  Tensor scales are device floats (NV only, else NULL).
 * Errors: k % 32 (MX) or k % 16 (NV) != 0 -> FP4_ERR_SHAPE.
 */
int fp4_gemm(fp4_format fmt,
             const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale,
             int64_t m, int64_t n, int64_t k,
             void* c, fp4_dtype c_dtype, int64_t ldc, void* stream);

/*
 * MXFP4 KV-cache append ("DeepSeek-V4 FP4 QAT" article, section 3.3: the KV
 * cache is kept in MXFP4 and each new token's vector is quantized as it joins
 * the cache; the FP4 QK scores of the attention indexer are then fp4_gemm of
 * the MXFP4 queries against the cache rows, the "DeepSeek-V4" architecture
 * article, section 3, lightning indexer).  Each cache row is one token's vector
 * of d values in the MXFP4 layout above (32-element blocks along d, each with
 * its own UE8M0 byte), so a row's scales never depend on other tokens.
 *   For t in [0, tokens): if 0 <= slots[t] < capacity, row t of x is quantized
 *   exactly as fp4_quantize_mx does and written to cache row slots[t]; tokens
 *   whose slot is outside that range (padding) are skipped.  The in-range slots
 *   must be distinct.
 * x_bf16: [tokens, ld_x] bf16; slots: int32 [tokens] (device); cache_codes:
 * [capacity, d/2]; cache_scales: [capacity, d/32].
 * Errors: d % 32 != 0 -> FP4_ERR_SHAPE.  Inputs must be finite.
 */
int fp4_kv_append_mx(const void* x_bf16, int64_t tokens, int64_t d, int64_t ld_x, const int32_t* slots,
                     uint8_t* cache_codes, uint8_t* cache_scales, int64_t capacity, void* stream);

/*
 * Fake quantization for quantization-aware training ("DeepSeek-V4 FP4 QAT"
 * article, section 2.2: quantize-dequantize nodes on the expert weights in the
 * training forward pass): out = dequant(quantize(x)) in one pass over x, equal
 * element for element to fp4_quantize_mx / fp4_quantize_nv followed by
 * fp4_dequant (same rounding rules, same tensor-scale handling), with no codes
 * or scales materialized.
 *   NV: as fp4_quantize_nv, s_t is computed (and written to *tensor_scale; the
 *   workspace is then required) unless tensor_scale_is_input != 0.  MX:
 *   tensor_scale and the workspace are ignored (may be NULL).
 * x_bf16: [rows, ld_x] bf16; out: [rows, ld_out] of out_dtype.  out may be x
 * itself (in place: same pointer, ld_out == ld_x, bf16 output); any other
 * overlap of x and out is FP4_ERR_INVALID.
 * Errors: k % 32 (MX) or k % 16 (NV) != 0 -> FP4_ERR_SHAPE; NV workspace too
 * small -> FP4_ERR_WORKSPACE.  Inputs must be finite.
 */
int fp4_fake_quant(fp4_format fmt, const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x,
                   void* out, fp4_dtype out_dtype, int64_t ld_out,
                   float* tensor_scale, int tensor_scale_is_input,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Straight-through-estimator backward of the fake-quant node ("DeepSeek-V4"
 * architecture article, section 6.3: the gradient of the quantized weight is
 * handed unchanged to the fp32 master weight):
 *   grad_master[r, c] = (accumulate ? grad_master[r, c] : 0) + grad[r, c],
 * one fp32 addition (round to nearest even) per element.
 * grad: [rows, ld_grad] of grad_dtype (bf16 or fp32); grad_master: fp32
 * [rows, ld_master].  Errors: k % 8 != 0 -> FP4_ERR_SHAPE.
 */
int fp4_ste_backward(const void* grad, fp4_dtype grad_dtype, int64_t rows, int64_t k, int64_t ld_grad,
                     float* grad_master, int64_t ld_master, int accumulate, void* stream);

/*
 * W4A8: FP4 weights with FP8 activations ("DeepSeek-V4 FP4 QAT" article,
 * section 4.3: the recommended deployment pairing; section 4.2: FP4 expands into
 * FP8 without loss).  Activations use MXFP8: E4M3 elements (OCP FP8 E4M3FN,
 * largest value 448) with one UE8M0 scale per 32 elements along k, the same
 * block structure as the MXFP4 weights ("DeepSeek-V4" article, section 6.3;
 * explainer section 3).
 *
 * fp4_quantize_mxfp8: per row and 32-element block, amax = max|x|;
 *   E = floor(log2 amax) - 8 (8 = E4M3's largest exponent; E = -127 when
 *   amax = 0), clamped to [-127, 127]; scales = E + 127; code byte = E4M3
 *   round-to-nearest-even of |x| * 2^-E, saturating at 448 (0x7E), with the
 *   sign bit of x in bit 7 (so -0.0 gives 0x80).
 *   x_bf16: [rows, ld_x] bf16; codes8: [rows, k] bytes; scales: [rows, k/32].
 *   Errors: k % 32 != 0 -> FP4_ERR_SHAPE.  Inputs must be finite.
 */
int fp4_quantize_mxfp8(const void* x_bf16, int64_t rows, int64_t k, int64_t ld_x,
                       uint8_t* codes8, uint8_t* scales, void* stream);

/*
 * Lossless MXFP4 -> MXFP8 re-encoding (QAT article, section 4.2; explainer,
 * section 6: E2M1 values are E4M3 values): every E2M1 code becomes the E4M3
 * byte of the same value (sign kept, -0 -> 0x80); the UE8M0 scales are
 * unchanged, so the caller pairs codes8 with the MXFP4 tensor's own scales.
 * codes: [rows, k/2] packed E2M1; codes8: [rows, k] bytes.
 * Errors: k % 32 != 0 -> FP4_ERR_SHAPE.
 */
int fp4_mx_to_mxfp8(const uint8_t* codes, int64_t rows, int64_t k, uint8_t* codes8, void* stream);

/*
 * MXFP4 -> FP8 dequantization through E4M3 block scales ("DeepSeek-V4 FP4 QAT"
 * article, section 4.2: the scale array is re-encoded in E4M3, the 4-bit codes
 * are widened to FP8 and the FP8 scale multiplies the FP8 data; "DeepSeek-V4"
 * architecture article, section 6.3: lossless while the block scale ratio stays
 * under a threshold).  E4M3 spans only 2^-9 .. 448, so the tensor carries one
 * fp32 power of two in front:
 *   E_max = max over blocks of (scale byte - 127); k = E_max - 6;
 *   *tensor_scale = 2^k;  for block b, j = E_b - k (<= 6):
 *   block_scales_e4m3[b] = E4M3 round-to-nearest-even of 2^j (exact for j >= -9;
 *     2^-10 ties to 0);
 *   values_e4m3[r, c] = E4M3 round-to-nearest-even of MAG(code) * block scale,
 *     with the code's sign bit in bit 7 (the largest value is 6 * 2^6 = 384, so
 *     nothing saturates); the dequantized element is that value * 2^k.
 *   *n_inexact_blocks = number of blocks holding an element whose value * 2^k
 *     differs from its MX value.  It is 0 whenever every block exponent is at
 *     least E_max - 14 (a largest-to-smallest block scale ratio of at most 2^14).
 * codes: [rows, k/2]; scales_e8m0: [rows, k/32]; values_e4m3: [rows, k] bytes;
 * block_scales_e4m3: [rows, k/32] or NULL (not written); tensor_scale: 1 device
 * float; n_inexact_blocks: 1 device int32 (cleared, then accumulated, while the
 * call runs).  workspace / workspace_bytes: optional, as for fp4_remap_mx_to_nv
 * (two launches with it, three without; the same results).
 * Errors: k % 32 != 0 -> FP4_ERR_SHAPE; workspace too small, or NULL with
 * workspace_bytes != 0 -> FP4_ERR_WORKSPACE.
 */
int fp4_mx_dequant_fp8(const uint8_t* codes, const uint8_t* scales_e8m0, int64_t rows, int64_t k,
                       uint8_t* values_e4m3, uint8_t* block_scales_e4m3, float* tensor_scale,
                       int32_t* n_inexact_blocks, void* workspace, size_t workspace_bytes, void* stream);

/*
 * W4A8 GEMM: C[m, n] = sum_k A_hat[m, k] * B_hat[n, k] with fp32 accumulation,
 * A_hat the MXFP8 activations (a_codes8 [m, k] E4M3 bytes, a_scales [m, k/32])
 * and B_hat the MXFP4 weights (b_codes [n, k/2], b_scales [n, k/32]), both
 * exactly dequantized.  Mixed-format scaled MFMA (E4M3 x E2M1) with the UE8M0
 * block scales applied by the matrix core.
 * c: [m, ldc] of c_dtype.  Errors: k % 32 != 0 -> FP4_ERR_SHAPE.
 */
int fp4_gemm_w4a8(const uint8_t* a_codes8, const uint8_t* a_scales,
                  const uint8_t* b_codes, const uint8_t* b_scales,
                  int64_t m, int64_t n, int64_t k,
                  void* c, fp4_dtype c_dtype, int64_t ldc, void* stream);

/*
 * Optional intermediate outputs of fp4_moe_grouped_gemm, for staged testing.
 * Every member may be NULL.  Slot s = t * topk + j (token t, choice j).
 *   x_codes   uint8 [tokens, hidden/2], x_scales [tokens, hidden/32|16]  Q(x)
 *   counts    int32 [num_experts]    slots routed to each expert
 *   offsets   int32 [num_experts+1]  exclusive prefix sum of counts
 *   perm      int32 [tokens*topk]    slots grouped by expert, stable
 *   gate_up   fp32  [tokens*topk, 2*inter]  g (first inter) then u, per slot
 *   h_bf16    bf16  [tokens*topk, inter]    SiLU(g)*u rounded to bf16
 *   h_codes   uint8 [tokens*topk, inter/2], h_scales [tokens*topk, inter/32|16]
 *   y         fp32  [tokens*topk, hidden]   down-projection output per slot
 * Stage inputs, for testing each fused stage on given data (NULL = compute):
 *   gate_up_in   fp32 [tokens*topk, 2*inter]: g (first inter) then u per slot,
 *                already including NV tensor scales; replaces the gate/up
 *                product, and SiLU*mul, the bf16 rounding and the quantization
 *                of h run on these values.
 *   h_codes_in, h_scales_in  [tokens*topk, inter/2], [tokens*topk, inter/32|16]:
 *                quantized h per slot (NV: with s_t = act_tensor_scales[1]);
 *                replaces the computed Q(h) as the input of the down stage.
 * Stage timing: stage_events[i], when not NULL, is a hipEvent_t recorded on
 * the call's stream at stage boundary i: 0 entry, 1 after Q(x), 2 after the
 * routing metadata, 3 after gate/up (with SiLU*mul and Q(h)), 4 after down,
 * 5 after the combine.
 */
typedef struct fp4_moe_debug {
    uint8_t* x_codes;
    uint8_t* x_scales;
    int32_t* counts;
    int32_t* offsets;
    int32_t* perm;
    float* gate_up;
    void* h_bf16;
    uint8_t* h_codes;
    uint8_t* h_scales;
    float* y;
    const float* gate_up_in;
    const uint8_t* h_codes_in;
    const uint8_t* h_scales_in;
    void* stage_events[6];
} fp4_moe_debug;

/*
 * Routed-expert MoE layer on block-scaled FP4 weights and activations
 * (explainer, section 3: the routed experts' w1/w2/w3 are the quantized
 * layers; "DeepSeek-V4" article, section 2: 384 routed experts, 6 active;
 * section 6.1: dispatch to experts and combine back).  For each token t and
 * choice j with e = topk_ids[t, j]:
 *   x_hat = dequant(quant(x[t]))  (MX; or NV with s_t = act_tensor_scales[0])
 *   g = x_hat . w1[e]^T, u = x_hat . w3[e]^T   (w13[e] rows 0..inter-1 are w1,
 *                                               rows inter..2*inter-1 are w3)
 *   h = bf16(SiLU(g) * u); h_hat = dequant(quant(h)) (NV: s_t = act_tensor_scales[1])
 *   y = h_hat . w2[e]^T;  out[t] = bf16(sum_j topk_weights[t, j] * y)
 * x_bf16 [tokens, hidden]; topk_ids int32 [tokens, topk] in [0, num_experts);
 * topk_weights fp32 [tokens, topk];
 * w13_codes [E, 2*inter, hidden/2], w13_scales [E, 2*inter, hidden/32|16];
 * w2_codes [E, hidden, inter/2], w2_scales [E, hidden, inter/32|16];
 * NV: w13_tensor_scales, w2_tensor_scales fp32 [E] and act_tensor_scales fp32 [2]
 * (device); MX: all three NULL.  out_bf16 [tokens, hidden].
 * workspace: at least fp4_moe_workspace_bytes(...) bytes of device memory.
 * Errors: hidden or inter not a multiple of 128, or tokens*topk above about
 * 4.1 million -> FP4_ERR_SHAPE; topk outside [1, 16] or num_experts outside
 * [1, 1024] -> FP4_ERR_INVALID; workspace too small -> FP4_ERR_WORKSPACE.
 * A slot whose expert id lies outside [0, num_experts) is routed nowhere and
 * contributes nothing to out.  The combine sums each token's weighted rows in
 * fp32 in order j = 0 .. topk-1 without atomics, so out is deterministic.
 */
int fp4_moe_grouped_gemm(fp4_format fmt, const void* x_bf16, int64_t tokens, int64_t hidden,
                         const int32_t* topk_ids, const float* topk_weights, int topk,
                         int num_experts, int64_t inter,
                         const uint8_t* w13_codes, const uint8_t* w13_scales,
                         const float* w13_tensor_scales,
                         const uint8_t* w2_codes, const uint8_t* w2_scales,
                         const float* w2_tensor_scales,
                         const float* act_tensor_scales,
                         void* out_bf16, void* workspace, size_t workspace_bytes,
                         const fp4_moe_debug* dbg, void* stream);
size_t fp4_moe_workspace_bytes(fp4_format fmt, int64_t tokens, int64_t hidden, int topk,
                               int num_experts, int64_t inter);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */
