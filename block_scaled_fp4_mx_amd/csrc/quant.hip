// Block-scaled FP4 (and MXFP8 activation) quantize / dequantize / MX->NV remap
// kernels for gfx950.
//
// All four are HBM-streaming kernels: one lane owns 8 consecutive elements
// (one 16-byte bf16 load, one 4-byte code store), so a wavefront reads 1 KiB of
// contiguous input per instruction.  An MX block (32 elements) spans 4 adjacent
// lanes and an NV group (16 elements) 2 lanes; the block/group amax is
// combined across those lanes with DPP quad permutes (no LDS traffic).
#include <mutex>

#include "quant_device.h"

namespace fp4 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;      // 16-byte loads in flight per lane (tensor amax pass)
constexpr int kMxUnroll = 2;    // MX quantize: 16-byte loads per lane per iteration
constexpr unsigned kMxMaxBlocks = 2048;

inline unsigned grid_for(int64_t units, int per_thread = 1) {
    int64_t b = (units + (int64_t)kThreads * per_thread - 1) / ((int64_t)kThreads * per_thread);
    if (b > (1 << 20)) b = 1 << 20;
    return (unsigned)(b < 1 ? 1 : b);
}

template <bool kContig>
__device__ __forceinline__ int64_t x_offset(int64_t u, int64_t upr, int64_t ldx) {
    if (kContig) return u * 8;
    const int64_t r = u / upr;
    return r * ldx + (u - r * upr) * 8;
}

// Output of the fused quantize -> dequantize (fake-quant) mode of the quantize
// kernels: kOutCodes writes codes and scales; kOutBf16 / kOutF32 write the
// dequantized values instead (row pitch ld_out elements).
constexpr int kOutCodes = 0, kOutBf16 = 1, kOutF32 = 2;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kOutSlots = 3;   // codes and scales of row r go to row slots[r] (skipped if outside [0, capacity))

// Element offset of unit u (n consecutive elements; upr units per row).
template <bool kContig>
__device__ __forceinline__ int64_t unit_offset(int64_t u, int64_t upr, int64_t n, int64_t ld) {
    if (kContig) return u * n;
    const int64_t r = u / upr;
    return r * ld + (u - r * upr) * n;
}

// Stores n (8 or 16) fp32 values as bf16 (RNE) or fp32.
template <int kOut, int n>
__device__ __forceinline__ void store_values(void* out, int64_t o, const float* f) {
    if (kOut == kOutF32) {
        f32x4_t* p = reinterpret_cast<f32x4_t*>(static_cast<float*>(out) + o);
#pragma unroll
        for (int i = 0; i < n / 4; ++i)
            __builtin_nontemporal_store(f32x4_t{f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]}, p + i);
    } else {
        u32x4_t* p = reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(out) + o);
#pragma unroll
        for (int i = 0; i < n / 8; ++i) {
            const u32x4_t q = {f32_to_bf16_rne(f[8 * i + 0]) | (f32_to_bf16_rne(f[8 * i + 1]) << 16),
                               f32_to_bf16_rne(f[8 * i + 2]) | (f32_to_bf16_rne(f[8 * i + 3]) << 16),
                               f32_to_bf16_rne(f[8 * i + 4]) | (f32_to_bf16_rne(f[8 * i + 5]) << 16),
                               f32_to_bf16_rne(f[8 * i + 6]) | (f32_to_bf16_rne(f[8 * i + 7]) << 16)};
            __builtin_nontemporal_store(q, p + i);
        }
    }
}

// Dequantized values of 8 packed codes with scale sc (and, for NV, tensor scale
// st): MAG * sc is exact (at most 6 significant bits); NV rounds once more by
// the multiply with st, as the dequantizer does.
template <bool kNV>
__device__ __forceinline__ void dequant8(uint32_t c, float sc, float st, float* f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t code = (c >> (4 * i)) & 0xFu;
        float val = __fmul_rn(e2m1_mag(code & 7u), sc);
        if (kNV) val = __fmul_rn(val, st);
        f[i] = (code & 8u) ? -val : val;
    }
}

// 2^(b - 127) for a UE8M0 byte; b == 0 is the fp32 subnormal 2^-127.
__device__ __forceinline__ float ue8m0_value(uint32_t b) {
    return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// ------------------------------------------------------------------ MX quantize
// Lane u owns elements 8u..8u+7 of the row-major [rows, k] input (codes word u,
// scale byte u/4).  Each lane issues kMxUnroll loads before converting.  With
// kOut != kOutCodes the lane writes its 8 dequantized values to out instead
// (fake-quant); kContig then also means ld_out == k.  x and out may be the same
// buffer: every lane reads its elements before it writes them.
template <bool kContig, int kOut = kOutCodes>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, void* out = nullptr, int64_t ld_out = 0,
    const int32_t* __restrict__ slots = nullptr, int64_t capacity = 0) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t step = (int64_t)gridDim.x * kThreads * kMxUnroll;
    const bool small = total <= 0xFFFFFFFFll;        // row of a unit by 32-bit division
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kMxUnroll + threadIdx.x; base < total; base += step) {
        uint4 v[kMxUnroll];
        int64_t row[kMxUnroll];
        int32_t slotv[kMxUnroll];                     // slot mode: loaded with x, used by the stores
#pragma unroll
        for (int j = 0; j < kMxUnroll; ++j) {
            const int64_t u = base + (int64_t)j * kThreads;
            if (u < total) {
                v[j] = *reinterpret_cast<const uint4*>(x + x_offset<kContig>(u, upr, ldx));
                if (kOut == kOutSlots) {
                    row[j] = small ? (int64_t)((uint32_t)u / (uint32_t)upr) : u / upr;
                    slotv[j] = slots[row[j]];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kMxUnroll; ++j) {
            const int64_t u = base + (int64_t)j * kThreads;
            if (u < total) {
                const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
                uint32_t sbyte;
                const uint32_t packed = mx_quant8(w, sbyte);
                if (kOut == kOutCodes) {
                    reinterpret_cast<uint32_t*>(codes)[u] = packed;
                    if ((threadIdx.x & 3) == 0) scales[u >> 2] = (uint8_t)sbyte;
                } else if (kOut == kOutSlots) {
                    const int64_t r = row[j];
                    const int64_t slot = slotv[j];
                    if (slot >= 0 && slot < capacity) {
                        const int64_t v = slot * upr + (u - r * upr);
                        reinterpret_cast<uint32_t*>(codes)[v] = packed;
                        if ((threadIdx.x & 3) == 0) scales[v >> 2] = (uint8_t)sbyte;
                    }
                } else {
                    float f[8];
                    dequant8<false>(packed, ue8m0_value(sbyte), 1.0f, f);
                    store_values<kOut, 8>(out, unit_offset<kContig>(u, upr, 8, ld_out), f);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ MXFP8 quantize
// Same lane mapping as the MX quantizer: lane u owns elements 8u..8u+7 (codes
// bytes 8u..8u+7, one 8-byte store) and a quad of lanes one 32-element block.
template <bool kContig>
__global__ __launch_bounds__(kThreads) void mxfp8_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t step = (int64_t)gridDim.x * kThreads * kMxUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kMxUnroll + threadIdx.x; base < total; base += step) {
        uint4 v[kMxUnroll];
#pragma unroll
        for (int j = 0; j < kMxUnroll; ++j) {
            const int64_t u = base + (int64_t)j * kThreads;
            if (u < total) v[j] = *reinterpret_cast<const uint4*>(x + x_offset<kContig>(u, upr, ldx));
        }
#pragma unroll
        for (int j = 0; j < kMxUnroll; ++j) {
            const int64_t u = base + (int64_t)j * kThreads;
            if (u < total) {
                const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
                uint32_t sbyte;
                reinterpret_cast<uint2*>(codes)[u] = mxfp8_quant8(w, sbyte);
                if ((threadIdx.x & 3) == 0) scales[u >> 2] = (uint8_t)sbyte;
            }
        }
    }
}

// ------------------------------------------------------------------ MXFP4 -> MXFP8
// Lane u re-encodes code word u (8 E2M1 codes) into 8 E4M3 bytes; the UE8M0
// scales carry over unchanged, so the caller keeps using the same scale tensor.
__global__ __launch_bounds__(kThreads) void mx_to_mxfp8_kernel(const uint32_t* __restrict__ codes, int64_t words,
                                                              uint2* __restrict__ out) {
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < words; u += (int64_t)gridDim.x * kThreads) {
        const uint32_t w = codes[u];
        uint32_t o[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i >> 2] |= e2m1_to_e4m3((w >> (4 * i)) & 15u) << (8 * (i & 3));
        out[u] = make_uint2(o[0], o[1]);
    }
}

// ------------------------------------------------------------------ NV quantize
// Two passes when s_t is computed: (1) per-workgroup maxima of |x| into the
// workspace; (2) every quantize workgroup reduces those partials itself (the
// first reads of x already in flight), derives s_t, and workgroup 0 stores it.
// The second read of x mostly hits the last-level cache for tensors that fit.
constexpr int kNvAmaxBlocks = 1024;   // partial maxima written by pass 1
constexpr int kNvDepth = 1;           // 16-groups per lane whose loads are in flight (32 B each)
constexpr unsigned kNvMaxBlocks = 1024;
static_assert(kNvAmaxBlocks % kThreads == 0, "pass 2 loads kNvAmaxBlocks / kThreads partial maxima per lane");

template <bool kContig>
__global__ __launch_bounds__(kThreads) void nv_amax_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx, uint32_t* __restrict__ part) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
    uint32_t am = 0;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < total; base += step) {
        uint4 v[kUnroll];
#pragma unroll
        for (int j = 0; j < kUnroll; ++j) {
            const int64_t u = base + (int64_t)j * kThreads;
            v[j] = u < total ? *reinterpret_cast<const uint4*>(x + x_offset<kContig>(u, upr, ldx)) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < kUnroll; ++j)
            am = max(am, max(max(mag_max2(v[j].x), mag_max2(v[j].y)), max(mag_max2(v[j].z), mag_max2(v[j].w))));
    }
    for (int off = 32; off > 0; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = red[0];
        for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
        part[blockIdx.x] = m;
    }
}

template <bool kContig>
__device__ __forceinline__ void nv_load16(const uint16_t* __restrict__ x, int64_t u, int64_t gpr, int64_t ldx,
                                          uint4& a, uint4& b) {
    int64_t o;
    if (kContig) {
        o = u * 16;
    } else {
        const int64_t r = u / gpr;
        o = r * ldx + (u - r * gpr) * 16;
    }
    const uint4* p = reinterpret_cast<const uint4*>(x + o);
    a = p[0];
    b = p[1];
}

// Lane u owns 16-groups u, u + stride, ... (elements 16u .. 16u + 15 of their
// rows): 8 code bytes and one scale byte each.  The loads of the next two
// groups are in flight while one is converted.  npart > 0: s_t comes from the
// pass-1 partial maxima (and is stored by workgroup 0); npart == 0: s_t is read
// from *ts.  With kOut != kOutCodes the lane writes its 16 dequantized values
// (fp32 RNE(MAG * s_g * s_t), or that rounded to bf16) instead of codes and
// scales; kContig then also means ld_out == k.  x and out may be the same
// buffer: a group's loads are issued before its values are stored, and the
// groups in flight are the lane's own.
template <bool kContig, int kOut = kOutCodes>
__global__ __launch_bounds__(kThreads) void nv_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ ts, const uint32_t* __restrict__ part, int npart,
    void* out = nullptr, int64_t ld_out = 0) {
    __shared__ NvRecip rtab[128];
    __shared__ uint32_t red[kThreads / 64];
    __shared__ float st_sh;
    const int64_t gpr = k >> 4;
    const int64_t total = rows * gpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    uint4 va[kNvDepth], vb[kNvDepth];
#pragma unroll
    for (int j = 0; j < kNvDepth; ++j) {
        const int64_t uj = u + j * stride;
        if (uj < total) nv_load16<kContig>(x, uj, gpr, ldx, va[j], vb[j]);
    }
    if (npart > 0) {
        // a lane's partial maxima (npart <= kNvAmaxBlocks) are loaded together
        uint32_t pv[kNvAmaxBlocks / kThreads];
#pragma unroll
        for (int j = 0; j < kNvAmaxBlocks / kThreads; ++j) {
            const int i = threadIdx.x + j * kThreads;
            pv[j] = i < npart ? part[i] : 0u;
        }
        uint32_t am = pv[0];
#pragma unroll
        for (int j = 1; j < kNvAmaxBlocks / kThreads; ++j) am = max(am, pv[j]);
        for (int off = 32; off > 0; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
        if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t m = red[0];
            for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
            // s_t = fp32(amax / 2688): the fp64 quotient is correctly rounded, and
            // rounding it again to fp32 is exact (an 8-bit numerator over 21 * 2^7
            // is a short dyadic or far from every fp32 rounding midpoint)
            const float st = (float)((double)__uint_as_float(m << 16) / 2688.0);
            st_sh = st;
            if (blockIdx.x == 0) *ts = st;
        }
    } else if (threadIdx.x == 0) {
        st_sh = *ts;
    }
    __syncthreads();
    const double st = (double)st_sh;
    const bool live = st > 0.0;
    const double inv_st = live ? 1.0 / st : 0.0;
    if (threadIdx.x < 128) {
        const uint32_t g = threadIdx.x;
        rtab[g] = (live && g > 0 && g < 127) ? nv_recip_entry(g, inv_st) : NvRecip{0.f, 0.f};
    }
    __syncthreads();
    const double inv6st = live ? 1.0 / (6.0 * st) : 0.0;
    const bool fast = inv6st >= 0x1p-126 && inv6st < 0x1p127;
    const float inv6st32 = fast ? (float)inv6st : 0.0f;
    for (; u < total; u += kNvDepth * stride) {
#pragma unroll
        for (int j = 0; j < kNvDepth; ++j) {
            const int64_t uj = u + j * stride;
            if (uj < total) {
                const uint32_t w[8] = {va[j].x, va[j].y, va[j].z, va[j].w, vb[j].x, vb[j].y, vb[j].z, vb[j].w};
                const int64_t un = uj + kNvDepth * stride;      // refill this slot
                if (un < total) nv_load16<kContig>(x, un, gpr, ldx, va[j], vb[j]);
                const uint32_t sg = nv_group_scale(amax16_bits(w), inv6st32, inv6st, fast);
                const uint2 c = nv_codes16(w, sg, st, rtab[sg]);
                if (kOut == kOutCodes) {
                    *reinterpret_cast<uint2*>(codes + uj * 8) = c;
                    scales[uj] = (uint8_t)sg;
                } else {
                    float f[16];
                    const float sc = e4m3_value(sg), st32 = st_sh;
                    dequant8<true>(c.x, sc, st32, f);
                    dequant8<true>(c.y, sc, st32, f + 8);
                    store_values<kOut, 16>(out, unit_offset<kContig>(uj, gpr, 16, ld_out), f);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ dequant
// Lane unit u = elements 8u .. 8u + 7 of the row-major input (one code word,
// one 16-byte bf16 store, so a store instruction writes 1 KiB contiguously).
// The grid is capped and every lane keeps kDqUnroll units' loads in flight
// before converting, so the small code and scale loads overlap their latency.
constexpr int kDqUnroll = 4;
constexpr unsigned kDqMaxBlocks = 2048;
template <bool kNV, bool kF32, bool kContig>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ ts, int64_t rows, int64_t k, void* __restrict__ out, int64_t ld) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t step = (int64_t)gridDim.x * kThreads * kDqUnroll;
    const float st = kNV ? *ts : 1.0f;
    for (int64_t base = (int64_t)blockIdx.x * kThreads * kDqUnroll + threadIdx.x; base < total; base += step) {
        uint32_t c[kDqUnroll], sb[kDqUnroll];
#pragma unroll
        for (int j = 0; j < kDqUnroll; ++j) {
            const int64_t u = base + (int64_t)j * kThreads;
            if (u < total) {
                c[j] = reinterpret_cast<const uint32_t*>(codes)[u];
                sb[j] = scales[kNV ? (u >> 1) : (u >> 2)];
            }
        }
#pragma unroll
        for (int j = 0; j < kDqUnroll; ++j) {
            const int64_t u = base + (int64_t)j * kThreads;
            if (u < total) {
                const float sc = kNV ? e4m3_value(sb[j]) : ue8m0_value(sb[j]);
                float f[8];
                dequant8<kNV>(c[j], sc, st, f);
                store_values<kF32 ? kOutF32 : kOutBf16, 8>(out, unit_offset<kContig>(u, upr, 8, ld), f);
            }
        }
    }
}

// ------------------------------------------------------------------ STE backward
// Straight-through gradient of the fake-quant node into fp32 master-weight
// gradients: g_master = (accumulate ? g_master : 0) + g, one fp32 add (RNE) per
// element.  Lane u owns 8 consecutive elements of a row.
template <bool kGradF32>
__global__ __launch_bounds__(kThreads) void ste_backward_kernel(const void* __restrict__ g, int64_t rows, int64_t k,
                                                               int64_t ldg, float* __restrict__ gm, int64_t ldm,
                                                               int accumulate) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += (int64_t)gridDim.x * kThreads) {
        const int64_t r = u / upr, c = (u - r * upr) * 8;
        float gv[8];
        if (kGradF32) {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(g) + r * ldg + c);
            const float4 a = p[0], b = p[1];
            gv[0] = a.x; gv[1] = a.y; gv[2] = a.z; gv[3] = a.w; gv[4] = b.x; gv[5] = b.y; gv[6] = b.z; gv[7] = b.w;
        } else {
            const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(g) + r * ldg + c);
            const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gv[2 * i] = bf16_lo(w[i]);
                gv[2 * i + 1] = bf16_hi(w[i]);
            }
        }
        float4* m = reinterpret_cast<float4*>(gm + r * ldm + c);
        float4 m0 = make_float4(0.f, 0.f, 0.f, 0.f), m1 = m0;
        if (accumulate) {
            m0 = m[0];
            m1 = m[1];
        }
        m[0] = make_float4(__fadd_rn(m0.x, gv[0]), __fadd_rn(m0.y, gv[1]), __fadd_rn(m0.z, gv[2]), __fadd_rn(m0.w, gv[3]));
        m[1] = make_float4(__fadd_rn(m1.x, gv[4]), __fadd_rn(m1.y, gv[5]), __fadd_rn(m1.z, gv[6]), __fadd_rn(m1.w, gv[7]));
    }
}

// ------------------------------------------------------------------ tensor-wide scale passes
// The MX -> NV remap and the MX -> FP8 dequantization both need E_max, the
// largest block exponent of the whole tensor, before any output is final.
// With a caller workspace of one byte per pass-1 workgroup, two launches:
//   pass 1 (scale_max_kernel, many workgroups): workgroup g writes the largest
//     scale byte of its share to workspace byte g and workgroup 0 clears the
//     inexact counter;
//   pass 2 (many workgroups): each workgroup reduces the pass-1 bytes to E_max
//     and converts its blocks; inexact blocks are added to the counter (one
//     atomic per workgroup that found any); workgroup 0 writes the tensor scale.
// Without workspace, three: pass 1 writes its bytes to the start of the output
// array instead, pass 2 skips the first `reserved` blocks, whose output bytes
// hold them, and pass 3 (one workgroup) converts those blocks last and writes
// the tensor scale.
// (A grid-wide "last workgroup finishes" ticket in pass 2 would save a launch,
// but thousands of same-address atomics serialize: measured 44 us for 4096^2.)
constexpr int kScaleMaxChunk = 4096;   // scale bytes per pass-1 workgroup
constexpr int kScaleMaxGroups = 256;   // at most one byte per pass-2 thread

__global__ __launch_bounds__(kThreads) void scale_max_kernel(const uint8_t* __restrict__ s, int64_t nb,
                                                             uint8_t* __restrict__ part, int32_t* __restrict__ cnt) {
    const int64_t lo = (int64_t)blockIdx.x * nb / gridDim.x, hi = (int64_t)(blockIdx.x + 1) * nb / gridDim.x;
    uint32_t m = 0;
    // bytes before the first 16-byte boundary, the 16-byte body, then the tail
    const int64_t a0 = min((lo + 15) & ~(int64_t)15, hi), a1 = max(a0, hi & ~(int64_t)15);
    for (int64_t i = lo + threadIdx.x; i < a0; i += kThreads) m = max(m, (uint32_t)s[i]);
    for (int64_t i = a1 + threadIdx.x; i < hi; i += kThreads) m = max(m, (uint32_t)s[i]);
    const uint4* s16 = reinterpret_cast<const uint4*>(s + a0);
    for (int64_t q = threadIdx.x; q < (a1 - a0) >> 4; q += kThreads) {
        const uint4 v = s16[q];
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int t = 0; t < 4; ++t)
            m = max(m, max(max(w[t] & 0xFFu, (w[t] >> 8) & 0xFFu), max((w[t] >> 16) & 0xFFu, w[t] >> 24)));
    }
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
        part[blockIdx.x] = (uint8_t)m;
        if (blockIdx.x == 0) *cnt = 0;
    }
}

inline unsigned scale_max_groups(int64_t nb) {
    int64_t g = (nb + kScaleMaxChunk - 1) / kScaleMaxChunk;
    return (unsigned)(g < 1 ? 1 : (g > kScaleMaxGroups ? kScaleMaxGroups : g));
}

// E_max + 127 from the pass-1 bytes (every thread gets it).
__device__ __forceinline__ uint32_t reduce_part(const uint8_t* part, int npart, uint32_t* red) {
    uint32_t m = threadIdx.x < (unsigned)npart ? (uint32_t)part[threadIdx.x] : 0u;
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red[0];
    for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
    return m;
}

// Adds the workgroup's inexact blocks to the counter (one atomic, if any).
__device__ __forceinline__ void add_count(uint32_t mine, int32_t* cnt, uint32_t* sh) {
    for (int off = 32; off > 0; off >>= 1) mine += (uint32_t)__shfl_xor((int)mine, off);
    __syncthreads();                       // the reduce_part slots are free again
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = mine;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int i = 0; i < kThreads / 64; ++i) t += sh[i];
        if (t) atomicAdd(cnt, (int32_t)t);
    }
}

// ------------------------------------------------------------------ MX -> NV remap
// s_t = 2^(E_max - 8); both E4M3 group scales of block b are 2^(E_b - k),
// exact for j = E_b - k in [-9, 8]; a block with a nonzero code below that
// range is inexact (2^-10 ties to 0).  A lane takes four consecutive blocks:
// one 4-byte scale load, one 8-byte store.
__device__ __forceinline__ uint32_t remap_scale(uint32_t sbyte, int kexp, bool& low) {
    const int j = (int)sbyte - 127 - kexp;                // <= 8
    low = j < -9;
    if (j >= -6) return (uint32_t)(j + 7) << 3;           // normal 2^j
    if (j >= -9) return 1u << (j + 9);                    // subnormal 2^j = 2^(j+9) * 2^-9
    return 0u;                                            // 2^-10 ties to 0, below rounds to 0
}

__device__ __forceinline__ uint32_t remap_nonzero(const uint8_t* __restrict__ codes, int64_t b) {
    const uint4 a = reinterpret_cast<const uint4*>(codes + b * 16)[0];
    return ((a.x | a.y | a.z | a.w) & 0x77777777u) ? 1u : 0u;
}

// Blocks [b0, b1) (b0 a multiple of 4), E_max from the npart bytes at `part`;
// workgroup 0 writes the tensor scale when ts is not null.  The lane's first
// scale word is loaded before the reduction of the partial maxima.
__global__ __launch_bounds__(kThreads) void remap_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ s, uint8_t* snv,
                                                         const uint8_t* part, int npart, int64_t b0, int64_t b1,
                                                         float* __restrict__ ts, int32_t* __restrict__ n_inexact) {
    __shared__ uint32_t red[kThreads / 64];
    const int64_t nq = (b1 - b0 + 3) >> 2;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    auto load = [&](int64_t qq) -> uint32_t {
        const int64_t i = b0 + 4 * qq;
        if (i + 4 <= b1) return *reinterpret_cast<const uint32_t*>(s + i);
        uint32_t w = 0;
        for (int t = 0; t < 4 && i + t < b1; ++t) w |= (uint32_t)s[i + t] << (8 * t);
        return w;
    };
    uint32_t w = q < nq ? load(q) : 0u;
    const int kexp = (int)reduce_part(part, npart, red) - 127 - 8;
    __syncthreads();                       // every thread has read the pass-1 bytes before any is rewritten
    uint32_t bad = 0;
    while (q < nq) {
        const int64_t i = b0 + 4 * q;
        uint32_t o[4];
        bool low[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            o[t] = remap_scale((w >> (8 * t)) & 0xFFu, kexp, low[t]);
            o[t] |= o[t] << 8;
        }
        if (i + 4 <= b1) {
            *reinterpret_cast<uint2*>(snv + 2 * i) = make_uint2(o[0] | o[1] << 16, o[2] | o[3] << 16);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (low[t]) bad += remap_nonzero(codes, i + t);
        } else {
            for (int t = 0; t < 4 && i + t < b1; ++t) {
                reinterpret_cast<uint16_t*>(snv)[i + t] = (uint16_t)o[t];
                if (low[t]) bad += remap_nonzero(codes, i + t);
            }
        }
        q += stride;
        if (q < nq) w = load(q);
    }
    add_count(bad, n_inexact, red);
    if (ts != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *ts = ldexpf(1.0f, kexp);          // 2^-135 .. 2^119; below 2^-126 a subnormal
}

// ------------------------------------------------------------------ MX -> FP8 dequant
// s_t = 2^k with k = E_max - 6.  For block exponent j = E_b - k (<= 6) the E4M3
// block scale is s8 = RNE(2^j) (exact for j >= -9, 2^-10 ties to 0) and each
// element becomes RNE_E4M3(MAG * s8) with the code's sign.  MAG = (1 + h/2) 2^p
// for magnitude index i >= 1 (p = -1, 0, 0, 1, 1, 2, 2; h = i + 1 & 1 beyond
// i = 1), so with s8 = 2^j the value is (1 + h/2) 2^e, e = p + j >= -10:
//   e >= -6       normal byte (e + 7) << 3 | h << 2 (exact; e <= 8 gives 384),
//   e = -7, -8    subnormal (2 + h) << (e + 8) (exact),
//   e = -9        (2 + h) / 2: h = 0 gives 1; h = 1 ties 1.5 to 2 (inexact),
//   e = -10       (2 + h) / 4: 0.5 ties to 0, 0.75 rounds to 1 (both inexact).
// The block's 8 value bytes go into two words, so v_perm_b32 maps four codes'
// magnitude indices to their bytes at once.  `bad` has bit i set when
// magnitude i is inexact in this block.
__device__ __forceinline__ void fp8_block_table(int j, uint32_t& tlo, uint32_t& thi, uint32_t& bad, uint32_t& s8) {
    tlo = thi = 0u;
    bad = 0u;
    if (j < -9) {                               // the scale itself rounds to zero
        s8 = 0u;
        bad = 0xFEu;
        return;
    }
    s8 = j >= -6 ? (uint32_t)(j + 7) << 3 : 1u << (j + 9);
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        const int p = i == 1 ? -1 : (i >> 1) - 1;
        const uint32_t h = i == 1 ? 0u : (uint32_t)(i & 1);
        const int e = p + j;
        uint32_t b;
        if (e >= -6) {
            b = ((uint32_t)(e + 7) << 3) | (h << 2);
        } else if (e >= -8) {
            b = (2u + h) << (e + 8);
        } else if (e == -9) {
            b = h ? 2u : 1u;
            bad |= h << i;
        } else {
            b = h;
            bad |= 1u << i;
        }
        if (i < 4) tlo |= b << (8 * i);
        else thi |= b << (8 * (i - 4));
    }
}

// Eight codes (one word) -> eight E4M3 bytes (two words); `hit` collects the
// magnitude indices present.
__device__ __forceinline__ uint2 fp8_expand8(uint32_t c, uint32_t tlo, uint32_t thi, uint32_t& hit) {
    const uint32_t mag = c & 0x77777777u;
    const uint32_t sgn = c & 0x88888888u;
    // magnitude nibbles 0..3 and 4..7 spread into bytes (perm selectors)
    const uint32_t sel0 = (mag & 0x7u) | ((mag >> 4) & 0x7u) << 8 | ((mag >> 8) & 0x7u) << 16 | ((mag >> 12) & 0x7u) << 24;
    const uint32_t sel1 = ((mag >> 16) & 0x7u) | ((mag >> 20) & 0x7u) << 8 | ((mag >> 24) & 0x7u) << 16 | (mag >> 28) << 24;
    uint2 r;
    r.x = __builtin_amdgcn_perm(thi, tlo, sel0);
    r.y = __builtin_amdgcn_perm(thi, tlo, sel1);
    // sign bit 3 of nibble q goes to bit 7 of byte q
    r.x |= ((sgn & 0x8u) << 4) | ((sgn & 0x80u) << 8) | ((sgn & 0x800u) << 12) | ((sgn & 0x8000u) << 16);
    r.y |= ((sgn >> 16) & 0x8u) << 4 | ((sgn >> 16) & 0x80u) << 8 | ((sgn >> 16) & 0x800u) << 12 |
           ((sgn >> 16) & 0x8000u) << 16;
#pragma unroll
    for (int q = 0; q < 8; ++q) hit |= 1u << ((mag >> (4 * q)) & 7u);
    return r;
}

// One block per lane: 16 code bytes in, 32 E4M3 bytes out.  Blocks within 11
// binades of the largest (j >= -5) have every value normal and exact: the table
// is the E4M3 bytes of the E2M1 magnitudes at j = 0 (0x30, 0x38, 0x3C, 0x40,
// 0x44, 0x48, 0x4C) with j added to each nonzero byte's exponent field (no
// byte drops below 8, so no borrow crosses bytes).  Other blocks take the
// general table.  Returns 1 for an inexact block.
__device__ __forceinline__ uint32_t fp8_block(uint4 c, uint32_t sbyte, uint8_t* v8,
                                              uint8_t* __restrict__ s8out, int64_t b, int kexp) {
    const int j = (int)sbyte - 127 - kexp;
    uint32_t tlo, thi, badm, s8;
    if (j >= -5) {
        tlo = 0x3C383000u + (uint32_t)(j * 0x08080800);
        thi = 0x4C484440u + (uint32_t)(j * 0x08080808);
        badm = 0u;
        s8 = (uint32_t)(j + 7) << 3;
    } else {
        fp8_block_table(j, tlo, thi, badm, s8);
    }
    uint32_t hit = 0;
    const uint2 o0 = fp8_expand8(c.x, tlo, thi, hit);
    const uint2 o1 = fp8_expand8(c.y, tlo, thi, hit);
    const uint2 o2 = fp8_expand8(c.z, tlo, thi, hit);
    const uint2 o3 = fp8_expand8(c.w, tlo, thi, hit);
    uint4* o = reinterpret_cast<uint4*>(v8 + b * 32);
    __builtin_nontemporal_store(u32x4_t{o0.x, o0.y, o1.x, o1.y}, reinterpret_cast<u32x4_t*>(o));
    __builtin_nontemporal_store(u32x4_t{o2.x, o2.y, o3.x, o3.y}, reinterpret_cast<u32x4_t*>(o) + 1);
    if (s8out != nullptr) s8out[b] = (uint8_t)s8;
    return (hit & badm) ? 1u : 0u;
}

constexpr int kFp8Depth = 4;

// Blocks [b0, b1), E_max from the npart bytes at `part`; workgroup 0 writes
// the tensor scale when ts is not null.
__global__ __launch_bounds__(kThreads) void fp8_dequant_kernel(const uint8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ s, uint8_t* v8,
                                                               uint8_t* __restrict__ s8out, const uint8_t* part,
                                                               int npart, int64_t b0, int64_t b1,
                                                               float* __restrict__ ts,
                                                               int32_t* __restrict__ n_inexact) {
    __shared__ uint32_t red[kThreads / 64];
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    // kFp8Depth blocks per lane: every load is issued before the first
    // conversion, the first group's before the reduction of the partial maxima
    uint4 c[kFp8Depth];
    uint32_t sb[kFp8Depth];
    auto load = [&](int64_t bb) {
#pragma unroll
        for (int d = 0; d < kFp8Depth; ++d) {
            const int64_t bd = bb + d * stride;
            if (bd < b1) {
                c[d] = reinterpret_cast<const uint4*>(codes)[bd];
                sb[d] = s[bd];
            }
        }
    };
    int64_t b = b0 + (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (b < b1) load(b);
    const int kexp = (int)reduce_part(part, npart, red) - 127 - 6;
    __syncthreads();                       // every thread has read the pass-1 bytes before any is rewritten
    uint32_t bad = 0;
    while (b < b1) {
#pragma unroll
        for (int d = 0; d < kFp8Depth; ++d) {
            const int64_t bd = b + d * stride;
            if (bd < b1) bad += fp8_block(c[d], sb[d], v8, s8out, bd, kexp);
        }
        b += kFp8Depth * stride;
        if (b < b1) load(b);
    }
    add_count(bad, n_inexact, red);
    if (ts != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        *ts = ldexpf(1.0f, kexp);          // 2^-133 .. 2^121; below 2^-126 a subnormal
}

}  // namespace

hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
    const int64_t units = rows * (k / 8);
    unsigned g = grid_for(units, kMxUnroll);
    if (g > kMxMaxBlocks) g = kMxMaxBlocks;
    if (ldx == k)
        mx_quantize_kernel<true><<<g, kThreads, 0, s>>>(x, rows, k, ldx, codes, scales);
    else
        mx_quantize_kernel<false><<<g, kThreads, 0, s>>>(x, rows, k, ldx, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                                 uint8_t* codes, uint8_t* scales, hipStream_t s) {
    const int64_t units = rows * (k / 8);
    unsigned g = grid_for(units, kMxUnroll);
    if (g > kMxMaxBlocks) g = kMxMaxBlocks;
    if (ldx == k)
        mxfp8_quantize_kernel<true><<<g, kThreads, 0, s>>>(x, rows, k, ldx, codes, scales);
    else
        mxfp8_quantize_kernel<false><<<g, kThreads, 0, s>>>(x, rows, k, ldx, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_to_mxfp8(const uint8_t* codes, int64_t rows, int64_t k, uint8_t* codes8, hipStream_t s) {
    const int64_t words = rows * (k / 8);
    unsigned g = grid_for(words);
    if (g > kMxMaxBlocks) g = kMxMaxBlocks;
    mx_to_mxfp8_kernel<<<g, kThreads, 0, s>>>(reinterpret_cast<const uint32_t*>(codes), words,
                                              reinterpret_cast<uint2*>(codes8));
    return hipGetLastError();
}

// Pass 1 of an NV quantize with a computed tensor scale; returns the number of
// partial maxima written.
static int launch_nv_amax(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint32_t* amax_ws, hipStream_t s) {
    unsigned g = grid_for(rows * (k / 8), kUnroll);
    if (g > (unsigned)kNvAmaxBlocks) g = kNvAmaxBlocks;
    if (ldx == k)
        nv_amax_kernel<true><<<g, kThreads, 0, s>>>(x, rows, k, ldx, amax_ws);
    else
        nv_amax_kernel<false><<<g, kThreads, 0, s>>>(x, rows, k, ldx, amax_ws);
    return (int)g;
}

hipError_t launch_quantize_nv(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* ts, bool ts_is_input,
                              uint32_t* amax_ws, hipStream_t s) {
    const bool contig = ldx == k;
    const int npart = ts_is_input ? 0 : launch_nv_amax(x, rows, k, ldx, amax_ws, s);
    unsigned gq = grid_for(rows * (k / 16));
    if (gq > kNvMaxBlocks) gq = kNvMaxBlocks;
    if (contig)
        nv_quantize_kernel<true><<<gq, kThreads, 0, s>>>(x, rows, k, ldx, codes, scales, ts, amax_ws, npart);
    else
        nv_quantize_kernel<false><<<gq, kThreads, 0, s>>>(x, rows, k, ldx, codes, scales, ts, amax_ws, npart);
    return hipGetLastError();
}

// ------------------------------------------------------------------ allocation-free NV quantize
// Scratch of the NV quantize for callers that cannot allocate: the pass-1
// partial maxima of the tensor amax (one word per pass-1 workgroup, at most
// kNvAmaxBlocks).  Each GPU holds its own copy of this array for the life of
// the process; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in, not a device address).  Pass 1 writes every word that
// pass 2 reads, so nothing needs clearing between calls; calls that overlap
// in time on one GPU share the array and race.
constexpr int kNvScratchWords = 1024;
static_assert(kNvAmaxBlocks <= kNvScratchWords, "pass 1 writes at most kNvAmaxBlocks partial maxima");
static __device__ __align__(256) uint32_t scratch[kNvScratchWords];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint32_t* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (looked up once per device).
static hipError_t nv_scratch(uint32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<uint32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

size_t nv_scratch_bytes() { return sizeof(uint32_t) * kNvScratchWords; }

hipError_t launch_quantize_nv_noalloc(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, uint8_t* codes,
                                      uint8_t* scales, float* ts, bool ts_is_input, hipStream_t s) {
    uint32_t* ws = nullptr;
    if (!ts_is_input) {
        const hipError_t e = nv_scratch(&ws);
        if (e != hipSuccess) return e;
    }
    return launch_quantize_nv(x, rows, k, ldx, codes, scales, ts, ts_is_input, ws, s);
}

hipError_t launch_kv_append(const uint16_t* x, int64_t tokens, int64_t d, int64_t ldx, const int32_t* slots,
                            uint8_t* codes, uint8_t* scales, int64_t capacity, hipStream_t s) {
    unsigned g = grid_for(tokens * (d / 8), kMxUnroll);
    if (g > kMxMaxBlocks) g = kMxMaxBlocks;
    if (ldx == d)
        mx_quantize_kernel<true, kOutSlots><<<g, kThreads, 0, s>>>(x, tokens, d, ldx, codes, scales, nullptr, 0, slots,
                                                                   capacity);
    else
        mx_quantize_kernel<false, kOutSlots><<<g, kThreads, 0, s>>>(x, tokens, d, ldx, codes, scales, nullptr, 0, slots,
                                                                    capacity);
    return hipGetLastError();
}

hipError_t launch_fake_quant(int fmt, const uint16_t* x, int64_t rows, int64_t k, int64_t ldx, void* out,
                             int out_f32, int64_t ld_out, float* tensor_scale, bool ts_is_input, uint32_t* amax_ws,
                             hipStream_t s) {
    const bool contig = ldx == k && ld_out == k;
    if (fmt == FP4_FMT_MX) {
        unsigned g = grid_for(rows * (k / 8), kMxUnroll);
        if (g > kMxMaxBlocks) g = kMxMaxBlocks;
#define FQ_MX(C, O) mx_quantize_kernel<C, O><<<g, kThreads, 0, s>>>(x, rows, k, ldx, nullptr, nullptr, out, ld_out)
        if (contig)
            out_f32 ? FQ_MX(true, kOutF32) : FQ_MX(true, kOutBf16);
        else
            out_f32 ? FQ_MX(false, kOutF32) : FQ_MX(false, kOutBf16);
#undef FQ_MX
        return hipGetLastError();
    }
    const int npart = ts_is_input ? 0 : launch_nv_amax(x, rows, k, ldx, amax_ws, s);
    unsigned g = grid_for(rows * (k / 16));
    if (g > kNvMaxBlocks) g = kNvMaxBlocks;
#define FQ_NV(C, O) \
    nv_quantize_kernel<C, O><<<g, kThreads, 0, s>>>(x, rows, k, ldx, nullptr, nullptr, tensor_scale, amax_ws, npart, out, ld_out)
    if (contig)
        out_f32 ? FQ_NV(true, kOutF32) : FQ_NV(true, kOutBf16);
    else
        out_f32 ? FQ_NV(false, kOutF32) : FQ_NV(false, kOutBf16);
#undef FQ_NV
    return hipGetLastError();
}

hipError_t launch_ste_backward(const void* g, int g_f32, int64_t rows, int64_t k, int64_t ldg, float* gm, int64_t ldm,
                               int accumulate, hipStream_t s) {
    unsigned gr = grid_for(rows * (k / 8));
    if (gr > kMxMaxBlocks) gr = kMxMaxBlocks;
    if (g_f32)
        ste_backward_kernel<true><<<gr, kThreads, 0, s>>>(g, rows, k, ldg, gm, ldm, accumulate);
    else
        ste_backward_kernel<false><<<gr, kThreads, 0, s>>>(g, rows, k, ldg, gm, ldm, accumulate);
    return hipGetLastError();
}

size_t scale_max_workspace_bytes(int64_t rows, int64_t k) {
    return scale_max_groups(rows * (k / 32));
}

hipError_t launch_remap(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                        uint8_t* scales_nv, float* ts, int32_t* n_inexact, uint8_t* ws, hipStream_t s) {
    const int64_t nb = rows * (k / 32);
    const unsigned g1 = scale_max_groups(nb);
    // without workspace the maxima go to the first output bytes, 2 per block
    // (a multiple of 4: remap_kernel's lanes take aligned groups of 4 blocks)
    const int64_t reserved = ws ? 0 : min((int64_t)((g1 + 1) / 2 + 3) & ~(int64_t)3, nb);
    uint8_t* part = ws ? ws : scales_nv;
    scale_max_kernel<<<g1, kThreads, 0, s>>>(scales, nb, part, n_inexact);
    unsigned g2 = grid_for((nb - reserved + 3) / 4, 1);
    if (g2 > kMxMaxBlocks) g2 = kMxMaxBlocks;
    remap_kernel<<<g2, kThreads, 0, s>>>(codes, scales, scales_nv, part, (int)g1, reserved, nb, ws ? ts : nullptr,
                                         n_inexact);
    if (!ws) remap_kernel<<<1, kThreads, 0, s>>>(codes, scales, scales_nv, part, (int)g1, 0, reserved, ts, n_inexact);
    return hipGetLastError();
}

hipError_t launch_dequant_fp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, uint8_t* v8,
                              uint8_t* s8, float* ts, int32_t* n_inexact, uint8_t* ws, hipStream_t s) {
    const int64_t nb = rows * (k / 32);
    const unsigned g1 = scale_max_groups(nb);
    // without workspace the maxima go to the first value bytes, 32 per block
    const int64_t reserved = ws ? 0 : min((int64_t)(g1 + 31) / 32, nb);
    uint8_t* part = ws ? ws : v8;
    scale_max_kernel<<<g1, kThreads, 0, s>>>(scales, nb, part, n_inexact);
    unsigned g2 = grid_for(nb - reserved, kFp8Depth);
    if (g2 > kMxMaxBlocks) g2 = kMxMaxBlocks;
    fp8_dequant_kernel<<<g2, kThreads, 0, s>>>(codes, scales, v8, s8, part, (int)g1, reserved, nb, ws ? ts : nullptr,
                                               n_inexact);
    if (!ws)
        fp8_dequant_kernel<<<1, kThreads, 0, s>>>(codes, scales, v8, s8, part, (int)g1, 0, reserved, ts, n_inexact);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, const float* ts,
                          int64_t rows, int64_t k, void* out, int out_f32, int64_t ld, hipStream_t s) {
    const int64_t units = rows * (k / 8);
    unsigned g = grid_for(units, kDqUnroll);
    if (g > kDqMaxBlocks) g = kDqMaxBlocks;
    const bool c = ld == k;
    const bool nv = fmt == FP4_FMT_NV;
#define FP4_DQ(NV, F32, C) dequant_kernel<NV, F32, C><<<g, kThreads, 0, s>>>(codes, scales, ts, rows, k, out, ld)
    if (nv) {
        if (out_f32) { if (c) FP4_DQ(true, true, true); else FP4_DQ(true, true, false); }
        else         { if (c) FP4_DQ(true, false, true); else FP4_DQ(true, false, false); }
    } else {
        if (out_f32) { if (c) FP4_DQ(false, true, true); else FP4_DQ(false, true, false); }
        else         { if (c) FP4_DQ(false, false, true); else FP4_DQ(false, false, false); }
    }
#undef FP4_DQ
    return hipGetLastError();
}

}  // namespace fp4
