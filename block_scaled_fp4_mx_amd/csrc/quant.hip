// Block-scaled FP4 quantize / dequantize / MX->NV remap kernels for gfx950.
//
// All four are HBM-streaming kernels: one lane owns 8 consecutive elements
// (one 16-byte bf16 load, one 4-byte code store), so a wavefront reads 1 KiB of
// contiguous input per instruction.  An MX block (32 elements) spans 4 adjacent
// lanes and an NV group (16 elements) 2 lanes; the block/group amax is
// combined across those lanes with DPP quad permutes (no LDS traffic).
#include "fp4_internal.h"

namespace fp4 {
namespace {

constexpr int kThreads = 256;

// DPP quad permutations: lane i of each group of 4 reads lane perm[i].
__device__ __forceinline__ uint32_t quad_swap1(uint32_t v) {   // (1,0,3,2)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t v) {   // (2,3,0,1)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
}

// |x| of the two bf16 halves of a word, as 15-bit magnitudes (their integer order
// is the order of the finite values).
__device__ __forceinline__ uint32_t mag_max2(uint32_t w) {
    return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
}

inline unsigned grid_for(int64_t units) {
    int64_t b = (units + kThreads - 1) / kThreads;
    if (b > (1 << 20)) b = 1 << 20;
    return (unsigned)(b < 1 ? 1 : b);
}

// ------------------------------------------------------------------ MX quantize
// Per 32-block: amax from the bf16 magnitude bits; the biased exponent field e
// of amax gives floor(log2 amax) = e - 127 for normal amax, so the block
// exponent E = e - 129 and the scale byte E + 127 = e - 2, clamped at 0 (which
// also covers zero and subnormal amax, whose floor(log2) is below -126).
// Elements are scaled by 2^-E (exact: a power of two applied to a bf16 value,
// result below 8) and rounded to E2M1 with nearest-even.
template <bool kContig>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += stride) {
        int64_t xo;
        if (kContig) {
            xo = u * 8;
        } else {
            const int64_t r = u / upr;
            xo = r * ldx + (u - r * upr) * 8;
        }
        const uint4 v = *reinterpret_cast<const uint4*>(x + xo);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t am = max(max(mag_max2(w[0]), mag_max2(w[1])), max(mag_max2(w[2]), mag_max2(w[3])));
        am = max(am, quad_swap1(am));
        am = max(am, quad_swap2(am));
        const uint32_t e = am >> 7;
        const uint32_t sbyte = e > 2u ? e - 2u : 0u;
        const float inv = __uint_as_float((254u - sbyte) << 23);      // 2^-E, E = sbyte - 127
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            const float a = __uint_as_float((b & 0x7FFFu) << 16);
            const uint32_t idx = e2m1_index_rne(__fmul_rn(a, inv));
            packed |= (((b >> 12) & 8u) | idx) << (4 * i);
        }
        reinterpret_cast<uint32_t*>(codes)[u] = packed;
        if ((threadIdx.x & 3) == 0) scales[u >> 2] = (uint8_t)sbyte;
    }
}

// ------------------------------------------------------------------ NV quantize
__global__ void nv_amax_init_kernel(uint32_t* amax) { *amax = 0u; }

template <bool kContig>
__global__ __launch_bounds__(kThreads) void nv_amax_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx, uint32_t* amax_out) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t am = 0;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += stride) {
        int64_t xo;
        if (kContig) {
            xo = u * 8;
        } else {
            const int64_t r = u / upr;
            xo = r * ldx + (u - r * upr) * 8;
        }
        const uint4 v = *reinterpret_cast<const uint4*>(x + xo);
        am = max(am, max(max(mag_max2(v.x), mag_max2(v.y)), max(mag_max2(v.z), mag_max2(v.w))));
    }
    for (int off = 32; off > 0; off >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t m = red[0];
        for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
        atomicMax(amax_out, m);
    }
}

// s_t = fp32(amax / 2688): the fp64 quotient is correctly rounded, and rounding
// it again to fp32 is exact because an 8-bit numerator over 21 * 2^7 is either
// a short dyadic (exact) or far from every fp32 rounding midpoint.
__global__ void nv_tensor_scale_kernel(const uint32_t* amax, float* ts) {
    const float a = __uint_as_float(*amax << 16);
    *ts = (float)((double)a / 2688.0);
}

// One lane owns 8 elements; a 16-group spans lanes (2i, 2i+1).
//   s_g = E4M3(amax_g / (6 s_t))  computed in fp64 (exact quotient rounding).
//   code = E2M1(|x| / d), d = s_g s_t (exact in fp64, <= 28 bits).
// Codes use a bracket: with r = 1/d, v_lo = |x| * r(1 - 2^-22) and
// v_hi = |x| * r(1 + 2^-22) in fp32 lie strictly below and above the exact
// quotient, so equal E2M1 roundings of both are the exact rounding.  Otherwise
// the quotient is within 2^-21 of the midpoint between the two candidates and
// |x| is compared with midpoint * d exactly in fp64.
template <bool kContig>
__global__ __launch_bounds__(kThreads) void nv_quantize_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t k, int64_t ldx,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const float* __restrict__ ts) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const double st = (double)*ts;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += stride) {
        int64_t xo;
        if (kContig) {
            xo = u * 8;
        } else {
            const int64_t r = u / upr;
            xo = r * ldx + (u - r * upr) * 8;
        }
        const uint4 v = *reinterpret_cast<const uint4*>(x + xo);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t am = max(max(mag_max2(w[0]), mag_max2(w[1])), max(mag_max2(w[2]), mag_max2(w[3])));
        am = max(am, quad_swap1(am));
        const double amax = (double)__uint_as_float(am << 16);
        uint32_t sg = (st > 0.0) ? e4m3_rne_sat(amax / (6.0 * st)) : 0u;
        uint32_t packed = 0;
        if (sg != 0u) {
            const double d = (double)e4m3_value(sg) * st;
            const double r = 1.0 / d;
            const bool fast = r < 1.0e37;
            const float r_lo = (float)(r * (1.0 - 0x1p-22));
            const float r_hi = (float)(r * (1.0 + 0x1p-22));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t b = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
                const float a = __uint_as_float((b & 0x7FFFu) << 16);
                uint32_t idx;
                const uint32_t i_lo = fast ? e2m1_index_rne(__fmul_rn(a, r_lo)) : 0u;
                const uint32_t i_hi = fast ? e2m1_index_rne(__fmul_rn(a, r_hi)) : 7u;
                if (i_lo == i_hi) {
                    idx = i_lo;
                } else {
                    // exact decision among all eight magnitudes (rare)
                    const double ad = (double)a;
                    idx = 0;
#pragma unroll
                    for (uint32_t j = 0; j < 7; ++j) {
                        const double t = 0.5 * ((double)e2m1_mag(j) + (double)e2m1_mag(j + 1)) * d;
                        // tie at midpoint j|j+1 goes to the even index
                        const bool up = (j & 1u) ? (ad >= t) : (ad > t);
                        idx += up ? 1u : 0u;
                    }
                }
                packed |= (((b >> 12) & 8u) | idx) << (4 * i);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t b = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
                packed |= ((b >> 12) & 8u) << (4 * i);
            }
        }
        reinterpret_cast<uint32_t*>(codes)[u] = packed;
        if ((threadIdx.x & 1) == 0) scales[u >> 1] = (uint8_t)sg;
    }
}

// ------------------------------------------------------------------ dequant
template <bool kNV, bool kF32, bool kContig>
__global__ __launch_bounds__(kThreads) void dequant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ ts, int64_t rows, int64_t k, void* __restrict__ out, int64_t ld) {
    const int64_t upr = k >> 3;
    const int64_t total = rows * upr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const float st = kNV ? *ts : 1.0f;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += stride) {
        const uint32_t c = reinterpret_cast<const uint32_t*>(codes)[u];
        float sc;
        if (kNV) {
            sc = e4m3_value(scales[u >> 1]);
        } else {
            const uint32_t sb = scales[u >> 2];
            // 2^(sb - 127); sb == 0 is the fp32 subnormal 2^-127
            sc = sb ? __uint_as_float(sb << 23) : __uint_as_float(0x00400000u);
        }
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t code = (c >> (4 * i)) & 0xFu;
            float val = __fmul_rn(e2m1_mag(code & 7u), sc);   // exact (<= 6 significant bits)
            if (kNV) val = __fmul_rn(val, st);                 // the single rounding
            f[i] = (code & 8u) ? -val : val;
        }
        int64_t o;
        if (kContig) {
            o = u * 8;
        } else {
            const int64_t r = u / upr;
            o = r * ld + (u - r * upr) * 8;
        }
        if (kF32) {
            float4* p = reinterpret_cast<float4*>(static_cast<float*>(out) + o);
            p[0] = make_float4(f[0], f[1], f[2], f[3]);
            p[1] = make_float4(f[4], f[5], f[6], f[7]);
        } else {
            uint4 q;
            q.x = f32_to_bf16_rne(f[0]) | (f32_to_bf16_rne(f[1]) << 16);
            q.y = f32_to_bf16_rne(f[2]) | (f32_to_bf16_rne(f[3]) << 16);
            q.z = f32_to_bf16_rne(f[4]) | (f32_to_bf16_rne(f[5]) << 16);
            q.w = f32_to_bf16_rne(f[6]) | (f32_to_bf16_rne(f[7]) << 16);
            *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + o) = q;
        }
    }
}

// ------------------------------------------------------------------ MX -> NV remap
// Pass 1 reduces the largest scale byte into *n_inexact (used as scratch);
// pass 2 turns it into s_t = 2^(E_max - 8) and clears the counter; pass 3 writes
// both E4M3 group scales of every block and counts blocks that lose precision.
__global__ void remap_init_kernel(int32_t* n) { *n = 0; }

__global__ __launch_bounds__(kThreads) void remap_max_kernel(const uint8_t* __restrict__ s, int64_t nb,
                                                             int32_t* mx) {
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nb; i += stride) m = max(m, (uint32_t)s[i]);
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    __shared__ uint32_t red[kThreads / 64];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; ++i) m = max(m, red[i]);
        atomicMax(mx, (int32_t)m);
    }
}

__global__ void remap_scale_kernel(int32_t* n, float* ts) {
    const int emax = *n - 127;
    *ts = ldexpf(1.0f, emax - 8);          // 2^-135 .. 2^119; below 2^-126 a subnormal
    *n = 0;
}

__global__ __launch_bounds__(kThreads) void remap_kernel(const uint8_t* __restrict__ codes,
                                                         const uint8_t* __restrict__ s, int64_t nb,
                                                         uint8_t* __restrict__ snv, const float* ts,
                                                         int32_t* n_inexact) {
    const int kexp = ilogbf(*ts);          // k = E_max - 8 (exact for subnormal 2^k too)
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nb; i += stride) {
        const int j = (int)s[i] - 127 - kexp;              // <= 8
        uint32_t sg;
        if (j >= -6) {
            sg = (uint32_t)(j + 7) << 3;                      // normal 2^j
        } else if (j >= -9) {
            sg = 1u << (j + 9);                               // subnormal 2^j = 2^(j+9) * 2^-9
        } else {
            sg = 0u;                                          // 2^-10 ties to 0, below rounds to 0
            const uint4* c = reinterpret_cast<const uint4*>(codes + i * 16);
            const uint4 a = c[0];
            const uint32_t nz = (a.x | a.y | a.z | a.w) & 0x77777777u;
            if (nz) atomicAdd(n_inexact, 1);
        }
        const uint16_t pair = (uint16_t)(sg | (sg << 8));
        reinterpret_cast<uint16_t*>(snv)[i] = pair;
    }
}

}  // namespace

hipError_t launch_quantize_mx(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
    const int64_t units = rows * (k / 8);
    if (ldx == k)
        mx_quantize_kernel<true><<<grid_for(units), kThreads, 0, s>>>(x, rows, k, ldx, codes, scales);
    else
        mx_quantize_kernel<false><<<grid_for(units), kThreads, 0, s>>>(x, rows, k, ldx, codes, scales);
    return hipGetLastError();
}

hipError_t launch_quantize_nv(const uint16_t* x, int64_t rows, int64_t k, int64_t ldx,
                              uint8_t* codes, uint8_t* scales, float* ts, bool ts_is_input,
                              uint32_t* amax_ws, hipStream_t s) {
    const int64_t units = rows * (k / 8);
    const bool contig = ldx == k;
    if (!ts_is_input) {
        nv_amax_init_kernel<<<1, 1, 0, s>>>(amax_ws);
        unsigned g = grid_for(units);
        if (g > 2048) g = 2048;
        if (contig)
            nv_amax_kernel<true><<<g, kThreads, 0, s>>>(x, rows, k, ldx, amax_ws);
        else
            nv_amax_kernel<false><<<g, kThreads, 0, s>>>(x, rows, k, ldx, amax_ws);
        nv_tensor_scale_kernel<<<1, 1, 0, s>>>(amax_ws, ts);
    }
    if (contig)
        nv_quantize_kernel<true><<<grid_for(units), kThreads, 0, s>>>(x, rows, k, ldx, codes, scales, ts);
    else
        nv_quantize_kernel<false><<<grid_for(units), kThreads, 0, s>>>(x, rows, k, ldx, codes, scales, ts);
    return hipGetLastError();
}

hipError_t launch_remap(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                        uint8_t* scales_nv, float* ts, int32_t* n_inexact, hipStream_t s) {
    const int64_t nb = rows * (k / 32);
    remap_init_kernel<<<1, 1, 0, s>>>(n_inexact);
    unsigned g = grid_for(nb);
    if (g > 1024) g = 1024;
    remap_max_kernel<<<g, kThreads, 0, s>>>(scales, nb, n_inexact);
    remap_scale_kernel<<<1, 1, 0, s>>>(n_inexact, ts);
    remap_kernel<<<grid_for(nb), kThreads, 0, s>>>(codes, scales, nb, scales_nv, ts, n_inexact);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const uint8_t* codes, const uint8_t* scales, const float* ts,
                          int64_t rows, int64_t k, void* out, int out_f32, int64_t ld, hipStream_t s) {
    const int64_t units = rows * (k / 8);
    const unsigned g = grid_for(units);
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
