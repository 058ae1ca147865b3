// Peak-rate microbenchmarks of the MI355X units the block-scaled FP4 kernels
// are bound by, measured rather than taken from the data sheet:
//   * matrix-core rate of each MFMA shape the kernels issue, from registers
//     (8 waves per workgroup, independent accumulators, random operands and
//     scale bytes, no memory or LDS traffic in the timed loop);
//   * device-memory copy bandwidth (a plain 16-byte-per-lane copy);
//   * the per-CU rate of global_load_lds_dwordx4 (global memory to LDS
//     DMA), the copy path of the LDS-staged GEMM tiles, from an L2-resident
//     source so the figure is the path's own limit, not HBM's;
//   * the per-CU LDS read rate of ds_read_b128 (the tiles' fragment reads).
// Each entry point allocates and frees its own buffers, times with HIP events
// around `reps` launches after a warm-up launch, and returns 0 or the HIP error
// code.  Not part of the library's ABI: a separate shared object that
// peak_probe.py loads.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kThreads = 512;          // 8 waves, 2 per SIMD, as in the GEMM tiles
constexpr int kInWords = 4096 * 20;    // random operand words; lane t reads words (t % 4096) * 20 ...

// Matrix-core rate.  kind 0: scaled E2M1 x E2M1 16x16x128 (32 accumulators
// per wave); 1: scaled E2M1 x E2M1 32x32x64 (8 accumulators); 2: E2M1 x E4M3
// 16x16x128 (the W4A8 pairing); 3: f16 16x16x32 (the NV tiles' expanded
// operands).  Every MFMA of a round reads the same operand registers and
// writes its own accumulator, so the rounds are independent matrix work.
template <int kKind>
__global__ __launch_bounds__(kThreads, 1) void mfma_rate_kernel(const int* __restrict__ in, float* __restrict__ out,
                                                                int iters) {
    const int t = blockIdx.x * kThreads + threadIdx.x;
    const int* p = in + (t & 4095) * 20;
    const v8i a4 = {p[0], p[1], p[2], p[3], 0, 0, 0, 0};
    const v8i a4b = {p[4], p[5], p[6], p[7], 0, 0, 0, 0};
    const v8i a8 = {p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]};
    const int sa = 120 + (p[16] & 7), sb = 120 + (p[17] & 7);
    float s = 0.f;
    if constexpr (kKind == 1) {
        v16f acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4((i & 1) ? a4b : a4, a4, acc[i], 4, 4, 0, sa, 0,
                                                                         sb);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) s += acc[i][0] + acc[i][15];
    } else if constexpr (kKind == 3) {
        h8_t h, hb;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // small finite fp16 values from the random bits (exponent field 13..16)
            h[i] = (_Float16)((float)((p[i] >> 8) & 0xFF) * (1.0f / 256.0f) + 0.5f);
            hb[i] = (_Float16)((float)(p[8 + i] & 0xFF) * (1.0f / 256.0f) + 0.5f);
        }
        v4f acc[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16((i & 1) ? hb : h, h, acc[i], 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) s += acc[i][0] + acc[i][3];
    } else {
        v4f acc[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if constexpr (kKind == 0)
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4((i & 1) ? a4b : a4, a4, acc[i], 4, 4, 0, sa,
                                                                              0, sb);
                else   // E2M1 first operand, E4M3 second, as the W4A8 tile issues them
                    acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4((i & 1) ? a4b : a4, a8, acc[i], 4, 0, 0, sa,
                                                                              0, sb);
            }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) s += acc[i][0] + acc[i][3];
    }
    out[t] = s;
}

// Plain copy, one 16-byte load and store per lane and iteration.
__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ void wait_vm_zero() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

constexpr int kDmaPerRound = 8;        // 1 KiB DMAs per wave and round: 64 KiB per workgroup
constexpr int kDmaSrcBytes = 1 << 20;  // source buffer (L2-resident after the warm-up launch)

// Global-to-LDS DMA stream: each round every wave copies kDmaPerRound KiB of
// the source (wave-private LDS region of 8 KiB, source offset rotating within
// the 1 MiB buffer) and waits for them, so a workgroup moves 64 KiB per round.
__global__ __launch_bounds__(kThreads, 1) void dma_rate_kernel(const uint8_t* __restrict__ src, float* __restrict__ out,
                                                               int iters) {
    __shared__ __align__(16) uint8_t lds[8 * kDmaPerRound * 1024];
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const uint32_t lane_off = (threadIdx.x & 63) * 16;
    const uint32_t lbase = (uint32_t)(uintptr_t)(lds_ptr_t)(void*)lds + wave * kDmaPerRound * 1024;
    for (int it = 0; it < iters; ++it) {
        // 64 KiB window per round, start rotating over the 1 MiB source
        const uint32_t win = (uint32_t)((blockIdx.x * 7 + it) % (kDmaSrcBytes / 65536)) * 65536u;
#pragma unroll
        for (int q = 0; q < kDmaPerRound; ++q)
            dma16(src, win + (uint32_t)(wave * kDmaPerRound + q) * 1024u + lane_off, lbase + q * 1024);
        wait_vm_zero();
    }
    __syncthreads();
    out[blockIdx.x * kThreads + threadIdx.x] = (float)lds[(threadIdx.x * 97) % sizeof(lds)];
}

// LDS read rate: every wave reads 16-byte chunks of its own 8 KiB region with
// ds_read_b128 (consecutive lanes, consecutive chunks: no bank conflicts), 8
// reads per round, the chunk set rotating with the round so no read can be
// hoisted out of the loop.
__global__ __launch_bounds__(kThreads, 1) void lds_read_kernel(float* __restrict__ out, int iters) {
    __shared__ __align__(16) uint4 lds[8 * 512];            // 64 KiB: 8 waves x 512 chunks
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int i = threadIdx.x; i < 8 * 512; i += kThreads) lds[i] = make_uint4(i, i * 3u, i * 5u, i * 7u);
    __syncthreads();
    uint4 acc = make_uint4(0, 0, 0, 0);
    const uint4* mine = lds + wave * 512;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const uint4 v = mine[((it + q) & 7) * 64 + lane];
            acc.x ^= v.x;
            acc.y += v.y;
            acc.z ^= v.z;
            acc.w += v.w;
        }
    }
    out[blockIdx.x * kThreads + threadIdx.x] = (float)(acc.x ^ acc.y ^ acc.z ^ acc.w);
}

template <typename F>
hipError_t timed(F launch, int reps, float* ms) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        launch();   // warm-up
        e = hipGetLastError();
    }
    if (e == hipSuccess) {
        hipEventRecord(e0, 0);
        for (int r = 0; r < reps; ++r) launch();
        hipEventRecord(e1, 0);
        e = hipEventSynchronize(e1);
    }
    if (e == hipSuccess) e = hipEventElapsedTime(ms, e0, e1);
    if (e == hipSuccess) e = hipGetLastError();
    if (e0) hipEventDestroy(e0);
    if (e1) hipEventDestroy(e1);
    return e;
}

}  // namespace

extern "C" {

// Matrix-core rate of MFMA kind 0..3 (see mfma_rate_kernel) on `groups`
// workgroups of 8 waves, `iters` rounds each; *tflops = the rate in TFLOP/s.
int peak_mfma(int kind, int groups, int iters, int reps, double* tflops) {
    if (kind < 0 || kind > 3 || groups <= 0 || iters <= 0 || reps <= 0 || !tflops) return -1;
    int* in = nullptr;
    float* out = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&in, kInWords * sizeof(int))) != hipSuccess) return (int)e;
    if ((e = hipMalloc(&out, (size_t)groups * kThreads * sizeof(float))) != hipSuccess) {
        hipFree(in);
        return (int)e;
    }
    int* h = static_cast<int*>(malloc(kInWords * sizeof(int)));
    if (!h) {
        hipFree(in);
        hipFree(out);
        return -1;
    }
    uint32_t x = 12345u;
    for (int i = 0; i < kInWords; ++i) {   // xorshift32 random operand bits
        x ^= x << 13;
        x ^= x >> 17;
        x ^= x << 5;
        h[i] = (int)x;
    }
    e = hipMemcpy(in, h, kInWords * sizeof(int), hipMemcpyHostToDevice);
    free(h);
    float ms = 0.f;
    if (e == hipSuccess) {
        auto launch = [&]() {
            switch (kind) {
                case 0: mfma_rate_kernel<0><<<groups, kThreads>>>(in, out, iters); break;
                case 1: mfma_rate_kernel<1><<<groups, kThreads>>>(in, out, iters); break;
                case 2: mfma_rate_kernel<2><<<groups, kThreads>>>(in, out, iters); break;
                default: mfma_rate_kernel<3><<<groups, kThreads>>>(in, out, iters); break;
            }
        };
        e = timed(launch, reps, &ms);
    }
    hipFree(in);
    hipFree(out);
    if (e != hipSuccess) return (int)e;
    // flops per MFMA: 2 * 16*16*128, 2 * 32*32*64, 2 * 16*16*128, 2 * 16*16*32; MFMAs per wave and round: 32, 8, 32, 32
    const double per_mfma[4] = {65536.0, 131072.0, 65536.0, 16384.0};
    const double per_round[4] = {32.0, 8.0, 32.0, 32.0};
    const double flop = per_mfma[kind] * per_round[kind] * iters * (double)groups * 8.0 * reps;
    *tflops = flop / (ms * 1e-3) / 1e12;
    return 0;
}

// Device copy of `bytes` (a multiple of 16) from one buffer to another;
// *gbps = (read + written bytes) / time in GB/s.
int peak_copy(int64_t bytes, int reps, double* gbps) {
    if (bytes <= 0 || bytes % 16 || reps <= 0 || !gbps) return -1;
    void *src = nullptr, *dst = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&src, bytes)) != hipSuccess) return (int)e;
    if ((e = hipMalloc(&dst, bytes)) != hipSuccess) {
        hipFree(src);
        return (int)e;
    }
    e = hipMemset(src, 1, bytes);
    float ms = 0.f;
    if (e == hipSuccess) {
        const int64_t n = bytes / 16;
        auto launch = [&]() {
            copy_kernel<<<8192, 256>>>(static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
        };
        e = timed(launch, reps, &ms);
    }
    hipFree(src);
    hipFree(dst);
    if (e != hipSuccess) return (int)e;
    *gbps = 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9;
    return 0;
}

// Global-to-LDS DMA rate on `groups` workgroups (one per CU at most: the
// kernel's LDS and launch bounds keep one resident), `iters` rounds of 64 KiB
// each; *gbps_per_group = bytes moved per workgroup per second, in GB/s.
int peak_lds_dma(int groups, int iters, int reps, double* gbps_per_group) {
    if (groups <= 0 || iters <= 0 || reps <= 0 || !gbps_per_group) return -1;
    uint8_t* src = nullptr;
    float* out = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&src, kDmaSrcBytes)) != hipSuccess) return (int)e;
    if ((e = hipMalloc(&out, (size_t)groups * kThreads * sizeof(float))) != hipSuccess) {
        hipFree(src);
        return (int)e;
    }
    e = hipMemset(src, 3, kDmaSrcBytes);
    float ms = 0.f;
    if (e == hipSuccess) {
        auto launch = [&]() { dma_rate_kernel<<<groups, kThreads>>>(src, out, iters); };
        e = timed(launch, reps, &ms);
    }
    hipFree(src);
    hipFree(out);
    if (e != hipSuccess) return (int)e;
    *gbps_per_group = 65536.0 * iters * reps / (ms * 1e-3) / 1e9;
    return 0;
}

// LDS read rate on `groups` workgroups, `iters` rounds of 8 KiB per wave;
// *gbps_per_group = bytes read per workgroup per second, in GB/s.
int peak_lds_read(int groups, int iters, int reps, double* gbps_per_group) {
    if (groups <= 0 || iters <= 0 || reps <= 0 || !gbps_per_group) return -1;
    float* out = nullptr;
    hipError_t e;
    if ((e = hipMalloc(&out, (size_t)groups * kThreads * sizeof(float))) != hipSuccess) return (int)e;
    float ms = 0.f;
    auto launch = [&]() { lds_read_kernel<<<groups, kThreads>>>(out, iters); };
    e = timed(launch, reps, &ms);
    hipFree(out);
    if (e != hipSuccess) return (int)e;
    *gbps_per_group = 8.0 * 8192.0 * iters * reps / (ms * 1e-3) / 1e9;
    return 0;
}

}  // extern "C"
