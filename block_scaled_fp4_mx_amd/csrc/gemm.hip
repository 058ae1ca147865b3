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
#include "gemm_mx_tile.h"
#include "gemm_nv_wide.h"
#include "gemm_w4a8_tile.h"
#include "mma_core.h"

namespace fp4 {
namespace {

constexpr int kBM = 128, kBN = 128, kThreads = 256;
constexpr bool kW8Lag = true;   // W4A8 tile: half the waves run half a step behind
constexpr int64_t kSkinnyMinN = 4096;   // B rows from which few-row A products use the streaming kernel
constexpr int kSkinnyKF = 1;            // 16-row B fragments per wave in the streaming kernel

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

// Block tile 128x128: four waves in a 2x2 grid, each a 64x64 MMA core.  FMT is
// FP4_FMT_MX, FP4_FMT_NV or kFmtW4A8 (MXFP8 A times MXFP4 B).
constexpr int kFmtW4A8 = 2;
template <int FMT>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts,
    int64_t m, int64_t n, int64_t k, void* __restrict__ c, int c_f32, int64_t ldc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * kBM + (wave >> 1) * 64;
    const int64_t n0 = (int64_t)blockIdx.x * kBN + (wave & 1) * 64;
    const int blk = FMT == FP4_FMT_NV ? 16 : 32;
    const int64_t a_row_bytes = FMT == kFmtW4A8 ? k : k / 2;
    const int lr = lane & 15;
    const uint8_t *a_rows[4], *a_srow[4], *b_rows[4], *b_srow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = m0 + i * 16 + lr;
        a_rows[i] = r < m ? ac + r * a_row_bytes : nullptr;
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
    } else if (FMT == kFmtW4A8) {
        mma_w4a8_64x64(acc, a_rows, a_srow, b_rows, b_srow, k, lane);
    } else {
        mma_nv_64x64(acc, a_rows, a_srow, b_rows, b_srow, k, lane);
        scale = __fmul_rn(*ats, *bts);
    }
    store_tile(acc, c, c_f32, ldc, m, n, m0, n0, lane, scale);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// MX GEMM for few A rows (m <= 64) and many B rows, e.g. indexer scores of a
// handful of queries against a long key cache: the work is streaming B once.
// A workgroup owns 64 B rows (4 waves x one 16-row fragment) and all A rows
// (NQ fragments of 16).  K runs in chunks of 512 values: the workgroup stages
// the chunk of A (codes and scales) in LDS once, and each wave reads its A
// fragments from there, so A crosses L2 once per workgroup rather than once
// per wave; the wave's B chunks and scales come straight from global memory,
// issued before the A staging so their latency overlaps it.  Per 128-value
// step a lane carries one 16-byte B chunk and its scale byte, and issues NQ
// scaled MFMAs with the B fragment first, so its accumulator values are 4
// consecutive B rows (output columns) of one A row: one 16-byte (fp32) or
// 8-byte (bf16) store each.  Rows past m or n are clamped for the loads and
// never stored.  LDS: A row r's 16-byte chunk c at chunk c ^ (r & 15), so the
// 16 rows a fragment read touches sit in 16 different bank groups.
constexpr int kSkChunkK = 512;                      // K values staged per chunk
constexpr int kSkRowB = kSkChunkK / 2;              // code bytes per staged A row
template <int NQ, int KF>
__global__ __launch_bounds__(256) void gemm_mx_skinny_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int64_t m, int64_t n, int64_t k, void* __restrict__ c, int c_f32, int64_t ldc) {
    __shared__ __align__(16) uint8_t a_lds[NQ * 16 * kSkRowB];
    __shared__ __align__(16) uint8_t as_lds[NQ * 16 * 16];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int lr = lane & 15, lk = lane >> 4;
    const int64_t kb = k / 2, kbl = k / 32;
    const int64_t n0 = (int64_t)blockIdx.x * (64 * KF) + wave * (16 * KF);
    const uint8_t* bp[KF];
    const uint8_t* bsp[KF];
#pragma unroll
    for (int f = 0; f < KF; ++f) {
        const int64_t brow = min(n0 + f * 16 + lr, n - 1);
        bp[f] = bc + brow * kb + lk * 16;
        bsp[f] = bs + brow * kbl + lk;
    }
    v4f acc[KF][NQ];
#pragma unroll
    for (int f = 0; f < KF; ++f)
#pragma unroll
        for (int i = 0; i < NQ; ++i) acc[f][i] = v4f{0.f, 0.f, 0.f, 0.f};
    const int nsteps = (int)(k / 128);
    for (int s0 = 0; s0 < nsteps; s0 += 4) {
        const int ns = min(4, nsteps - s0);            // steps in this chunk
        uint4 bv[KF][4];
        int sb[KF][4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < ns) {
#pragma unroll
                for (int f = 0; f < KF; ++f) {
                    bv[f][q] = *reinterpret_cast<const uint4*>(bp[f] + (s0 + q) * 64);
                    sb[f][q] = bsp[f][(s0 + q) * 4];
                }
            }
        __syncthreads();                                // the previous chunk's A reads are done
        // stage A: NQ*16 rows x (ns*64) code bytes and ns*4 scale bytes
        const int cpr = ns * 4;                         // 16-byte code chunks per row in this chunk
        for (int e = t; e < NQ * 16 * cpr; e += 256) {
            const int r = e / cpr, ch = e - r * cpr;
            const int64_t arow = min((int64_t)r, m - 1);
            const uint4 v = *reinterpret_cast<const uint4*>(ac + arow * kb + (int64_t)s0 * 64 + ch * 16);
            *reinterpret_cast<uint4*>(a_lds + r * kSkRowB + ((ch ^ (r & 15)) << 4)) = v;
        }
        for (int e = t; e < NQ * 16 * cpr; e += 256) {
            const int r = e / cpr, b = e - r * cpr;    // scale byte b of the chunk (cpr = ns*4 blocks)
            const int64_t arow = min((int64_t)r, m - 1);
            as_lds[r * 16 + b] = as[arow * kbl + (int64_t)s0 * 4 + b];
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q >= ns) break;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int r = i * 16 + lr, ch = q * 4 + lk;
                const uint4 av = *reinterpret_cast<const uint4*>(a_lds + r * kSkRowB + ((ch ^ (r & 15)) << 4));
                const int sa = as_lds[r * 16 + q * 4 + lk];
                const v8i af = v8i{(int)av.x, (int)av.y, (int)av.z, (int)av.w, 0, 0, 0, 0};
#pragma unroll
                for (int f = 0; f < KF; ++f)
                    acc[f][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        v8i{(int)bv[f][q].x, (int)bv[f][q].y, (int)bv[f][q].z, (int)bv[f][q].w, 0, 0, 0, 0}, af,
                        acc[f][i], 4, 4, 0, sb[f][q], 0, sa);
            }
        }
    }
    const int esz = c_f32 ? 4 : 2;
#pragma unroll
    for (int f = 0; f < KF; ++f) {
        const int64_t col = n0 + f * 16 + lk * 4;
        const bool vec = ((ldc * esz) & (c_f32 ? 15 : 7)) == 0 && col + 4 <= n;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int64_t row = i * 16 + lr;
            if (row >= m || col >= n) continue;
            const v4f v = acc[f][i];
            if (c_f32) {
                float* dst = static_cast<float*>(c) + row * ldc + col;
                if (vec) {
                    __builtin_nontemporal_store(u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                        __float_as_uint(v[2]), __float_as_uint(v[3])},
                                                reinterpret_cast<u32x4_t*>(dst));
                } else {
                    for (int e = 0; e < 4 && col + e < n; ++e) dst[e] = v[e];
                }
            } else {
                uint16_t* dst = static_cast<uint16_t*>(c) + row * ldc + col;
                if (vec) {
                    *reinterpret_cast<uint2*>(dst) = make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                                                f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
                } else {
                    for (int e = 0; e < 4 && col + e < n; ++e) dst[e] = (uint16_t)f32_to_bf16_rne(v[e]);
                }
            }
        }
    }
}

// Tile order: consecutive workgroups go to different XCDs (round robin), so
// workgroup b is given tile (b % 8) * (tiles / 8) + b / 8 when the tile count
// is a multiple of 8: each XCD then owns a contiguous run of tiles, and tiles
// are numbered in groups of 4 tile-rows (column-major inside a group), so an
// XCD's run is a compact block of tiles that shares A and B slabs in its L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    int t = blockIdx.x;
    if ((total & 7) == 0) t = (t & 7) * (total >> 3) + (t >> 3);
    constexpr int G = 4;
    const int group = t / (G * tiles_n);
    const int rows_in_group = min(G, tiles_m - group * G);
    const int r = t - group * G * tiles_n;
    tm = group * G + r % rows_in_group;
    tn = r / rows_in_group;
}

// A whole 16-byte piece of C; kStream: a non-temporal store (measured faster
// for the W4A8 and NV GEMMs' outputs, 1% slower for the MX GEMM's).
template <bool kStream>
__device__ __forceinline__ void store_piece(uint8_t* dst, uint4 v) {
    if (kStream)
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(dst));
    else
        *reinterpret_cast<uint4*>(dst) = v;
}

// Stores rows_pass rows of a tile staged in LDS (row r's 16-byte chunk c at
// chunk c ^ (r & 15), rowb bytes per row) to C rows grow0 .. and columns n0 ..,
// one 16-byte piece per thread and iteration; pieces past m or n are dropped
// or written element by element.
template <bool kStream>
__device__ __forceinline__ void store_rows_from_lds(const uint8_t* csm, int rows_pass, int chunks_row, int rowb,
                                                    int64_t grow0, int64_t n0, int64_t m, int64_t n, void* c,
                                                    int c_f32, int64_t ldc, bool vec) {
    const int esz = c_f32 ? 4 : 2;
    for (int q = threadIdx.x; q < rows_pass * chunks_row; q += blockDim.x) {
        const int row = q / chunks_row, ch = q - row * chunks_row;
        const int64_t grow = grow0 + row;
        const int64_t gcol = n0 + ch * (16 / esz);
        if (grow >= m || gcol >= n) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(csm + row * rowb + ((ch ^ (row & 15)) << 4));
        uint8_t* dst = static_cast<uint8_t*>(c) + (grow * ldc + gcol) * esz;
        if (vec && gcol + 16 / esz <= n) {
            store_piece<kStream>(dst, v);
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            for (int e = 0; e < 16 / esz && gcol + e < n; ++e) {
                if (c_f32)
                    reinterpret_cast<uint32_t*>(dst)[e] = w[e];
                else
                    reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
            }
        }
    }
}

// MX GEMM on 256 x 256 tiles (LDS-staged, see gemm_mx_tile.h).
__global__ __launch_bounds__(kTileThreads, 1) void gemm_mx_256_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int64_t m, int64_t n, int64_t k, void* __restrict__ c, int c_f32,
    int64_t ldc, int tiles_m, int tiles_n) {
    __shared__ __align__(16) MxSmem sm;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kTileM, n0 = (int64_t)tn * kTileN;
    const int64_t kbytes = k / 2, kblocks = k / 32;
    const int t = threadIdx.x;
    MxDenseSrc A, B;
    mx_dense_src(A, ac, as, m0, m, kbytes, kblocks);
    mx_dense_src(B, bc, bs, n0, n, kbytes, kblocks);
    v4f acc[kWaveFragsN][8];
#pragma unroll
    for (int j = 0; j < kWaveFragsN; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
    mx_tile_mainloop_rows(sm, A, B, kblocks, acc, m - m0 - (int64_t)(threadIdx.x >> 8) * 128, m - m0);

    // Epilogue through LDS: the tile (bf16: all 256 rows; fp32: 128 rows per
    // pass) is written in the accumulator layout, then stored row by row in
    // 16-byte pieces, so every global store instruction writes whole rows of
    // the tile.  A row's 16-byte chunk c sits at chunk c ^ (row & 15), which
    // spreads the 16 rows a fragment store touches over the banks.
    const int lane = t & 63, wave = t >> 6, wm = wave >> 2, wn = wave & 3;
    const int lr = lane & 15, lk = lane >> 4;
    const int esz = c_f32 ? 4 : 2;
    const int rowb = kTileN * esz;                   // bytes of one tile row
    const int rows_pass = c_f32 ? 128 : 256;
    const int chunks_row = rowb / 16;
    const bool vec = ((ldc * esz) & 15) == 0;
    uint8_t* csm = reinterpret_cast<uint8_t*>(&sm);
    for (int pass = 0; pass < kTileM / rows_pass; ++pass) {
        __syncthreads();                             // the stages (or the previous pass) are free
        if (!c_f32 || wm == pass) {
#pragma unroll
            for (int j = 0; j < kWaveFragsN; ++j)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int row = (c_f32 ? 0 : wm * 128) + i * 16 + lr;   // row within the pass
                    const int colb = (wn * kWaveN + j * 16 + lk * 4) * esz;  // byte within the row
                    uint8_t* dst = csm + row * rowb + ((((colb >> 4) ^ (row & 15)) << 4) | (colb & 15));
                    const v4f v = acc[j][i];
                    if (c_f32)
                        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                    else
                        *reinterpret_cast<uint2*>(dst) =
                            make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                       f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
                }
        }
        __syncthreads();
        store_rows_from_lds<false>(csm, rows_pass, chunks_row, rowb, m0 + pass * rows_pass, n0, m, n, c, c_f32, ldc,
                                   vec);
    }
}

// W4A8 GEMM on 256 x 256 tiles (gemm_w4a8_tile.h): MXFP8 activations (A,
// [m, k] bytes) times MXFP4 weights (B, [n, k/2]).  Epilogue as in the MX
// kernel: the accumulators go to LDS in passes of 128 (bf16) or 64 (fp32) rows
// and leave as whole-row 16-byte pieces.
template <bool LAG>
__global__ __launch_bounds__(kW8Threads, 1) void gemm_w4a8_256_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const uint8_t* __restrict__ bc,
    const uint8_t* __restrict__ bs, int64_t m, int64_t n, int64_t k, void* __restrict__ c, int c_f32,
    int64_t ldc, int tiles_m, int tiles_n) {
    __shared__ __align__(16) W8Smem sm;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kW8TileM, n0 = (int64_t)tn * kW8TileN;
    W8Src S;
    w8_src(S, ac, as, bc, bs, m0, n0, m, n, k);
    v4f acc[kW8FragsN][kW8FragsM];
#pragma unroll
    for (int j = 0; j < kW8FragsN; ++j)
#pragma unroll
        for (int i = 0; i < kW8FragsM; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
    w8_mainloop<LAG>(sm, S, (int)(k / kW8StepK), acc);

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lk = lane >> 4;
    const int esz = c_f32 ? 4 : 2;
    const int rowb = kW8TileN * esz;
    const int rows_pass = c_f32 ? 64 : 128;
    static_assert(128 * kW8TileN * 2 <= (int)sizeof(W8Smem), "C staging exceeds the tile's LDS");
    const int chunks_row = rowb / 16;
    const bool vec = ((ldc * esz) & 15) == 0;
    uint8_t* csm = reinterpret_cast<uint8_t*>(&sm);
    for (int pass = 0; pass < kW8TileM / rows_pass; ++pass) {
        __syncthreads();
        if ((wm * 64) / rows_pass == pass) {
#pragma unroll
            for (int j = 0; j < kW8FragsN; ++j)
#pragma unroll
                for (int i = 0; i < kW8FragsM; ++i) {
                    const int row = wm * 64 - pass * rows_pass + i * 16 + lr;
                    const int colb = (wn * 128 + j * 16 + lk * 4) * esz;
                    uint8_t* dst = csm + row * rowb + ((((colb >> 4) ^ (row & 15)) << 4) | (colb & 15));
                    const v4f v = acc[j][i];
                    if (c_f32)
                        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
                    else
                        *reinterpret_cast<uint2*>(dst) =
                            make_uint2(f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16),
                                       f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16));
                }
        }
        __syncthreads();
        store_rows_from_lds<true>(csm, rows_pass, chunks_row, rowb, m0 + pass * rows_pass, n0, m, n, c, c_f32, ldc,
                                  vec);
    }
}

// NV GEMM on the wide 128 x 512 tiles (gemm_nv_wide.h): B expanded to fp16 in
// registers, A expanded into LDS one step ahead, fp16 MFMA, tensor scales in
// the epilogue; C goes through LDS and leaves in whole-row 16-byte pieces.
__global__ __launch_bounds__(kNvThreads, 1) void gemm_nv_tile_kernel(
    const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as, const float* __restrict__ ats,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, const float* __restrict__ bts, int64_t m,
    int64_t n, int64_t k, void* __restrict__ c, int c_f32, int64_t ldc, int tiles_m, int tiles_n) {
    __shared__ __align__(16) NwSmem sm;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * kNwM, n0 = (int64_t)tn * kNwN;
    const uint32_t kb = (uint32_t)(k / 2), kg = (uint32_t)(k / 16);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    NwSrc S{};
    S.ac = ac;
    S.as = as;
    S.b = bc;
    S.s = bs;
    S.acoff = (uint32_t)min(m0 + nw_ac_row(), m - 1) * kb + nw_ac_chunk();
    S.asoff = (uint32_t)min(m0 + nw_as_row(), m - 1) * kg + nw_s_col();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int brow = nw_b_row(q);
        S.boff[q] = (uint32_t)min(n0 + brow, n - 1) * kb + nw_b_chunk(brow);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) S.soff[j] = (uint32_t)min(n0 + nw_s_row(j), n - 1) * kg + nw_s_col();
    v4f acc[kNwMf][4];
#pragma unroll
    for (int mf = 0; mf < kNwMf; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = v4f{0.f, 0.f, 0.f, 0.f};
    nw_mainloop_rows(sm, S, (int)(k / kNwK), acc, m - m0);

    // Epilogue through LDS in four passes of 32 rows (unrolled, so each pass
    // reads only its own accumulator fragments): the pass's accumulators are
    // written in the output layout, then its rows leave as whole-row 16-byte
    // pieces.
    const float scale = __fmul_rn(*ats, *bts);
    const int esz = c_f32 ? 4 : 2;
    const int rowb = kNwN * esz + 16;                // padded LDS row pitch (bytes)
    constexpr int kRowsPass = 32;
    static_assert(kRowsPass * (kNwN * 4 + 16) <= (int)sizeof(sm), "C staging exceeds the tile's LDS");
    const int chunks_row = kNwN * esz / 16;
    const bool vec = ((ldc * esz) & 15) == 0;
    uint8_t* csm = reinterpret_cast<uint8_t*>(&sm);
#pragma unroll
    for (int pass = 0; pass < kNwM / kRowsPass; ++pass) {
        __syncthreads();                             // the stages (or the previous pass) are free
#pragma unroll
        for (int mf = pass * (kRowsPass / 16); mf < (pass + 1) * (kRowsPass / 16); ++mf)
#pragma unroll
            for (int nf = 0; nf < 4; ++nf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = mf * 16 + lq * 4 + r - pass * kRowsPass, col = wave * 64 + nf * 16 + lr;
                    const float v = __fmul_rn(acc[mf][nf][r], scale);
                    if (c_f32)
                        *reinterpret_cast<float*>(csm + row * rowb + col * 4) = v;
                    else
                        *reinterpret_cast<uint16_t*>(csm + row * rowb + col * 2) = (uint16_t)f32_to_bf16_rne(v);
                }
        __syncthreads();
        for (int q = threadIdx.x; q < kRowsPass * chunks_row; q += kNvThreads) {
            const int row = q / chunks_row, ch = q - row * chunks_row;
            const int64_t grow = m0 + pass * kRowsPass + row, gcol = n0 + ch * (16 / esz);
            if (grow >= m || gcol >= n) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(csm + row * rowb + ch * 16);
            uint8_t* dst = static_cast<uint8_t*>(c) + (grow * ldc + gcol) * esz;
            if (vec && gcol + 16 / esz <= n) {
                store_piece<true>(dst, v);
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
                for (int e = 0; e < 16 / esz && gcol + e < n; ++e) {
                    if (c_f32)
                        reinterpret_cast<uint32_t*>(dst)[e] = w[e];
                    else
                        reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
                }
            }
        }
    }
}
}  // namespace

hipError_t launch_gemm_mx(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s) {
    const int64_t tiles_m = (m + kTileM - 1) / kTileM, tiles_n = (n + kTileN - 1) / kTileN;
    const bool small_ops = m * (k / 2) < (1ll << 31) && n * (k / 2) < (1ll << 31);
    if (m <= 64 && n >= kSkinnyMinN && k % 128 == 0 && k > 0 && (n + 63) / 64 < (1ll << 31)) {
        constexpr int KF = kSkinnyKF;
        const unsigned grid = (unsigned)((n + 64 * KF - 1) / (64 * KF));
        switch ((int)((m + 15) / 16)) {
#define SKINNY(NQ) \
    case NQ: gemm_mx_skinny_kernel<NQ, KF><<<grid, 256, 0, s>>>(ac, as, bc, bs, m, n, k, c, c_f32, ldc); break;
            SKINNY(1) SKINNY(2) SKINNY(3) SKINNY(4)
#undef SKINNY
        }
    } else if (k % 512 == 0 && k > 0 && small_ops && tiles_m * tiles_n >= 64 && tiles_m * tiles_n < (1ll << 31)) {
        gemm_mx_256_kernel<<<(unsigned)(tiles_m * tiles_n), kTileThreads, 0, s>>>(ac, as, bc, bs, m, n, k, c, c_f32, ldc,
                                                                         (int)tiles_m, (int)tiles_n);
    } else {
        dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
        gemm_kernel<FP4_FMT_MX><<<grid, kThreads, 0, s>>>(ac, as, nullptr, bc, bs, nullptr, m, n, k, c, c_f32, ldc);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w4a8(const uint8_t* ac, const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                            int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc, hipStream_t s) {
    const int64_t tiles_m = (m + kW8TileM - 1) / kW8TileM, tiles_n = (n + kW8TileN - 1) / kW8TileN;
    const bool small_ops = m * k < (1ll << 31) && n * (k / 2) < (1ll << 31);
    if (k % 512 == 0 && k > 0 && small_ops && tiles_m * tiles_n >= 64 && tiles_m * tiles_n < (1ll << 31)) {
        gemm_w4a8_256_kernel<kW8Lag><<<(unsigned)(tiles_m * tiles_n), kW8Threads, 0, s>>>(
            ac, as, bc, bs, m, n, k, c, c_f32, ldc, (int)tiles_m, (int)tiles_n);
    } else {
        dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
        gemm_kernel<kFmtW4A8><<<grid, kThreads, 0, s>>>(ac, as, nullptr, bc, bs, nullptr, m, n, k, c, c_f32, ldc);
    }
    return hipGetLastError();
}

hipError_t launch_gemm_nv(const uint8_t* ac, const uint8_t* as, const float* ats,
                          const uint8_t* bc, const uint8_t* bs, const float* bts,
                          int64_t m, int64_t n, int64_t k, void* c, int c_f32, int64_t ldc,
                          hipStream_t s) {
    const int64_t tiles_m = (m + kNwM - 1) / kNwM, tiles_n = (n + kNwN - 1) / kNwN;
    const bool small_ops = m * (k / 2) < (1ll << 31) && n * (k / 2) < (1ll << 31);
    if (k % kNwK == 0 && k > 0 && small_ops && tiles_m * tiles_n >= 16 && tiles_m * tiles_n < (1ll << 31)) {
        gemm_nv_tile_kernel<<<(unsigned)(tiles_m * tiles_n), kNvThreads, 0, s>>>(
            ac, as, ats, bc, bs, bts, m, n, k, c, c_f32, ldc, (int)tiles_m, (int)tiles_n);
    } else {
        dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
        gemm_kernel<FP4_FMT_NV><<<grid, kThreads, 0, s>>>(ac, as, ats, bc, bs, bts, m, n, k, c, c_f32, ldc);
    }
    return hipGetLastError();
}

}  // namespace fp4
