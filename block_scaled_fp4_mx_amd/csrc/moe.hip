// Routed-expert MoE layer on block-scaled FP4 for gfx950.
//
// Pipeline (all on one stream, no host synchronization):
//   1. quantize X per token row (MX, or NV with the calibrated activation s_t);
//   2. routing metadata on the device: per-block expert histograms, one scan
//      block (offsets, per-block bases, row-tile list) and a stable placement
//      of every slot s = t*topk + j into its expert's segment (perm / slot_pos);
//      batches of at most 512 slots do all of it in one workgroup;
//   3. grouped gate/up GEMM over row tiles of each expert's segment, gathering
//      the quantized X rows through perm; each wave holds g and u for the same
//      (row, column) positions, so the epilogue forms h = SiLU(g) * u in
//      registers, rounds it to bf16 and quantizes it (MX or NV) straight from LDS;
//   4. grouped down GEMM on the quantized h rows (NV decode batches: their
//      exact fp16 expansion, written by the gate/up epilogue; NV prefill and
//      MX: the codes and scales), whose epilogue multiplies by the routing
//      weight and writes the fp32 row of the slot into a [slots, hidden] buffer;
//   5. combine: each token's topk rows summed in fp32 in slot order, then
//      rounded to bf16 (no atomics, so the output is deterministic).
// The steps follow the expert path of the routed experts' w1/w3/w2 projections
// ("DeepSeek-V4.1-Flash-NVFP4" explainer, section 3) and the dispatch /
// combine of tokens to experts ("DeepSeek-V4" article, section 6.1).
#include "gemm_mx_tile.h"
#include "gemm_nv_tile.h"
#include "gemm_nv_wide.h"
#include "mma_core.h"
#include "quant_device.h"

namespace fp4 {
namespace {

constexpr int kRouteSlots = 512;    // slots per routing block (bit masks of 16 words per expert)
constexpr int kMaxExperts = 1024;
constexpr int kBM = 128;            // routed rows per fallback grouped-GEMM tile
constexpr int kMinTileRows = 32;    // smallest row tile of any path
constexpr int kNvDecodeTokens = 128;  // NV batches up to this many tokens use the decode tiles
constexpr int kGuCols = 64;         // intermediate columns (of g and of u) per gate/up tile
constexpr int kDnCols = 128;        // hidden columns per down tile
constexpr int kThreads = 256;
constexpr int kScanBatch = 16;     // routing blocks read together by the scan

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Layout {
    size_t xc, xs, counts, offsets, blockbase, perm, slot_pos, tile_e, tile_r, ntiles, hc, hs, ybuf, x16, h16, total;
    bool x16_h16;                      // the fp16 expansions are allocated
    int64_t nblk, max_tiles;
};

Layout layout(int fmt, int64_t T, int64_t H, int topk, int E, int64_t I) {
    Layout L{};
    const int64_t S = T * topk;
    const int blk = fmt == FP4_FMT_MX ? 32 : 16;
    L.nblk = (S + kRouteSlots - 1) / kRouteSlots;
    // row tiles are 32 or 64 (NV tiles), 128 (fallback) or 256 (MX tiles) routed
    // rows: at most ceil(S / 32) + one partial tile per expert
    L.max_tiles = (S + kMinTileRows - 1) / kMinTileRows + (E < S ? E : S);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += a256(bytes); return at; };
    L.xc = take((size_t)T * H / 2);
    L.xs = take((size_t)T * H / blk);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.blockbase = take((size_t)L.nblk * E * 4);
    L.perm = take((size_t)S * 4);
    L.slot_pos = take((size_t)S * 4);
    L.tile_e = take((size_t)L.max_tiles * 4);
    L.tile_r = take((size_t)L.max_tiles * 4);
    L.ntiles = take(4);
    L.hc = take((size_t)S * I / 2);
    L.hs = take((size_t)S * I / blk);
    L.ybuf = take((size_t)S * H * 4);
    L.x16_h16 = fmt == FP4_FMT_NV && T <= kNvDecodeTokens;
    if (L.x16_h16) {                   // fp16 expansions of Q(x) and Q(h) for the decode NV tiles
        L.x16 = take((size_t)T * H * 2);
        L.h16 = take((size_t)S * I * 2);
    }
    L.total = o;
    return L;
}

// ------------------------------------------------------------------ routing
// Per block of kRouteSlots slots: expert histogram in LDS -> blockcount[b][e].
__global__ __launch_bounds__(kRouteSlots) void route_count_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                                  int32_t* __restrict__ blockcount) {
    __shared__ int32_t cnt[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += kRouteSlots) cnt[e] = 0;
    __syncthreads();
    const int64_t s = (int64_t)blockIdx.x * kRouteSlots + threadIdx.x;
    if (s < S) {
        const int e = ids[s];
        if ((unsigned)e < (unsigned)E) atomicAdd(&cnt[e], 1);   // other ids route nowhere
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kRouteSlots) blockcount[(int64_t)blockIdx.x * E + e] = cnt[e];
}

// Exclusive scan of a pair of ints over a 1024-thread block.
__device__ void block_scan2(int& a, int& b, int* sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int ia = a, ib = b;
    for (int off = 1; off < 64; off <<= 1) {
        const int ta = __shfl_up(ia, off), tb = __shfl_up(ib, off);
        if (lane >= off) { ia += ta; ib += tb; }
    }
    if (lane == 63) { sh[wave] = ia; sh[16 + wave] = ib; }
    __syncthreads();
    if (threadIdx.x == 0) {
        int ra = 0, rb = 0;
        for (int w = 0; w < 16; ++w) {
            const int xa = sh[w], xb = sh[16 + w];
            sh[w] = ra; sh[16 + w] = rb;
            ra += xa; rb += xb;
        }
        sh[32] = ra; sh[33] = rb;
    }
    __syncthreads();
    a = ia - a + sh[wave];
    b = ib - b + sh[16 + wave];
}

// One block: totals per expert, exclusive offsets, per-block bases (in place of
// the block counts) and the list of row tiles (expert, first row).
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ blockcount, int64_t nblk, int E,
                                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_r,
                                                          int32_t* __restrict__ ntiles, int tile_rows) {
    __shared__ int sh[40];
    constexpr int EPT = kMaxExperts / 1024;       // experts per thread (1)
    int tot[EPT];
    int rows = 0, tiles = 0;
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = threadIdx.x * EPT + q;
        int t = 0;
        if (e < E) {
            // batches of independent loads: the loop is bound by load latency
            int64_t b = 0;
            for (; b + kScanBatch <= nblk; b += kScanBatch) {
                int v[kScanBatch];
#pragma unroll
                for (int u = 0; u < kScanBatch; ++u) v[u] = blockcount[(b + u) * E + e];
#pragma unroll
                for (int u = 0; u < kScanBatch; ++u) t += v[u];
            }
            for (; b < nblk; ++b) t += blockcount[b * E + e];
        }
        tot[q] = t;
        rows += t;
        tiles += (t + tile_rows - 1) / tile_rows;
        if (e < E) counts[e] = t;
    }
    int prow = rows, ptile = tiles;
    block_scan2(prow, ptile, sh);
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = threadIdx.x * EPT + q;
        if (e >= E) break;
        offsets[e] = prow;
        int base = prow;
        int64_t b = 0;
        for (; b + kScanBatch <= nblk; b += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) v[u] = blockcount[(b + u) * E + e];
#pragma unroll
            for (int u = 0; u < kScanBatch; ++u) {
                blockcount[(b + u) * E + e] = base;
                base += v[u];
            }
        }
        for (; b < nblk; ++b) {
            const int c = blockcount[b * E + e];
            blockcount[b * E + e] = base;
            base += c;
        }
        const int nt = (tot[q] + tile_rows - 1) / tile_rows;
        for (int i = 0; i < nt; ++i) {
            tile_e[ptile + i] = e;
            tile_r[ptile + i] = prow + i * tile_rows;
        }
        ptile += nt;
        prow += tot[q];
    }
    if (threadIdx.x == 0) {
        offsets[E] = sh[32];
        *ntiles = sh[33];
    }
}

// Batches of at most kRouteSlots slots: counts, offsets, the row-tile list and
// the stable placement in one workgroup (the same results as the three
// kernels with a single routing block; one launch instead of three).
__global__ __launch_bounds__(1024) void route_small_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                           int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tile_e, int32_t* __restrict__ tile_r,
                                                           int32_t* __restrict__ ntiles, int tile_rows,
                                                           int32_t* __restrict__ perm, int32_t* __restrict__ slot_pos) {
    constexpr int kWords = kRouteSlots / 32;
    extern __shared__ uint32_t lds[];                // mask [E][kWords], then count / base [E]
    uint32_t* mask = lds;
    int32_t* base = reinterpret_cast<int32_t*>(lds + E * kWords);
    __shared__ int sh[40];
    for (int i = threadIdx.x; i < E * kWords; i += 1024) mask[i] = 0u;
    for (int i = threadIdx.x; i < E; i += 1024) base[i] = 0;
    __syncthreads();
    const int s = (int)threadIdx.x;
    int e = -1;
    if (s < S) {
        e = ids[s];
        if ((unsigned)e < (unsigned)E) {
            atomicOr(&mask[e * kWords + (s >> 5)], 1u << (s & 31));
            atomicAdd(&base[e], 1);
        } else {
            e = -1;                                  // routes nowhere
        }
    }
    __syncthreads();
    const int t = (int)threadIdx.x;                  // expert t (E <= 1024)
    const int c = t < E ? base[t] : 0;
    const int ntl = (c + tile_rows - 1) / tile_rows;
    int prow = c, ptile = ntl;
    block_scan2(prow, ptile, sh);                    // exclusive; totals in sh[32], sh[33]
    if (t < E) {
        counts[t] = c;
        offsets[t] = prow;
        base[t] = prow;                              // only thread t reads and writes entry t
        for (int i = 0; i < ntl; ++i) {
            tile_e[ptile + i] = t;
            tile_r[ptile + i] = prow + i * tile_rows;
        }
    }
    if (t == 0) {
        offsets[E] = sh[32];
        *ntiles = sh[33];
    }
    __syncthreads();
    if (e >= 0) {
        const int w = s >> 5, bit = s & 31;
        int rank = __popc(mask[e * kWords + w] & ((1u << bit) - 1u));
        for (int ww = 0; ww < w; ++ww) rank += __popc(mask[e * kWords + ww]);
        const int pos = base[e] + rank;
        perm[pos] = s;
        slot_pos[s] = pos;
    }
}

// Stable placement: the rank of slot s among the earlier slots of its block with
// the same expert comes from a per-expert bit mask of the block's slots.
__global__ __launch_bounds__(kRouteSlots) void route_place_kernel(const int32_t* __restrict__ ids, int64_t S, int E,
                                                                  const int32_t* __restrict__ blockbase,
                                                                  int32_t* __restrict__ perm,
                                                                  int32_t* __restrict__ slot_pos) {
    constexpr int kWords = kRouteSlots / 32;
    extern __shared__ uint32_t mask[];               // [E][kWords]
    for (int i = threadIdx.x; i < E * kWords; i += kRouteSlots) mask[i] = 0u;
    __syncthreads();
    const int64_t s = (int64_t)blockIdx.x * kRouteSlots + threadIdx.x;
    const int w = threadIdx.x >> 5, bit = threadIdx.x & 31;
    int e = -1;
    if (s < S) {
        e = ids[s];
        if ((unsigned)e < (unsigned)E) atomicOr(&mask[e * kWords + w], 1u << bit);
        else e = -1;
    }
    __syncthreads();
    if (e >= 0) {
        int rank = __popc(mask[e * kWords + w] & ((1u << bit) - 1u));
        for (int ww = 0; ww < w; ++ww) rank += __popc(mask[e * kWords + ww]);
        const int pos = blockbase[(int64_t)blockIdx.x * E + e] + rank;
        perm[pos] = (int32_t)s;
        slot_pos[s] = pos;
    }
}

// ------------------------------------------------------------------ grouped GEMMs
struct GemmParams {
    int fmt;
    int64_t H, I;
    int topk;
    const uint8_t *xc, *xs;            // quantized X [T, H/2], [T, H/blk]
    const uint8_t *w13c, *w13s, *w2c, *w2s;
    const float *w13ts, *w2ts, *act_ts;
    const int32_t *perm, *offsets, *tile_e, *tile_r, *ntiles;
    const float* weights;              // [S]
    uint8_t *hc, *hs;                  // quantized h [S, I/2], [S, I/blk] in routed order (MX; NV wide tiles)
    float* ybuf;                       // [S, H]: w * y of slot s in row s
    const uint16_t* x16;               // NV decode tiles: fp16 code * s_g of Q(x) [T, H]
    uint16_t* h16;                     // NV decode tiles: fp16 code * s_g of Q(h) [S, I], written by gate/up
    int h16_by_slot;                   // NV decode tiles: h16 rows are slots (injected Q(h)), else routed positions
    fp4_moe_debug dbg;
};

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// w * y of one routed row's 4 columns into the fp32 y buffer.  Non-temporal:
// the rows are read once, by the combine, after the whole down stage.
__device__ __forceinline__ void store_y(float* dst, float wgt, float4 v) {
    __builtin_nontemporal_store(f32x4_t{__fmul_rn(wgt, v.x), __fmul_rn(wgt, v.y), __fmul_rn(wgt, v.z),
                                        __fmul_rn(wgt, v.w)},
                                reinterpret_cast<f32x4_t*>(dst));
}

__device__ __forceinline__ float silu_mul(float g, float u) {
    return (g / (1.0f + expf(-g))) * u;
}

// Routing of the rows a down tile stores: a lane loads the slot and routing
// weight of one routed position (nothing past the segment), ahead of the K
// loop, so that the epilogue takes them from a register (v_readlane) instead
// of two dependent loads per stored row.
struct RowRoute {
    int32_t slot = 0;
    float wgt = 0.f;
    __device__ __forceinline__ void load(const GemmParams& p, int64_t pos, int64_t rend, bool active) {
        if (active && pos < rend) {
            slot = p.perm[pos];
            wgt = p.weights[slot];
        }
    }
    __device__ __forceinline__ int64_t slot_of(int src) const { return __builtin_amdgcn_readlane(slot, src); }
    __device__ __forceinline__ float wgt_of(int src) const {
        return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), src));
    }
};

template <int FMT>
__global__ __launch_bounds__(kThreads) void moe_gate_up_kernel(GemmParams p) {
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t c0 = (int64_t)blockIdx.x * kGuCols;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lk = lane >> 4;
    const int blk = FMT == FP4_FMT_MX ? 32 : 16;
    const int64_t H = p.H, I = p.I;

    const uint8_t* a_rows[4];
    const uint8_t* a_srow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t pos = r0 + wm * 64 + i * 16 + lr;
        if (pos < rend) {
            const int64_t t = p.perm[pos] / p.topk;
            a_rows[i] = p.xc + t * (H / 2);
            a_srow[i] = p.xs + t * (H / blk);
        } else {
            a_rows[i] = nullptr;
            a_srow[i] = nullptr;
        }
    }
    const uint8_t* wc = p.w13c + (int64_t)e * (2 * I) * (H / 2);
    const uint8_t* ws = p.w13s + (int64_t)e * (2 * I) * (H / blk);
    const uint8_t* b_rows[4];
    const uint8_t* b_srow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t col = c0 + wn * 32 + (j & 1) * 16 + lr;          // j 0,1: gate; 2,3: up
        const int64_t brow = (j < 2 ? 0 : I) + col;
        b_rows[j] = wc + brow * (H / 2);
        b_srow[j] = ws + brow * (H / blk);
    }
    v4f acc[4][4];
    zero_acc(acc);
    const bool injected = p.dbg.gate_up_in != nullptr;
    if (injected) {
        // g|u given per slot (already scaled): place them in the accumulator layout
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t pos = r0 + wm * 64 + i * 16 + lk * 4 + r;
                if (pos >= rend) continue;
                const float* src = p.dbg.gate_up_in + (int64_t)p.perm[pos] * 2 * I;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = c0 + wn * 32 + (j & 1) * 16 + lr;
                    acc[i][j][r] = src[(j < 2 ? 0 : I) + col];
                }
            }
    } else if (FMT == FP4_FMT_MX) {
        mma_mx_64x64(acc, a_rows, a_srow, b_rows, b_srow, H, lane);
    } else {
        mma_nv_64x64(acc, a_rows, a_srow, b_rows, b_srow, H, lane);
    }

    const float gscale = (FMT == FP4_FMT_NV && !injected) ? __fmul_rn(p.act_ts[0], p.w13ts[e]) : 1.0f;
    __shared__ __align__(16) uint16_t hs[kBM * kGuCols];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = wm * 64 + i * 16 + lk * 4 + r;
                const int cl = wn * 32 + j * 16 + lr;
                float g = acc[i][j][r], u = acc[i][j + 2][r];
                if (FMT == FP4_FMT_NV && !injected) {
                    g = __fmul_rn(g, gscale);
                    u = __fmul_rn(u, gscale);
                }
                const uint32_t hb = f32_to_bf16_rne(silu_mul(g, u));
                hs[rl * kGuCols + cl] = (uint16_t)hb;
                const int64_t pos = r0 + rl;
                if (pos < rend && (p.dbg.gate_up || p.dbg.h_bf16)) {
                    const int64_t slot = p.perm[pos];
                    if (p.dbg.gate_up) {
                        p.dbg.gate_up[slot * 2 * I + c0 + cl] = g;
                        p.dbg.gate_up[slot * 2 * I + I + c0 + cl] = u;
                    }
                    if (p.dbg.h_bf16) static_cast<uint16_t*>(p.dbg.h_bf16)[slot * I + c0 + cl] = (uint16_t)hb;
                }
            }
    __syncthreads();
    // quantize the 128 x 64 bf16 tile: unit = 8 consecutive columns of one row
    const double st_h = FMT == FP4_FMT_NV ? (double)p.act_ts[1] : 0.0;
#pragma unroll
    for (int q = 0; q < (kBM * kGuCols / 8) / kThreads; ++q) {
        const int unit = threadIdx.x + q * kThreads;
        const int rl = unit / (kGuCols / 8), cu = unit % (kGuCols / 8);
        const uint4 v = *reinterpret_cast<const uint4*>(&hs[rl * kGuCols + cu * 8]);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t sb;
        const uint32_t packed = FMT == FP4_FMT_MX ? mx_quant8(w, sb) : nv_quant8(w, st_h, sb);
        const int64_t pos = r0 + rl;
        if (pos < rend) {
            const int64_t col = c0 + cu * 8;
            reinterpret_cast<uint32_t*>(p.hc + pos * (I / 2) + col / 2)[0] = packed;
            const bool lead = (cu % (blk / 8)) == 0;
            if (lead) p.hs[pos * (I / blk) + col / blk] = (uint8_t)sb;
            if (p.dbg.h_codes || p.dbg.h_scales) {
                const int64_t slot = p.perm[pos];
                if (p.dbg.h_codes) reinterpret_cast<uint32_t*>(p.dbg.h_codes + slot * (I / 2) + col / 2)[0] = packed;
                if (p.dbg.h_scales && lead) p.dbg.h_scales[slot * (I / blk) + col / blk] = (uint8_t)sb;
            }
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(kThreads) void moe_down_kernel(GemmParams p) {
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t n0 = (int64_t)blockIdx.x * kDnCols;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lr = lane & 15, lk = lane >> 4;
    const int blk = FMT == FP4_FMT_MX ? 32 : 16;
    const int64_t H = p.H, I = p.I;

    const uint8_t* a_rows[4];
    const uint8_t* a_srow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t pos = r0 + wm * 64 + i * 16 + lr;
        const bool ok = pos < rend;
        if (ok && p.dbg.h_codes_in) {            // quantized h given per slot
            const int64_t slot = p.perm[pos];
            a_rows[i] = p.dbg.h_codes_in + slot * (I / 2);
            a_srow[i] = p.dbg.h_scales_in + slot * (I / blk);
        } else {
            a_rows[i] = ok ? p.hc + pos * (I / 2) : nullptr;
            a_srow[i] = ok ? p.hs + pos * (I / blk) : nullptr;
        }
    }
    const uint8_t* wc = p.w2c + (int64_t)e * H * (I / 2);
    const uint8_t* ws = p.w2s + (int64_t)e * H * (I / blk);
    const uint8_t* b_rows[4];
    const uint8_t* b_srow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t brow = n0 + wn * 64 + j * 16 + lr;
        b_rows[j] = wc + brow * (I / 2);
        b_srow[j] = ws + brow * (I / blk);
    }
    v4f acc[4][4];
    zero_acc(acc);
    if (FMT == FP4_FMT_MX)
        mma_mx_64x64(acc, a_rows, a_srow, b_rows, b_srow, I, lane);
    else
        mma_nv_64x64(acc, a_rows, a_srow, b_rows, b_srow, I, lane);

    const float yscale = FMT == FP4_FMT_NV ? __fmul_rn(p.act_ts[1], p.w2ts[e]) : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t pos = r0 + wm * 64 + i * 16 + lk * 4 + r;
            if (pos >= rend) continue;
            const int64_t slot = p.perm[pos];
            const float wgt = p.weights[slot];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t col = n0 + wn * 64 + j * 16 + lr;
                float y = acc[i][j][r];
                if (FMT == FP4_FMT_NV) y = __fmul_rn(y, yscale);
                if (p.dbg.y) p.dbg.y[slot * H + col] = y;
                p.ybuf[slot * H + col] = __fmul_rn(wgt, y);
            }
        }
}

// ------------------------------------------------------------------ MX grouped GEMMs on LDS-staged tiles
// 256 routed rows x 256 slab rows per workgroup on the MX tile of
// gemm_mx_tile.h (K a multiple of 512).  A wave (wm, wn) owns routed rows
// wm*128 .. +127 and slab columns wn*64 .. +63; it computes only the 16-row
// fragments that hold rows of its expert's segment (it still moves data for
// the others).  Rows past the segment are pointed at the segment's last row.

// gate/up: slab row wn*64 + q holds w1 row c0 + wn*32 + q (q < 32) or the w3
// row of the same intermediate column (q >= 32), so fragments j = 0, 1 of a
// wave carry g and fragments j = 2, 3 the matching u.  The tile covers 128
// intermediate columns; h (bf16) goes through LDS and is quantized there.
constexpr int kGu2Cols = 128;
constexpr int kYRow = kTileN + 4;   // fp32 row pitch of the down tile's combine buffer (bank spread)
static_assert(128 * kYRow * 4 <= (int)sizeof(MxSmem), "combine buffer exceeds the tile's LDS");

__device__ __forceinline__ int64_t gu_weight_row(int slab_row, int64_t c0, int64_t I) {
    const int wn = slab_row >> 6, q = slab_row & 63;
    return (q >= 32 ? I : 0) + c0 + wn * 32 + (q & 31);
}

// h tile in LDS: 256 rows x 128 bf16; 16-byte unit u of row r is stored at unit
// u ^ (r & 15), so the epilogue's column-fragment stores spread over the banks.
__device__ __forceinline__ int h_unit_off(int row, int unit) { return row * kGu2Cols + ((unit ^ (row & 15)) << 3); }

__global__ __launch_bounds__(kTileThreads, 1) void moe_gate_up_mx256_kernel(GemmParams p) {
    __shared__ __align__(16) MxSmem sm;
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t c0 = (int64_t)blockIdx.x * kGu2Cols;
    const int64_t H = p.H, I = p.I;
    const uint32_t kbytes = (uint32_t)(H / 2), kblocks = (uint32_t)(H / 32);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3, lr = lane & 15, lk = lane >> 4;
    const bool injected = p.dbg.gate_up_in != nullptr;

    v4f acc[kWaveFragsN][8];
#pragma unroll
    for (int j = 0; j < kWaveFragsN; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};

    if (!injected) {
        MxSlabSrc A, B;
        A.codes = p.xc;
        A.scales = p.xs;
        B.codes = p.w13c + (int64_t)e * (2 * I) * (H / 2);
        B.scales = p.w13s + (int64_t)e * (2 * I) * (H / 32);
        const uint32_t ch = mx_chunk16();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t pos = min(r0 + mx_code_row(q), rend - 1);
            A.offs[q] = (uint32_t)(p.perm[pos] / p.topk) * kbytes + ch;
            B.offs[q] = (uint32_t)gu_weight_row(mx_code_row(q), c0, I) * kbytes + ch;
        }
        const int64_t spos = min(r0 + mx_scale_row(), rend - 1);
        A.soff = (uint32_t)(p.perm[spos] / p.topk) * kblocks;
        B.soff = (uint32_t)gu_weight_row(mx_scale_row(), c0, I) * kblocks;
        mx_tile_mainloop_rows(sm, A, B, H / 32, acc, rend - (r0 + wm * 128), rend - r0);
    } else {
        // g|u given per slot (debug injection): place them in the accumulator layout
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t pos = r0 + wm * 128 + i * 16 + lr;
            if (pos >= rend) continue;
            const float* src = p.dbg.gate_up_in + (int64_t)p.perm[pos] * 2 * I;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[j][i][r] = src[(j < 2 ? 0 : I) + c0 + wn * 32 + (j & 1) * 16 + lk * 4 + r];
        }
    }
    __syncthreads();   // every wave is done with the stages; the h tile reuses them

    uint16_t* hsm = reinterpret_cast<uint16_t*>(&sm.codes[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (r0 + wm * 128 + i * 16 >= rend) break;    // fragments past the segment (uniform): no h rows
        const int rl = wm * 128 + i * 16 + lr;
        const int64_t pos = r0 + rl;
        const bool dbg_row = pos < rend && (p.dbg.gate_up || p.dbg.h_bf16);
        const int64_t slot = dbg_row ? p.perm[pos] : 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int cl = wn * 32 + j * 16 + lk * 4;        // 4 consecutive intermediate columns
            uint32_t hb[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float g = acc[j][i][r], u = acc[j + 2][i][r];
                hb[r] = f32_to_bf16_rne(silu_mul(g, u));
                if (dbg_row && p.dbg.gate_up) {
                    p.dbg.gate_up[slot * 2 * I + c0 + cl + r] = g;
                    p.dbg.gate_up[slot * 2 * I + I + c0 + cl + r] = u;
                }
                if (dbg_row && p.dbg.h_bf16) static_cast<uint16_t*>(p.dbg.h_bf16)[slot * I + c0 + cl + r] = (uint16_t)hb[r];
            }
            *reinterpret_cast<uint2*>(&hsm[h_unit_off(rl, cl >> 3) + (cl & 7)]) =
                make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
        }
    }
    __syncthreads();
    // quantize the 256 x 128 h tile: unit = 8 consecutive columns of one row;
    // the 4 units of an MX block sit in 4 consecutive lanes
#pragma unroll
    for (int q = 0; q < (kTileM * kGu2Cols / 8) / kTileThreads; ++q) {
        const int unit = threadIdx.x + q * kTileThreads;
        const int rl = unit >> 4, cu = unit & 15;
        const int64_t pos = r0 + rl;
        if (pos >= rend) break;      // the rows of later units are further down
        const uint4 v = *reinterpret_cast<const uint4*>(&hsm[h_unit_off(rl, cu)]);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t sb;
        const uint32_t packed = mx_quant8(w, sb);
        {
            const int64_t col = c0 + cu * 8;
            reinterpret_cast<uint32_t*>(p.hc + pos * (I / 2) + col / 2)[0] = packed;
            const bool lead = (cu & 3) == 0;
            if (lead) p.hs[pos * (I / 32) + col / 32] = (uint8_t)sb;
            if (p.dbg.h_codes || p.dbg.h_scales) {
                const int64_t slot = p.perm[pos];
                if (p.dbg.h_codes) reinterpret_cast<uint32_t*>(p.dbg.h_codes + slot * (I / 2) + col / 2)[0] = packed;
                if (p.dbg.h_scales && lead) p.dbg.h_scales[slot * (I / 32) + col / 32] = (uint8_t)sb;
            }
        }
    }
}

// down: routed h rows (or, injected, each slot's given quantized h) times the
// 256 w2 rows n0 .. n0 + 255; y times the routing weight is added into the
// fp32 [tokens, hidden] buffer.
__global__ __launch_bounds__(kTileThreads, 1) void moe_down_mx256_kernel(GemmParams p) {
    __shared__ __align__(16) MxSmem sm;
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t n0 = (int64_t)blockIdx.x * kTileN;
    const int64_t H = p.H, I = p.I;
    const uint32_t kbytes = (uint32_t)(I / 2), kblocks = (uint32_t)(I / 32);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3, lr = lane & 15, lk = lane >> 4;

    MxSlabSrc A, B;
    const bool inj = p.dbg.h_codes_in != nullptr;
    A.codes = inj ? p.dbg.h_codes_in : p.hc;
    A.scales = inj ? p.dbg.h_scales_in : p.hs;
    const uint32_t ch = mx_chunk16();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t pos = min(r0 + mx_code_row(q), rend - 1);
        A.offs[q] = (uint32_t)(inj ? p.perm[pos] : pos) * kbytes + ch;
    }
    const int64_t spos = min(r0 + mx_scale_row(), rend - 1);
    A.soff = (uint32_t)(inj ? p.perm[spos] : spos) * kblocks;
    mx_slab_src(B, p.w2c + (int64_t)e * H * (I / 2), p.w2s + (int64_t)e * H * (I / 32), n0, H, I / 2, I / 32);

    // lane L < 32 routes row wave + 8 (L % 16) of band L / 16 (the rows the wave stores)
    RowRoute route;
    route.load(p, r0 + (lane >> 4 & 1) * 128 + wave + 8 * (lane & 15), rend, lane < 32);
    v4f acc[kWaveFragsN][8];
#pragma unroll
    for (int j = 0; j < kWaveFragsN; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = v4f{0.f, 0.f, 0.f, 0.f};
    mx_tile_mainloop_rows(sm, A, B, I / 32, acc, rend - (r0 + wm * 128), rend - r0);

    if (p.dbg.y) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t pos = r0 + wm * 128 + i * 16 + lr;
            if (pos >= rend) continue;
            const int64_t slot = p.perm[pos];
#pragma unroll
            for (int j = 0; j < kWaveFragsN; ++j)
                *reinterpret_cast<float4*>(&p.dbg.y[slot * H + n0 + wn * kWaveN + j * 16 + lk * 4]) =
                    make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
        }
    }
    // w * y of each routed row goes to its slot's row of the y buffer; the tile
    // passes through LDS one 128-row band at a time so that each store
    // instruction writes 1 KiB of one row.
    float* ysm = reinterpret_cast<float*>(&sm);
    for (int band = 0; band < 2; ++band) {
        __syncthreads();
        if (wm == band) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < kWaveFragsN; ++j)
                    *reinterpret_cast<float4*>(&ysm[(i * 16 + lr) * kYRow + wn * kWaveN + j * 16 + lk * 4]) =
                        make_float4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
        }
        __syncthreads();
        for (int k = 0; k < 128 / (kTileThreads / 64); ++k) {
            const int rr = wave + k * (kTileThreads / 64);
            const int64_t pos = r0 + band * 128 + rr;
            if (pos >= rend) break;     // rows are in order: the rest of this wave's rows are past the end too
            const int64_t slot = route.slot_of(band * 16 + k);
            const float wgt = route.wgt_of(band * 16 + k);
            const float4 v = *reinterpret_cast<const float4*>(&ysm[rr * kYRow + lane * 4]);
            store_y(p.ybuf + slot * H + n0 + lane * 4, wgt, v);
        }
    }
}

// ------------------------------------------------------------------ NV grouped GEMMs on LDS-staged tiles
// 64 routed rows x 256 weight rows per workgroup on the NV tile of
// gemm_nv_tile.h (hidden and intermediate multiples of 256).  A is the fp16
// expansion (code * s_g) of the quantized activations; each wave computes only
// the 16-row fragments that hold rows of its expert's segment.

// Rows of one NV operand -> exact fp16 values code * s_g (the tensor scale is
// left to the GEMM epilogue).  Lane per 16-group.
__global__ __launch_bounds__(kThreads) void expand_nv16_kernel(const uint8_t* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales, int64_t rows,
                                                               int64_t k, uint16_t* __restrict__ out) {
    const int64_t gpr = k >> 4, total = rows * gpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += stride) {
        const uint2 c = *reinterpret_cast<const uint2*>(codes + u * 8);
        const _Float16 sg = nv_scale_pair(scales[u])[0];
        const h8_t a = nv_expand8(c.x, sg), b = nv_expand8(c.y, sg);
        uint4* o = reinterpret_cast<uint4*>(out + u * 16);
        o[0] = __builtin_bit_cast(uint4, a);
        o[1] = __builtin_bit_cast(uint4, b);
    }
}

// gate/up: wave w owns slab rows w*32 .. +31: 16 w1 rows (intermediate columns
// c0 + w*16 ..) then the 16 w3 rows of the same columns, so fragment 0 holds g
// and fragment 1 the matching u.  A tile covers 128 intermediate columns.
constexpr int kNvGuCols = 128;

__device__ __forceinline__ int64_t gu_nv_row(int slab_row, int64_t c0, int64_t I) {
    const int w = slab_row >> 5, q = slab_row & 31;
    return (q >= 16 ? I : 0) + c0 + w * 16 + (q & 15);
}

template <int TM, int NS>
__global__ __launch_bounds__(kNvThreads, 1) void moe_gate_up_nv_kernel(GemmParams p) {
    __shared__ __align__(16) NvSmemT<TM, NS> sm;
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t c0 = (int64_t)blockIdx.x * kNvGuCols;
    const int64_t H = p.H, I = p.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const bool injected = p.dbg.gate_up_in != nullptr;

    v4f acc[4][2];
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) acc[mf][nf] = v4f{0.f, 0.f, 0.f, 0.f};

    if (!injected) {
        NvSrc S{};
        S.a = reinterpret_cast<const uint8_t*>(p.x16);
        S.b = p.w13c + (int64_t)e * (2 * I) * (H / 2);
        S.s = p.w13s + (int64_t)e * (2 * I) * (H / 16);
        const uint32_t apitch = (uint32_t)(H * 2), bpitch = (uint32_t)(H / 2), spitch = (uint32_t)(H / 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < TM / 16) {
                const int arow = nv_a_row<TM>(q);
                const int64_t pos = min(r0 + arow, rend - 1);
                S.aoff[q] = (uint32_t)(p.perm[pos] / p.topk) * apitch + nv_a_chunk(arow);
            }
            S.boff[q] = (uint32_t)gu_nv_row(mx_code_row(q), c0, I) * bpitch + mx_chunk16();
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) S.sdw[j] = (uint32_t)gu_nv_row(nv_sdw_row(j), c0, I) * spitch + nv_sdw_col();
        nv_tile_mainloop_rows(sm, S, (int)(H / 256), acc, rend - r0);
    } else {
        // g|u given per slot (debug injection, tensor scales included)
#pragma unroll
        for (int mf = 0; mf < TM / 16; ++mf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t pos = r0 + mf * 16 + lq * 4 + r;
                if (pos >= rend) continue;
                const float* src = p.dbg.gate_up_in + (int64_t)p.perm[pos] * 2 * I;
                acc[mf][0][r] = src[c0 + wave * 16 + lr];
                acc[mf][1][r] = src[I + c0 + wave * 16 + lr];
            }
    }
    __syncthreads();   // the h tile reuses the stages

    const float gscale = injected ? 1.0f : __fmul_rn(p.act_ts[0], p.w13ts[e]);
    uint16_t* hsm = reinterpret_cast<uint16_t*>(&sm);      // TM rows x 128 bf16
#pragma unroll
    for (int mf = 0; mf < TM / 16; ++mf)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rl = mf * 16 + lq * 4 + r;
            const int cl = wave * 16 + lr;
            const float g = injected ? acc[mf][0][r] : __fmul_rn(acc[mf][0][r], gscale);
            const float u = injected ? acc[mf][1][r] : __fmul_rn(acc[mf][1][r], gscale);
            const uint32_t hb = f32_to_bf16_rne(silu_mul(g, u));
            hsm[rl * kNvGuCols + cl] = (uint16_t)hb;
            const int64_t pos = r0 + rl;
            if (pos < rend && (p.dbg.gate_up || p.dbg.h_bf16)) {
                const int64_t slot = p.perm[pos];
                if (p.dbg.gate_up) {
                    p.dbg.gate_up[slot * 2 * I + c0 + cl] = g;
                    p.dbg.gate_up[slot * 2 * I + I + c0 + cl] = u;
                }
                if (p.dbg.h_bf16) static_cast<uint16_t*>(p.dbg.h_bf16)[slot * I + c0 + cl] = (uint16_t)hb;
            }
        }
    __syncthreads();
    // quantize the TM x 128 h tile: unit = 8 consecutive columns of one row; a
    // 16-group spans 2 consecutive lanes
    const double st_h = (double)p.act_ts[1];
#pragma unroll
    for (int q = 0; q < (TM * kNvGuCols / 8) / kNvThreads; ++q) {
        const int unit = threadIdx.x + q * kNvThreads;
        const int rl = unit / (kNvGuCols / 8), cu = unit % (kNvGuCols / 8);
        const uint4 v = *reinterpret_cast<const uint4*>(&hsm[rl * kNvGuCols + cu * 8]);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t sb;
        const uint32_t packed = nv_quant8(w, st_h, sb);
        const int64_t pos = r0 + rl;
        if (pos < rend) {
            const int64_t col = c0 + cu * 8;
            // the down tiles read Q(h) as its exact fp16 expansion
            *reinterpret_cast<h8_t*>(p.h16 + pos * I + col) = nv_expand8(packed, nv_scale_pair(sb)[0]);
            const bool lead = (cu & 1) == 0;
            if (p.dbg.h_codes || p.dbg.h_scales) {
                const int64_t slot = p.perm[pos];
                if (p.dbg.h_codes) reinterpret_cast<uint32_t*>(p.dbg.h_codes + slot * (I / 2) + col / 2)[0] = packed;
                if (p.dbg.h_scales && lead) p.dbg.h_scales[slot * (I / 16) + col / 16] = (uint8_t)sb;
            }
        }
    }
}

// down: the fp16 expansion of Q(h) for the tile's rows times w2 rows n0 .. n0 + 255.
constexpr int kNvYRow = kNvTileN + 4;   // fp32 row pitch of the combine staging tile

template <int TM, int NS>
__global__ __launch_bounds__(kNvThreads, 1) void moe_down_nv_kernel(GemmParams p) {
    __shared__ __align__(16) NvSmemT<TM, NS> sm;
    static_assert(TM * kNvYRow * 4 <= (int)sizeof(sm), "staging tile exceeds the NV tile's LDS");
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t n0 = (int64_t)blockIdx.x * kNvTileN;
    const int64_t H = p.H, I = p.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    NvSrc S{};
    S.a = reinterpret_cast<const uint8_t*>(p.h16);
    S.b = p.w2c + (int64_t)e * H * (I / 2);
    S.s = p.w2s + (int64_t)e * H * (I / 16);
    const uint32_t apitch = (uint32_t)(I * 2), bpitch = (uint32_t)(I / 2), spitch = (uint32_t)(I / 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (q < TM / 16) {
            const int arow = nv_a_row<TM>(q);
            const int64_t pos = min(r0 + arow, rend - 1);
            S.aoff[q] = (uint32_t)(p.h16_by_slot ? p.perm[pos] : pos) * apitch + nv_a_chunk(arow);
        }
        S.boff[q] = (uint32_t)min(n0 + mx_code_row(q), H - 1) * bpitch + mx_chunk16();
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) S.sdw[j] = (uint32_t)min(n0 + nv_sdw_row(j), H - 1) * spitch + nv_sdw_col();

    v4f acc[4][2];
#pragma unroll
    for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) acc[mf][nf] = v4f{0.f, 0.f, 0.f, 0.f};
    // lane L < TM / 8 routes row wave + 8 L (the rows the wave stores)
    RowRoute route;
    route.load(p, r0 + wave + 8 * lane, rend, lane < TM / 8);
    nv_tile_mainloop_rows(sm, S, (int)(I / 256), acc, rend - r0);
    __syncthreads();   // the staging tile reuses the stages

    const float yscale = __fmul_rn(p.act_ts[1], p.w2ts[e]);
    float* ysm = reinterpret_cast<float*>(&sm);
#pragma unroll
    for (int mf = 0; mf < TM / 16; ++mf)
#pragma unroll
        for (int nf = 0; nf < 2; ++nf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mf * 16 + lq * 4 + r;
                const int cl = wave * 32 + nf * 16 + lr;
                const float y = __fmul_rn(acc[mf][nf][r], yscale);
                ysm[rl * kNvYRow + cl] = y;
                const int64_t pos = r0 + rl;
                if (p.dbg.y && pos < rend) p.dbg.y[(int64_t)p.perm[pos] * H + n0 + cl] = y;
            }
    __syncthreads();
    for (int k = 0; k < TM / (kNvThreads / 64); ++k) {
        const int rr = wave + k * (kNvThreads / 64);
        const int64_t pos = r0 + rr;
        if (pos >= rend) break;     // rows are in order: the rest of this wave's rows are past the end too
        const int64_t slot = route.slot_of(k);
        const float wgt = route.wgt_of(k);
        const float4 v = *reinterpret_cast<const float4*>(&ysm[rr * kNvYRow + lane * 4]);
        store_y(p.ybuf + slot * H + n0 + lane * 4, wgt, v);
    }
}

// ---------------------------------------------------------------- wide NV tiles
// Prefill-sized batches: 128 routed rows x 512 weight rows per tile (the wide
// NV tile), both operands NVFP4 codes: gate/up gathers the rows of Q(x) of the
// tile's slots, down reads Q(h) as gate/up wrote it.  gate/up: wave w owns slab
// rows w*64 .. +63: 32 w1 rows (intermediate columns c0 + w*32 ..) then the 32
// w3 rows of the same columns, so fragments 0-1 hold g and fragments 2-3 the
// matching u.  A tile covers 256 intermediate columns.
constexpr int kNwGuCols = 256;

__device__ __forceinline__ int64_t gu_nw_row(int slab_row, int64_t c0, int64_t I) {
    const int w = slab_row >> 6, q = slab_row & 63;
    return (q >= 32 ? I : 0) + c0 + w * 32 + (q & 31);
}

__global__ __launch_bounds__(kNvThreads, 1) void moe_gate_up_nvw_kernel(GemmParams p) {
    __shared__ __align__(16) NwSmem sm;
    static_assert(kNwM * kNwGuCols * 2 <= (int)sizeof(sm), "h tile exceeds the wide tile's LDS");
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t c0 = (int64_t)blockIdx.x * kNwGuCols;
    const int64_t H = p.H, I = p.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const bool injected = p.dbg.gate_up_in != nullptr;

    v4f acc[kNwMf][4];
#pragma unroll
    for (int mf = 0; mf < kNwMf; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = v4f{0.f, 0.f, 0.f, 0.f};

    if (!injected) {
        NwSrc S{};
        S.ac = p.xc;
        S.as = p.xs;
        S.b = p.w13c + (int64_t)e * (2 * I) * (H / 2);
        S.s = p.w13s + (int64_t)e * (2 * I) * (H / 16);
        const uint32_t bpitch = (uint32_t)(H / 2), spitch = (uint32_t)(H / 16);
        // A rows: the tokens of the tile's slots (rows past the segment repeat its last)
        const int64_t ctok = p.perm[min(r0 + nw_ac_row(), rend - 1)] / p.topk;
        const int64_t stok = p.perm[min(r0 + nw_as_row(), rend - 1)] / p.topk;
        S.acoff = (uint32_t)ctok * bpitch + nw_ac_chunk();
        S.asoff = (uint32_t)stok * spitch + nw_s_col();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int brow = nw_b_row(q);
            S.boff[q] = (uint32_t)gu_nw_row(brow, c0, I) * bpitch + nw_b_chunk(brow);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) S.soff[j] = (uint32_t)gu_nw_row(nw_s_row(j), c0, I) * spitch + nw_s_col();
        nw_mainloop_rows(sm, S, (int)(H / kNwK), acc, rend - r0);
    } else {
        // g|u given per slot (debug injection, tensor scales included)
#pragma unroll
        for (int mf = 0; mf < kNwMf; ++mf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t pos = r0 + mf * 16 + lq * 4 + r;
                if (pos >= rend) continue;
                const float* src = p.dbg.gate_up_in + (int64_t)p.perm[pos] * 2 * I;
#pragma unroll
                for (int nf = 0; nf < 2; ++nf) {
                    acc[mf][nf][r] = src[c0 + wave * 32 + nf * 16 + lr];
                    acc[mf][nf + 2][r] = src[I + c0 + wave * 32 + nf * 16 + lr];
                }
            }
    }
    __syncthreads();   // the h tile reuses the stages

    const float gscale = injected ? 1.0f : __fmul_rn(p.act_ts[0], p.w13ts[e]);
    uint16_t* hsm = reinterpret_cast<uint16_t*>(&sm);      // 128 rows x 256 bf16
#pragma unroll
    for (int mf = 0; mf < kNwMf; ++mf) {
        if (r0 + mf * 16 >= rend) break;    // fragments past the segment (uniform): no h rows
#pragma unroll
        for (int nf = 0; nf < 2; ++nf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rl = mf * 16 + lq * 4 + r;
                const int cl = wave * 32 + nf * 16 + lr;
                const float g = injected ? acc[mf][nf][r] : __fmul_rn(acc[mf][nf][r], gscale);
                const float u = injected ? acc[mf][nf + 2][r] : __fmul_rn(acc[mf][nf + 2][r], gscale);
                const uint32_t hb = f32_to_bf16_rne(silu_mul(g, u));
                hsm[rl * kNwGuCols + cl] = (uint16_t)hb;
                const int64_t pos = r0 + rl;
                if (pos < rend && (p.dbg.gate_up || p.dbg.h_bf16)) {
                    const int64_t slot = p.perm[pos];
                    if (p.dbg.gate_up) {
                        p.dbg.gate_up[slot * 2 * I + c0 + cl] = g;
                        p.dbg.gate_up[slot * 2 * I + I + c0 + cl] = u;
                    }
                    if (p.dbg.h_bf16) static_cast<uint16_t*>(p.dbg.h_bf16)[slot * I + c0 + cl] = (uint16_t)hb;
                }
            }
    }
    __syncthreads();
    // quantize the 128 x 256 h tile: unit = 8 consecutive columns of one row; a
    // 16-group spans 2 consecutive lanes
    const double st_h = (double)p.act_ts[1];
#pragma unroll 2
    for (int q = 0; q < (kNwM * kNwGuCols / 8) / kNvThreads; ++q) {
        const int unit = threadIdx.x + q * kNvThreads;
        const int rl = unit / (kNwGuCols / 8), cu = unit % (kNwGuCols / 8);
        const int64_t pos = r0 + rl;
        if (pos >= rend) break;      // the rows of later units are further down
        const uint4 v = *reinterpret_cast<const uint4*>(&hsm[rl * kNwGuCols + cu * 8]);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        uint32_t sb;
        const uint32_t packed = nv_quant8(w, st_h, sb);
        const int64_t col = c0 + cu * 8;
        const bool lead = (cu & 1) == 0;
        // Q(h) in routed order, as the down tiles read it
        reinterpret_cast<uint32_t*>(p.hc + pos * (I / 2) + col / 2)[0] = packed;
        if (lead) p.hs[pos * (I / 16) + col / 16] = (uint8_t)sb;
        if (p.dbg.h_codes || p.dbg.h_scales) {
            const int64_t slot = p.perm[pos];
            if (p.dbg.h_codes) reinterpret_cast<uint32_t*>(p.dbg.h_codes + slot * (I / 2) + col / 2)[0] = packed;
            if (p.dbg.h_scales && lead) p.dbg.h_scales[slot * (I / 16) + col / 16] = (uint8_t)sb;
        }
    }
}

// down: Q(h) of the tile's rows (codes + E4M3 scales) times w2 rows
// n0 .. n0 + 511 (rows past H are clamped and their columns never stored).  The
// fp32 result leaves through LDS in two passes of 64 rows.
constexpr int kNwYRow = kNwN + 4;   // fp32 row pitch of the combine staging tile
constexpr int kNwYRows = 64;        // rows per staging pass
static_assert(kNwM == 2 * kNwYRows && kNwYRows / (kNvThreads / 64) == 8,
              "the wide down tile's row routing covers two passes of eight rows per wave");

__global__ __launch_bounds__(kNvThreads, 1) void moe_down_nvw_kernel(GemmParams p) {
    __shared__ __align__(16) NwSmem sm;
    static_assert(kNwYRows * kNwYRow * 4 <= (int)sizeof(sm), "staging tile exceeds the wide tile's LDS");
    const int tile = blockIdx.y;
    if (tile >= *p.ntiles) return;
    const int e = p.tile_e[tile];
    const int64_t r0 = p.tile_r[tile];
    const int64_t rend = p.offsets[e + 1];
    const int64_t n0 = (int64_t)blockIdx.x * kNwN;
    const int64_t H = p.H, I = p.I;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;

    // A = Q(h): gate/up's codes in routed order, or injected codes by slot
    const bool inj = p.dbg.h_codes_in != nullptr;
    NwSrc S{};
    S.ac = inj ? p.dbg.h_codes_in : p.hc;
    S.as = inj ? p.dbg.h_scales_in : p.hs;
    S.b = p.w2c + (int64_t)e * H * (I / 2);
    S.s = p.w2s + (int64_t)e * H * (I / 16);
    const uint32_t bpitch = (uint32_t)(I / 2), spitch = (uint32_t)(I / 16);
    {
        const int64_t cpos = min(r0 + nw_ac_row(), rend - 1), spos = min(r0 + nw_as_row(), rend - 1);
        S.acoff = (uint32_t)(inj ? p.perm[cpos] : cpos) * bpitch + nw_ac_chunk();
        S.asoff = (uint32_t)(inj ? p.perm[spos] : spos) * spitch + nw_s_col();
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int brow = nw_b_row(q);
        S.boff[q] = (uint32_t)min(n0 + brow, H - 1) * bpitch + nw_b_chunk(brow);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) S.soff[j] = (uint32_t)min(n0 + nw_s_row(j), H - 1) * spitch + nw_s_col();

    v4f acc[kNwMf][4];
#pragma unroll
    for (int mf = 0; mf < kNwMf; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = v4f{0.f, 0.f, 0.f, 0.f};
    // lane L < 16 routes row wave + 8 (L % 8) of staging pass L / 8 (the rows the wave stores)
    RowRoute route;
    route.load(p, r0 + (lane >> 3 & 1) * kNwYRows + wave + 8 * (lane & 7), rend, lane < 16);
    nw_mainloop_rows(sm, S, (int)(I / kNwK), acc, rend - r0);

    const float yscale = __fmul_rn(p.act_ts[1], p.w2ts[e]);
    float* ysm = reinterpret_cast<float*>(&sm);
#pragma unroll
    for (int pass = 0; pass < kNwM / kNwYRows; ++pass) {
        if (r0 + pass * kNwYRows >= rend) break;          // no rows of the problem in this pass (uniform)
        __syncthreads();   // the staging tile reuses the stages (or the previous pass)
#pragma unroll
        for (int mf = 0; mf < kNwYRows / 16; ++mf)
#pragma unroll
            for (int nf = 0; nf < 4; ++nf)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rl = mf * 16 + lq * 4 + r;
                    const int cl = wave * 64 + nf * 16 + lr;
                    const float y = __fmul_rn(acc[pass * (kNwYRows / 16) + mf][nf][r], yscale);
                    ysm[rl * kNwYRow + cl] = y;
                    const int64_t pos = r0 + pass * kNwYRows + rl;
                    if (p.dbg.y && pos < rend && n0 + cl < H) p.dbg.y[(int64_t)p.perm[pos] * H + n0 + cl] = y;
                }
        __syncthreads();
        for (int k = 0; k < kNwYRows / (kNvThreads / 64); ++k) {
            const int rr = wave + k * (kNvThreads / 64);
            const int64_t pos = r0 + pass * kNwYRows + rr;
            if (pos >= rend) break;     // rows are in order: the rest of this wave's rows are past the end too
            const int64_t slot = route.slot_of(pass * 8 + k);
            const float wgt = route.wgt_of(pass * 8 + k);
#pragma unroll
            for (int hh = 0; hh < kNwN / 256; ++hh) {
                const int col = hh * 256 + lane * 4;
                if (n0 + col >= H) break;     // H is a multiple of 4: a float4 is wholly in or out
                const float4 v = *reinterpret_cast<const float4*>(&ysm[rr * kNwYRow + col]);
                store_y(p.ybuf + slot * H + n0 + col, wgt, v);
            }
        }
    }
}

// out[t] = bf16(sum over j of w * y of slot t*topk + j), summed in fp32 in
// order j = 0 .. topk-1 over the slots whose expert id is in range.  A thread
// issues the loads of up to kCombineBatch slots at once (rows of unrouted
// slots are read but never added: a skipped slot leaves the sum as it is, a
// -0 included).
constexpr int kCombineBatch = 8;
__global__ __launch_bounds__(kThreads) void combine_kernel(const float4* __restrict__ ybuf,
                                                           const int32_t* __restrict__ ids, int topk, int E,
                                                           int64_t T, int64_t H4, uint2* __restrict__ out) {
    const int64_t n = T * H4;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
        const int64_t t = i / H4, c = i - t * H4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j0 = 0; j0 < topk; j0 += kCombineBatch) {
            float4 v[kCombineBatch];
            bool ok[kCombineBatch];
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const int j = j0 + u;
                const int64_t slot = t * topk + min(j, topk - 1);
                ok[u] = j < topk && (unsigned)ids[slot] < (unsigned)E;
                v[u] = ybuf[slot * H4 + c];
            }
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                if (ok[u]) {
                    acc.x = __fadd_rn(acc.x, v[u].x);
                    acc.y = __fadd_rn(acc.y, v[u].y);
                    acc.z = __fadd_rn(acc.z, v[u].z);
                    acc.w = __fadd_rn(acc.w, v[u].w);
                }
            }
        }
        __builtin_nontemporal_store(u32x2_t{f32_to_bf16_rne(acc.x) | (f32_to_bf16_rne(acc.y) << 16),
                                            f32_to_bf16_rne(acc.z) | (f32_to_bf16_rne(acc.w) << 16)},
                                    reinterpret_cast<u32x2_t*>(out + i));
    }
}

inline unsigned stream_grid(int64_t n) {
    int64_t b = (n + kThreads - 1) / kThreads;
    if (b > 8192) b = 8192;
    return (unsigned)(b < 1 ? 1 : b);
}
}  // namespace

int64_t moe_max_tiles(int64_t tokens, int topk, int num_experts) {
    return layout(FP4_FMT_MX, tokens, 128, topk, num_experts, 128).max_tiles;
}

size_t moe_workspace_bytes(int fmt, int64_t tokens, int64_t hidden, int topk, int num_experts, int64_t inter) {
    return layout(fmt, tokens, hidden, topk, num_experts, inter).total;
}

hipError_t launch_moe(const MoeArgs& a, hipStream_t s) {
    if (a.num_experts > kMaxExperts) return hipErrorInvalidValue;
    const Layout L = layout(a.fmt, a.tokens, a.hidden, a.topk, a.num_experts, a.inter);
    uint8_t* base = static_cast<uint8_t*>(a.ws);
    uint8_t* xc = base + L.xc;
    uint8_t* xs = base + L.xs;
    int32_t* counts = reinterpret_cast<int32_t*>(base + L.counts);
    int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
    int32_t* blockbase = reinterpret_cast<int32_t*>(base + L.blockbase);
    int32_t* perm = reinterpret_cast<int32_t*>(base + L.perm);
    int32_t* slot_pos = reinterpret_cast<int32_t*>(base + L.slot_pos);
    int32_t* tile_e = reinterpret_cast<int32_t*>(base + L.tile_e);
    int32_t* tile_r = reinterpret_cast<int32_t*>(base + L.tile_r);
    int32_t* ntiles = reinterpret_cast<int32_t*>(base + L.ntiles);
    uint8_t* hc = base + L.hc;
    uint8_t* hs = base + L.hs;
    float* ybuf = reinterpret_cast<float*>(base + L.ybuf);
    const int64_t T = a.tokens, H = a.hidden, I = a.inter, S = T * a.topk;
    const int E = a.num_experts;

    auto mark = [&](int i) {
        return a.dbg.stage_events[i] ? hipEventRecord(static_cast<hipEvent_t>(a.dbg.stage_events[i]), s) : hipSuccess;
    };
    if (hipError_t e0 = mark(0)) return e0;
    // 1. quantize X
    hipError_t err = a.fmt == FP4_FMT_MX
                         ? launch_quantize_mx(a.x, T, H, H, xc, xs, s)
                         : launch_quantize_nv(a.x, T, H, H, xc, xs, const_cast<float*>(a.act_ts), true, nullptr, s);
    if (err != hipSuccess || (err = mark(1)) != hipSuccess) return err;
    // 2. routing metadata
    // LDS-staged tiles: MX with hidden and inter multiples of 512 (256 routed
    // rows per tile), NV with multiples of 256 (32 routed rows per tile for
    // decode batches, 128 for larger ones)
    const bool tiled = a.fmt == FP4_FMT_MX && H % 512 == 0 && I % 512 == 0;
    const bool nv_tiled = a.fmt == FP4_FMT_NV && H % 256 == 0 && I % 256 == 0;
    const bool nv_decode = T <= kNvDecodeTokens;       // 32-row, three-stage NV tiles
    const int tile_rows = tiled ? kTileM : (nv_tiled ? (nv_decode ? 32 : kNwM) : kBM);
    // grid rows: at most ceil(S / tile_rows) full tiles plus one partial tile
    // per active expert (the workgroups past the actual count exit at once)
    const unsigned grid_tiles = (unsigned)((S + tile_rows - 1) / tile_rows + (E < S ? E : S));
    const size_t small_lds = (size_t)E * (kRouteSlots / 32 + 1) * 4;
    if (S <= kRouteSlots && small_lds <= 65536) {
        route_small_kernel<<<1, 1024, small_lds, s>>>(
            a.ids, S, E, counts, offsets, tile_e, tile_r, ntiles, tile_rows, perm, slot_pos);
    } else {
        route_count_kernel<<<(unsigned)L.nblk, kRouteSlots, 0, s>>>(a.ids, S, E, blockbase);
        route_scan_kernel<<<1, 1024, 0, s>>>(blockbase, L.nblk, E, counts, offsets, tile_e, tile_r, ntiles, tile_rows);
        route_place_kernel<<<(unsigned)L.nblk, kRouteSlots, (size_t)E * (kRouteSlots / 32) * 4, s>>>(
            a.ids, S, E, blockbase, perm, slot_pos);
    }
    if ((err = hipGetLastError()) != hipSuccess || (err = mark(2)) != hipSuccess) return err;

    GemmParams p{};
    p.fmt = a.fmt;
    p.H = H;
    p.I = I;
    p.topk = a.topk;
    p.xc = xc;
    p.xs = xs;
    p.w13c = a.w13c;
    p.w13s = a.w13s;
    p.w2c = a.w2c;
    p.w2s = a.w2s;
    p.w13ts = a.w13ts;
    p.w2ts = a.w2ts;
    p.act_ts = a.act_ts;
    p.perm = perm;
    p.offsets = offsets;
    p.tile_e = tile_e;
    p.tile_r = tile_r;
    p.ntiles = ntiles;
    p.weights = a.weights;
    p.hc = hc;
    p.hs = hs;
    p.ybuf = ybuf;
    p.dbg = a.dbg;
    uint16_t* x16 = L.x16_h16 ? reinterpret_cast<uint16_t*>(base + L.x16) : nullptr;
    uint16_t* h16 = L.x16_h16 ? reinterpret_cast<uint16_t*>(base + L.h16) : nullptr;
    p.x16 = x16;
    p.h16 = h16;
    p.h16_by_slot = a.dbg.h_codes_in != nullptr;
    // 3. gate/up + SiLU*mul + quantize h; 4. down + weighted combine
    if (nv_tiled && nv_decode) {
        expand_nv16_kernel<<<stream_grid(T * H / 16), kThreads, 0, s>>>(xc, xs, T, H, x16);
        moe_gate_up_nv_kernel<32, 3><<<dim3((unsigned)(I / kNvGuCols), grid_tiles), kNvThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(3)) != hipSuccess) return err;
        if (a.dbg.h_codes_in)      // injected Q(h), by slot: its expansion replaces the tiles' own
            expand_nv16_kernel<<<stream_grid(S * I / 16), kThreads, 0, s>>>(a.dbg.h_codes_in, a.dbg.h_scales_in, S, I,
                                                                             h16);
        moe_down_nv_kernel<32, 3><<<dim3((unsigned)(H / kNvTileN), grid_tiles), kNvThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(4)) != hipSuccess) return err;
    } else if (nv_tiled) {
        // wide tiles: Q(x) and Q(h) stay NVFP4 codes, expanded inside the tiles
        moe_gate_up_nvw_kernel<<<dim3((unsigned)(I / kNwGuCols), grid_tiles), kNvThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(3)) != hipSuccess) return err;
        moe_down_nvw_kernel<<<dim3((unsigned)((H + kNwN - 1) / kNwN), grid_tiles), kNvThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(4)) != hipSuccess) return err;
    } else if (tiled) {
        const dim3 g_gu((unsigned)(I / kGu2Cols), grid_tiles);
        const dim3 g_dn((unsigned)(H / kTileN), grid_tiles);
        moe_gate_up_mx256_kernel<<<g_gu, kTileThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(3)) != hipSuccess) return err;
        moe_down_mx256_kernel<<<g_dn, kTileThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(4)) != hipSuccess) return err;
    } else {
        const dim3 g_gu((unsigned)(I / kGuCols), grid_tiles);
        const dim3 g_dn((unsigned)(H / kDnCols), grid_tiles);
        if (a.fmt == FP4_FMT_MX) moe_gate_up_kernel<FP4_FMT_MX><<<g_gu, kThreads, 0, s>>>(p);
        else moe_gate_up_kernel<FP4_FMT_NV><<<g_gu, kThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(3)) != hipSuccess) return err;
        if (a.fmt == FP4_FMT_MX) moe_down_kernel<FP4_FMT_MX><<<g_dn, kThreads, 0, s>>>(p);
        else moe_down_kernel<FP4_FMT_NV><<<g_dn, kThreads, 0, s>>>(p);
        if ((err = hipGetLastError()) != hipSuccess || (err = mark(4)) != hipSuccess) return err;
    }
    // 5. weighted combine
    combine_kernel<<<stream_grid(T * H / 4), kThreads, 0, s>>>(reinterpret_cast<const float4*>(ybuf), a.ids, a.topk, E,
                                                                 T, H / 4, reinterpret_cast<uint2*>(a.out));
    if ((err = hipGetLastError()) != hipSuccess || (err = mark(5)) != hipSuccess) return err;
    const int bx = a.fmt == FP4_FMT_MX ? 32 : 16;
    if (a.dbg.x_codes &&
        (err = hipMemcpyAsync(a.dbg.x_codes, xc, (size_t)(T * H / 2), hipMemcpyDeviceToDevice, s)))
        return err;
    if (a.dbg.x_scales &&
        (err = hipMemcpyAsync(a.dbg.x_scales, xs, (size_t)(T * H / bx), hipMemcpyDeviceToDevice, s)))
        return err;
    if (a.dbg.counts && (err = hipMemcpyAsync(a.dbg.counts, counts, (size_t)E * 4, hipMemcpyDeviceToDevice, s)))
        return err;
    if (a.dbg.offsets &&
        (err = hipMemcpyAsync(a.dbg.offsets, offsets, (size_t)(E + 1) * 4, hipMemcpyDeviceToDevice, s)))
        return err;
    if (a.dbg.perm && (err = hipMemcpyAsync(a.dbg.perm, perm, (size_t)S * 4, hipMemcpyDeviceToDevice, s)))
        return err;
    return hipSuccess;
}

}  // namespace fp4
