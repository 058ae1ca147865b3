// LDS-staged W4A8 block tile for gfx950: MXFP8 (E4M3) activations times MXFP4
// (E2M1) weights, both with UE8M0 scales on 32-element blocks along K
// ("DeepSeek-V4 FP4 QAT" article, sections 4.2-4.3: FP4 weights with FP8
// activations, FP4 expanding losslessly into FP8).  One
// v_mfma_scale_f32_16x16x128_f8f6f4 takes the E2M1 weight fragment as its first
// operand and the E4M3 activation fragment as its second, with the UE8M0 block
// scales as per-lane operands.
//
// Operand layout of the mixed-format instruction (measured on gfx950 with a
// one-hot probe): the E2M1 operand's lane group g (lanes 16g .. 16g + 15, one
// row each) holds K values 32g .. 32g + 31 of a 128-value step, and the scale
// operand of lane group g applies to K block g of both operands; the E4M3
// operand's lane group g holds K values 16g .. 16g + 15 in bytes 0-15 and
// 64 + 16g .. 64 + 16g + 15 in bytes 16-31 (so block g's E4M3 bytes sit in the
// lane groups 2(g % 2) and 2(g % 2) + 1, first or second half by g / 2).
//
// 256 x 256 outputs per 512-thread workgroup; K advances 128 values per step.
// Per stage the A slab is [256 rows][128 B] of E4M3 codes and the B slab
// [256 rows][64 B] of packed E2M1 codes (48 KiB), two stages.  The 8 waves form
// a 4 (M) x 2 (N) grid; a wave owns 64 x 128 outputs: 4 activation fragments of
// 8 registers and 8 weight fragments of 4 registers per step, 32 MFMAs.
// Scale bytes travel 16 per row (four steps' worth) per request into a
// two-deep buffer, one u8 LDS read per fragment per step.
//
// Swizzles (a ds_read_b128 serves 8 lanes = 8 consecutive rows of one logical
// chunk; these put them on 8 different 16-byte bank groups):
//   A: 16-byte chunk c of row r sits at chunk c ^ (r & 7) (8 chunks per row);
//   B: chunk c of row r sits at chunk c ^ ((r >> 1) & 3) ^ ((r >> 3) & 1) (4 per
//      row; 16 consecutive rows land on distinct (r % 4, chunk) places of the
//      256-byte bank space).
// The copies (global_load_lds_dwordx4) write a wave's 1 KiB contiguously, lane
// l at byte 16 l, so each lane fetches the global chunk whose swizzled place is
// its own.
#pragma once

#include "gemm_mx_tile.h"

namespace fp4 {

constexpr int kW8TileM = 256, kW8TileN = 256, kW8StepK = 128;
constexpr int kW8ARow = 128, kW8BRow = 64, kW8ScaleRow = 16;
constexpr int kW8Threads = 512;
constexpr int kW8FragsM = 4, kW8FragsN = 8;   // per wave: 64 rows x 128 columns

struct W8Stage {
    uint8_t a[kW8TileM * kW8ARow];
    uint8_t b[kW8TileN * kW8BRow];
};
struct W8Scales {
    uint8_t a[kW8TileM * kW8ScaleRow];
    uint8_t b[kW8TileN * kW8ScaleRow];
};
struct W8Smem {
    W8Stage st[2];
    W8Scales sc[2];
};

// Depends on row bits 1-3 only, so fragments 16 rows apart share it.
__device__ __forceinline__ int w8_b_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }

// Dense operand sources: per-lane byte offsets (from the operand's base) of the
// K-step-0 chunk each copy fetches, and of the row's scales.  Rows past the
// end are pointed at the last row; their products reach only outputs that are
// never stored.  Offsets are 32-bit: each operand stays below 2 GiB.
struct W8Src {
    const uint8_t* a;          // E4M3 codes [m, k]
    const uint8_t* as;         // UE8M0 [m, k/32]
    const uint8_t* b;          // E2M1 codes [n, k/2]
    const uint8_t* bs;         // UE8M0 [n, k/32]
    uint32_t aoff[4], boff[2];
    uint32_t soff;             // A scale row (waves 0-3) or B scale row (waves 4-7)
};

// Copy roles.  A: wave w, copy q fills slab rows 32 w + 8 q .. + 7, lane l row
// 32 w + 8 q + l / 8 at chunk l % 8.  B: copy q fills rows 32 w + 16 q .. + 15,
// lane l row 32 w + 16 q + l / 4 at chunk l % 4.  Scales: waves 0-3 the A rows
// 64 w + l, waves 4-7 the B rows 64 (w - 4) + l.
__device__ __forceinline__ void w8_src(W8Src& S, const uint8_t* a, const uint8_t* as, const uint8_t* b,
                                       const uint8_t* bs, int64_t m0, int64_t n0, int64_t m, int64_t n, int64_t k) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    S.a = a;
    S.as = as;
    S.b = b;
    S.bs = bs;
    const uint32_t ka = (uint32_t)k, kb = (uint32_t)(k / 2), kbl = (uint32_t)(k / 32);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = wave * 32 + q * 8 + (lane >> 3);
        const uint32_t chunk = (uint32_t)((lane & 7) ^ (row & 7));
        S.aoff[q] = (uint32_t)min(m0 + row, m - 1) * ka + chunk * 16;
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int row = wave * 32 + q * 16 + (lane >> 2);
        const uint32_t chunk = (uint32_t)((lane & 3) ^ w8_b_swz(row));
        S.boff[q] = (uint32_t)min(n0 + row, n - 1) * kb + chunk * 16;
    }
    const int srow = (wave & 3) * 64 + lane;
    S.soff = wave < 4 ? (uint32_t)min(m0 + srow, m - 1) * kbl : (uint32_t)min(n0 + srow, n - 1) * kbl;
}

__device__ __forceinline__ void w8_issue_codes(W8Stage& st, const W8Src& S, int ks) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* a = S.a + (int64_t)ks * kW8ARow;
    const uint8_t* b = S.b + (int64_t)ks * kW8BRow;
    const uint32_t la = lds_addr(st.a) + wave * 4096, lb = lds_addr(st.b) + wave * 2048;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(a, S.aoff[q], la + q * 1024);
#pragma unroll
    for (int q = 0; q < 2; ++q) dma16(b, S.boff[q], lb + q * 1024);
}

// Scale bytes of steps 4p .. 4p + 3 (blocks 16p .. 16p + 15) of every row.
__device__ __forceinline__ void w8_issue_scales(W8Scales& sc, const W8Src& S, int p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < 4)
        dma16(S.as + (int64_t)p * 16, S.soff, lds_addr(sc.a) + wave * 1024);
    else
        dma16(S.bs + (int64_t)p * 16, S.soff, lds_addr(sc.b) + (wave - 4) * 1024);
}

// One step's fragments and scale operands of a wave.
struct W8Frags {
    v8i a[kW8FragsM];
    v8i b[kW8FragsN];
    int sa[kW8FragsM], sb[kW8FragsN];
};

// Per-lane LDS offsets of the wave's fragment 0 (fragment i is 16 rows further;
// 16-row steps keep r & 7 and the B swizzle's bits).
struct W8Lds {
    int a0, a1, b, sa, sb;
};

__device__ __forceinline__ W8Lds w8_lds(int wm, int wn, int lane) {
    const int lr = lane & 15, lk = lane >> 4;
    const int arow = wm * 64 + lr, brow = wn * 128 + lr;
    W8Lds o;
    o.a0 = arow * kW8ARow + ((lk ^ (arow & 7)) << 4);          // K 16 lk .. + 15
    o.a1 = arow * kW8ARow + (((4 + lk) ^ (arow & 7)) << 4);    // K 64 + 16 lk .. + 15
    o.b = brow * kW8BRow + ((lk ^ w8_b_swz(brow)) << 4);
    o.sa = arow * kW8ScaleRow + lk;
    o.sb = brow * kW8ScaleRow + lk;
    return o;
}

// Reads step ks's fragments (stage `st`, scale buffer `sc`, step ks & 3 of it).
__device__ __forceinline__ void w8_read(W8Frags& f, const W8Stage& st, const W8Scales& sc, const W8Lds& o, int ks) {
    const int sk = (ks & 3) * 4;
#pragma unroll
    for (int j = 0; j < kW8FragsN; ++j) {
        const uint4 v = *reinterpret_cast<const uint4*>(st.b + o.b + j * 16 * kW8BRow);
        f.b[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        f.sb[j] = sc.b[o.sb + j * 16 * kW8ScaleRow + sk];
    }
#pragma unroll
    for (int i = 0; i < kW8FragsM; ++i) {
        const uint4 lo = *reinterpret_cast<const uint4*>(st.a + o.a0 + i * 16 * kW8ARow);
        const uint4 hi = *reinterpret_cast<const uint4*>(st.a + o.a1 + i * 16 * kW8ARow);
        f.a[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        f.sa[i] = sc.a[o.sa + i * 16 * kW8ScaleRow + sk];
    }
}

// acc[j][i]: weight fragment j (output columns) x activation fragment i (rows);
// a lane's four values are four consecutive columns of one output row.  J0..J1
// selects the weight fragments.
template <int J0, int J1>
__device__ __forceinline__ void w8_mfma(v4f acc[kW8FragsN][kW8FragsM], const W8Frags& f) {
#pragma unroll
    for (int j = J0; j < J1; ++j)
#pragma unroll
        for (int i = 0; i < kW8FragsM; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[j], f.a[i], acc[j][i], 4, 0, 0, f.sb[j],
                                                                           0, f.sa[i]);
}

// Full K loop (acc zeroed by the caller; k a multiple of 512).  At the start of
// step ks the copies of step ks have landed (wait + barrier) and those of step
// ks + 1 (and, when ks + 1 is a multiple of 4, the scales of steps ks + 1 ..
// ks + 4) are issued into the buffers that step ks - 1 (resp. ks - 7 .. ks - 4)
// used.  With LAG, waves whose index has bit 1 set multiply the second half of
// their weight fragments one step late (right after the next barrier), so that
// on a SIMD one wave's LDS reads overlap the other wave's MFMAs; every
// accumulator still sees its K blocks in order.
template <bool LAG>
__device__ __forceinline__ void w8_mainloop(W8Smem& sm, const W8Src& S, int nsteps, v4f acc[kW8FragsN][kW8FragsM]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const bool lag = LAG && (__builtin_amdgcn_readfirstlane(wave) & 2) != 0;
    const W8Lds o = w8_lds(wm, wn, lane);
    w8_issue_codes(sm.st[0], S, 0);
    w8_issue_scales(sm.sc[0], S, 0);
    W8Frags f;
    for (int ks = 0; ks < nsteps; ++ks) {
        wait_copies_and_reads();
        __syncthreads();
        if (ks + 1 < nsteps) {
            w8_issue_codes(sm.st[(ks + 1) & 1], S, ks + 1);
            if (((ks + 1) & 3) == 0) w8_issue_scales(sm.sc[((ks + 1) >> 2) & 1], S, (ks + 1) >> 2);
        }
        if (lag && ks > 0) w8_mfma<kW8FragsN / 2, kW8FragsN>(acc, f);
        w8_read(f, sm.st[ks & 1], sm.sc[(ks >> 2) & 1], o, ks);
        w8_mfma<0, kW8FragsN / 2>(acc, f);
        if (!lag) w8_mfma<kW8FragsN / 2, kW8FragsN>(acc, f);
    }
    if (lag && nsteps > 0) w8_mfma<kW8FragsN / 2, kW8FragsN>(acc, f);
}

}  // namespace fp4
