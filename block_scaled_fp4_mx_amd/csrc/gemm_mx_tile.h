// LDS-staged MXFP4 block tile for gfx950: 256 x 256 outputs per 512-thread
// workgroup, K advancing 256 values (8 MX blocks, one 128-byte line per row)
// per step.
//
// Roles: the workgroup's A tile (rows of C) and B tile (columns of C) are both
// row-major [256][128 B] slabs of packed codes per step; the 8 waves form a
// 2 x 4 grid and each owns 128 x 64 outputs as 8 x 4 MFMA tiles of 16 x 16.
// Two waves share a SIMD: while one waits on LDS reads into fragment registers
// that its own in-flight MFMAs still read, the other keeps the matrix core
// busy.  The MFMA is issued with the B fragment as its first operand, so a
// lane's four accumulator values are four consecutive columns of one output
// row (8-byte bf16 stores).
//
// Measured limits on gfx950 shape the loop: L2 -> LDS traffic is bound by the
// number of requests, and LDS reads by the number of instructions (a 1-byte
// read costs about as much as a 16-byte one).  So:
//   - codes go straight from global memory into LDS (global_load_lds_dwordx4:
//     a wave writes 1 KiB, lane l at byte 16 l), two stages;
//   - UE8M0 scales travel 16 bytes per row (two steps' worth) per request into
//     a separate two-deep buffer, and a lane reads one step's 8 scale bytes of
//     a fragment row with one ds_read_b64, picking its byte with a shift;
//   - the second half-step's fragment reads are interleaved into the first
//     half-step's MFMA stream.
// Slab row r's 16-byte chunk c sits at chunk c ^ (r & 7); a load lane l writes
// chunk l & 7 of row l >> 3 and so fetches global chunk (l & 7) ^ (l >> 3).
// The 8 lanes that a ds_read_b128 serves together read 8 different rows of one
// logical chunk, which land on 8 different bank groups (no conflicts measured).
#pragma once


#include "mma_core.h"

namespace fp4 {

constexpr int kTileM = 256, kTileN = 256, kRowBytes = 128, kStepBlocks = 8;
constexpr int kTileThreads = 512;   // 8 waves: 2 along M x 4 along N
constexpr int kWaveN = 64;          // output columns per wave
constexpr int kWaveFragsN = kWaveN / 16;
constexpr int kScaleRow = 16;      // scale bytes per row held in LDS: two steps

struct MxCodes {
    uint8_t a[kTileM * kRowBytes];
    uint8_t b[kTileN * kRowBytes];
};
struct MxScales {
    uint8_t a[kTileM * kScaleRow];
    uint8_t b[kTileN * kScaleRow];
};
struct MxSmem {
    MxCodes codes[2];
    MxScales scales[2];
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global sources of one operand's slab, as per-lane byte offsets from a base
// that is the same for the whole workgroup (so the copies use the scalar-base
// addressing form).  Code load q (q = 0..3) of a lane fills slab row
// mx_code_row(q) at the lane's swizzled chunk; off[q] is the byte offset of that
// row's K-step-0 line plus the chunk.  Waves 0-3 fill the A scale rows, waves
// 4-7 the B ones, one row per lane (mx_scale_row); soff is the byte offset of
// that row's scales.  The rows may be any rows of the operand (the grouped MoE
// GEMMs gather them), so a slab row past the end of the problem is pointed at
// some valid row; its products only reach outputs that are never stored.
// Offsets are 32-bit: each operand (from its base) must stay below 4 GiB.
struct MxSlabSrc {
    const uint8_t* codes;
    const uint8_t* scales;
    uint32_t offs[4];
    uint32_t soff;
    __device__ __forceinline__ uint32_t off(int q) const { return offs[q]; }
};

// Dense operand whose slab rows are consecutive: the offsets are recomputed
// at each copy from the row base (a few ALU ops), which keeps eight registers
// free for the whole K loop.  The empty asm hides the row base's value, so the
// compiler cannot hoist the eight products out of the loop again.
struct MxDenseSrc {
    const uint8_t* codes;
    const uint8_t* scales;
    int row0;              // operand row of this lane's code copy q = 0
    int last;              // last valid operand row
    uint32_t kbytes, chunk;
    uint32_t soff;
    __device__ __forceinline__ uint32_t off(int q) const {
        int r = row0;
        asm volatile("" : "+v"(r));
        return (uint32_t)min(r + q * 8, last) * kbytes + chunk;
    }
};

__device__ __forceinline__ int mx_code_row(int q) {
    return (int)(threadIdx.x >> 6) * 32 + q * 8 + (int)((threadIdx.x & 63) >> 3);
}
__device__ __forceinline__ int mx_scale_row() { return (int)((threadIdx.x >> 6) & 3) * 64 + (int)(threadIdx.x & 63); }
__device__ __forceinline__ uint32_t mx_chunk16() {
    const uint32_t lane = threadIdx.x & 63;
    return ((lane & 7) ^ (lane >> 3)) * 16;
}

// Dense operand: slab rows r0 .. r0 + 255 of a [rows, kbytes] code matrix,
// clamped to its last row.
__device__ __forceinline__ void mx_dense_src(MxDenseSrc& s, const uint8_t* codes, const uint8_t* scales, int64_t r0,
                                             int64_t rows, int64_t kbytes, int64_t kblocks) {
    s.codes = codes;
    s.scales = scales;
    s.row0 = (int)r0 + mx_code_row(0);
    s.last = (int)rows - 1;
    s.kbytes = (uint32_t)kbytes;
    s.chunk = mx_chunk16();
    s.soff = (uint32_t)min((int)r0 + mx_scale_row(), (int)rows - 1) * (uint32_t)kblocks;
}

__device__ __forceinline__ void mx_slab_src(MxSlabSrc& s, const uint8_t* codes, const uint8_t* scales, int64_t r0,
                                            int64_t rows, int64_t kbytes, int64_t kblocks) {
    s.codes = codes;
    s.scales = scales;
    const int last = (int)rows - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        s.offs[q] = (uint32_t)min((int)r0 + mx_code_row(q), last) * (uint32_t)kbytes + mx_chunk16();
    s.soff = (uint32_t)min((int)r0 + mx_scale_row(), last) * (uint32_t)kblocks;
}

// Global -> LDS copies issued from inline asm: the LDS base goes to M0 in the
// same block (with the one wait state the M0 write needs).  The asm has no
// register results; completion is awaited explicitly (wait_vm_zero) before the
// barrier that precedes any read of the buffer.  Issued this way, the compiler
// does not hold the next stage's copies in flight against every LDS read of
// the current stage.
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_ptr_t)const_cast<void*>(p);
}

__device__ __forceinline__ void wait_vm_zero() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Before the barrier that hands a stage back to the copies: this wave's copies
// have landed and its LDS reads have returned their data (a wave may hold a
// half-step's fragments across the barrier, read from the stage the next
// copies overwrite).
__device__ __forceinline__ void wait_copies_and_reads() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// Only the A slab rows below arows (the rows of the fragments in use) are
// fetched; B always fills the whole slab.
template <class SA, class SB>
__device__ __forceinline__ void mx_issue_codes(MxCodes& st, const SA& A, const SB& B, int ks, int arows) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* ac = A.codes + (int64_t)ks * kRowBytes;
    const uint8_t* bc = B.codes + (int64_t)ks * kRowBytes;
    const uint32_t la = lds_addr(st.a) + wave * 4 * 1024, lb = lds_addr(st.b) + wave * 4 * 1024;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (wave * 32 + q * 8 < arows) dma16(ac, A.off(q), la + q * 1024);
        dma16(bc, B.off(q), lb + q * 1024);
    }
}

// Scale bytes of steps 2p and 2p + 1 (blocks 16p .. 16p + 15) of every row:
// waves 0-3 fetch the A rows, waves 4-7 the B rows.
template <class SA, class SB>
__device__ __forceinline__ void mx_issue_scales(MxScales& sc, const SA& A, const SB& B, int p, int arows) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (wave < 4) {
        if (wave * 64 < arows)
            dma16(A.scales + (int64_t)p * 16, A.soff, lds_addr(sc.a) + wave * 1024);
    } else {
        dma16(B.scales + (int64_t)p * 16, B.soff, lds_addr(sc.b) + (wave - 4) * 1024);
    }
}

// Per-lane LDS bases of this wave's fragments (row wm*128 + i*16 + lr has
// (row & 7) == (lr & 7), so fragment i is the base plus i * 16 rows).
struct MxLdsBase {
    int a[2], b[2];        // code byte offset within a stage, per half-step s
    int sa, sb;            // scale byte offset within a scale buffer
};

__device__ __forceinline__ MxLdsBase mx_lds_base(int wm, int wn, int lane) {
    const int lr = lane & 15, lk = lane >> 4;
    MxLdsBase b;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int coff = ((s * 4 + lk) ^ (lr & 7)) * 16;
        b.a[s] = (wm * 128 + lr) * kRowBytes + coff;
        b.b[s] = (wn * kWaveN + lr) * kRowBytes + coff;
    }
    b.sa = (wm * 128 + lr) * kScaleRow;
    b.sb = (wn * kWaveN + lr) * kScaleRow;
    return b;
}

__device__ __forceinline__ v8i frag_at(const uint8_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

// Scale operand for half-step s: byte s*4 + lk of the row's step bytes; the
// MFMA reads bits 7:0 of the operand.
__device__ __forceinline__ int scale_at(uint2 w, int s, int lk) {
    return (int)((s ? w.y : w.x) >> (8 * lk));
}

// One half-step's fragments and scale operands in registers.
struct MxFrags {
    v8i a[8], b[kWaveFragsN];
    int sa[8], sb[kWaveFragsN];
};

// Reads half-step S (K values S*128 .. of the step) of the stage `codes` for
// the wave's first NF row fragments; wsa / wsb hold the step's scale words.
template <int NF, int S>
__device__ __forceinline__ void mx_read_half(MxFrags& f, const MxCodes& codes, const MxLdsBase& lb, const uint2* wsa,
                                             const uint2* wsb, int lk) {
    const uint8_t* st_a = codes.a + lb.a[S];
    const uint8_t* st_b = codes.b + lb.b[S];
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        f.a[i] = frag_at(st_a + i * 16 * kRowBytes);
        f.sa[i] = scale_at(wsa[i], S, lk);
    }
#pragma unroll
    for (int j = 0; j < kWaveFragsN; ++j) {
        f.b[j] = frag_at(st_b + j * 16 * kRowBytes);
        f.sb[j] = scale_at(wsb[j], S, lk);
    }
}

template <int NF>
__device__ __forceinline__ void mx_mfma_half(v4f acc[kWaveFragsN][8], const MxFrags& f) {
#pragma unroll
    for (int j = 0; j < kWaveFragsN; ++j)
#pragma unroll
        for (int i = 0; i < NF; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(f.b[j], f.a[i], acc[j][i], 4, 4, 0, f.sb[j], 0,
                                                                           f.sa[i]);
}

// Full K loop of one 256 x 256 tile; acc zeroed by the caller.  At the start of
// step ks the copies of step ks have landed (wait + barrier) and those of step
// ks + 1 (and, when ks + 1 is even, the scales of steps ks + 1 and ks + 2) are
// issued into the buffers step ks - 1 used.  Each step is two half-steps of
// 128 K values: read the half's fragments from LDS, then one MFMA per
// accumulator.
//
// Half of the waves (those whose index has bit 1 set) run half a step behind
// the others: they hold the fragments of a step's second half across the
// barrier and multiply them at the start of the next step.  In lock step every
// wave would read its fragments from LDS right after each barrier while the
// matrix cores idle; staggered, half the waves read while the other half
// multiply.  (Of the splits tried, this one measured fastest; the result does
// not depend on it, since every accumulator still sees its K blocks in order.)
// Only the wave's first NF row fragments are computed (the grouped GEMMs pass
// fewer for a segment's last rows); every wave takes part in the copies and
// barriers whatever its NF.
template <int NF, class SA, class SB>
__device__ __forceinline__ void mx_tile_mainloop(MxSmem& sm, const SA& A, const SB& B, int64_t kblocks,
                                                 v4f acc[kWaveFragsN][8], int arows) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3, lk = lane >> 4;
    const bool lag = (__builtin_amdgcn_readfirstlane(wave) & 2) != 0;
    const int nsteps = (int)(kblocks / kStepBlocks);
    const MxLdsBase lb = mx_lds_base(wm, wn, lane);
    mx_issue_codes(sm.codes[0], A, B, 0, arows);
    mx_issue_scales(sm.scales[0], A, B, 0, arows);
    uint2 wsa[8], wsb[kWaveFragsN];
    MxFrags f;
    for (int ks = 0; ks < nsteps; ++ks) {
        wait_copies_and_reads();
        __syncthreads();
        if (ks + 1 < nsteps) {
            mx_issue_codes(sm.codes[(ks + 1) & 1], A, B, ks + 1, arows);
            if (((ks + 1) & 1) == 0) mx_issue_scales(sm.scales[((ks + 1) >> 1) & 1], A, B, (ks + 1) >> 1, arows);
        }
        if (NF == 0) continue;
        if (lag && ks > 0) mx_mfma_half<NF>(acc, f);          // second half of step ks - 1
        const uint8_t* sc_a = sm.scales[(ks >> 1) & 1].a + (ks & 1) * 8;
        const uint8_t* sc_b = sm.scales[(ks >> 1) & 1].b + (ks & 1) * 8;
#pragma unroll
        for (int i = 0; i < NF; ++i) wsa[i] = *reinterpret_cast<const uint2*>(sc_a + lb.sa + i * 16 * kScaleRow);
#pragma unroll
        for (int j = 0; j < kWaveFragsN; ++j) wsb[j] = *reinterpret_cast<const uint2*>(sc_b + lb.sb + j * 16 * kScaleRow);
        mx_read_half<NF, 0>(f, sm.codes[ks & 1], lb, wsa, wsb, lk);
        mx_mfma_half<NF>(acc, f);
        mx_read_half<NF, 1>(f, sm.codes[ks & 1], lb, wsa, wsb, lk);
        if (!lag) mx_mfma_half<NF>(acc, f);
    }
    if (NF != 0 && lag && nsteps > 0) mx_mfma_half<NF>(acc, f);
}

// The K loop for a wave of which only `rows` (from its first row on) are
// needed: ceil(rows / 16) row fragments, at least 0 and at most 8.  tile_rows
// (the rows of the whole tile from its first row on) bounds the A rows fetched.
template <class SA, class SB>
__device__ __forceinline__ void mx_tile_mainloop_rows(MxSmem& sm, const SA& A, const SB& B, int64_t kblocks,
                                                      v4f acc[kWaveFragsN][8], int64_t rows,
                                                      int64_t tile_rows) {
    // A slab rows to fetch: the tile's rows rounded up to whole fragments
    const int arows = __builtin_amdgcn_readfirstlane((int)min<int64_t>(kTileM, (tile_rows + 15) & ~int64_t(15)));
    const int nf = rows <= 0 ? 0 : (rows >= 128 ? 8 : (int)((rows + 15) >> 4));
    switch (__builtin_amdgcn_readfirstlane(nf)) {
        case 8: mx_tile_mainloop<8>(sm, A, B, kblocks, acc, arows); break;
        case 7: mx_tile_mainloop<7>(sm, A, B, kblocks, acc, arows); break;
        case 6: mx_tile_mainloop<6>(sm, A, B, kblocks, acc, arows); break;
        case 5: mx_tile_mainloop<5>(sm, A, B, kblocks, acc, arows); break;
        case 4: mx_tile_mainloop<4>(sm, A, B, kblocks, acc, arows); break;
        case 3: mx_tile_mainloop<3>(sm, A, B, kblocks, acc, arows); break;
        case 2: mx_tile_mainloop<2>(sm, A, B, kblocks, acc, arows); break;
        case 1: mx_tile_mainloop<1>(sm, A, B, kblocks, acc, arows); break;
        default: mx_tile_mainloop<0>(sm, A, B, kblocks, acc, arows); break;
    }
}

}  // namespace fp4
