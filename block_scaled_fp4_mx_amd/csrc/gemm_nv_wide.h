// Wide LDS-staged NVFP4 tile for gfx950: TM rows of A (fp16) x 512 rows of B
// (NVFP4 codes + E4M3 group scales), K advancing 128 values per step through a
// ring of NS stages; 512 threads, 8 waves, wave w computes all TM A rows x B
// rows w*64 .. w*64 + 63 (TM/16 x 4 accumulator fragments of 16 x 16).
// Configurations: 64 rows with three stages (dense NV GEMM, A given as codes)
// and 128 rows with two stages (prefill-sized MoE segments).
//
// Why this shape: each fp16 A fragment read from LDS (1 KiB per wave) feeds
// four MFMAs, so A costs 1/64 LDS byte per flop, half of what a 32-column wave
// tile costs (which saturates the 128 B/clk LDS port at the fp16 MFMA rate);
// each B fragment is expanded once per wave and feeds TM/16 MFMAs, so the
// expansion (one VALU lane-op per code) costs 1/(2 TM) lane-ops per flop, and
// every weight byte fetched serves TM rows.
// B is expanded in registers exactly as in the narrow NV tile: code * s_g is
// an fp16 with at most 6 significant bits, built by v_cvt_scalef32_pk_f16_fp4
// and a packed fp16 multiply by s_g.
//
// Stage layout per K step (128 values):
//   A fp16  TM rows x 256 B, 16-byte chunk c of row r at slot c ^ (r & 15);
//   B codes 512 rows x 64 B, chunk c of row r at slot c ^ nw_swz(r), which
//           puts any 8 (and any 16) consecutive rows of a fragment read on
//           different 16-byte bank groups;
//   B E4M3  512 rows x 8 B, row-major.
// Every stage arrives by global_load_lds DMA (dwordx4 for codes and fp16,
// dword for the scale bytes).  With A given as NVFP4 codes (the dense GEMM),
// the stages hold A's codes (64 x 64 B) and scales (64 x 8 B) instead, and the
// workgroup expands them into one shared fp16 A buffer each step.
//
// K permutation: within a step, lane group lq (= lane / 16) of every fragment
// holds K values 32 lq .. 32 lq + 31, word i of them (8 codes) going to
// sub-step i; the fp16 A chunk 4 lq + i holds the same K values.  A and B use
// the same permutation, so each MFMA pairs equal K indices.
#pragma once

#include "gemm_nv_tile.h"

namespace fp4 {

constexpr int kNwN = 512, kNwK = 128;
constexpr int kNwARow = kNwK * 2;    // fp16 A bytes of one row per step
constexpr int kNwBRow = kNwK / 2;    // code bytes of one row per step
constexpr int kNwSRow = kNwK / 16;   // E4M3 bytes of one row per step

template <int TM, bool ACODES>
struct NwStage {
    uint8_t a[ACODES ? 16 : TM * kNwARow];          // fp16 A
    uint8_t b[kNwN * kNwBRow];
    uint8_t s[kNwN * kNwSRow];
    uint8_t ac[ACODES ? TM * kNwBRow : 16];         // A codes, row-major (A given as NVFP4)
    uint8_t as[ACODES ? TM * kNwSRow : 16];         // A E4M3 bytes, row-major
};
template <int TM, int NS, bool ACODES>
struct NwSmem {
    static_assert((TM == 64 && NS == 3) || (TM == 128 && NS == 2), "supported wide-tile configurations");
    NwStage<TM, ACODES> st[NS];
    uint8_t a16[ACODES ? TM * kNwARow : 16];        // expanded A of the current step
};

// Sources of one tile as per-lane byte offsets from workgroup-uniform bases.
//   fp16 A: DMA q (0 .. TM/32 - 1) of wave w fills rows nw_a_row<TM>(q) (4 rows
//     per KiB);
//   B codes: DMA q (0..3) of wave w fills rows nw_b_row(q) (16 rows per KiB);
//   B scales: dword DMA j (0..1) of wave w fills rows nw_s_row(j), 4 of the
//     row's 8 bytes (nw_s_col);
//   A codes (waves 0-3, one DMA each) and A scales (waves 4-5, one dword DMA
//     each) when A is given as NVFP4.
// Each offset is the row's byte offset at K step 0 plus the lane's (swizzled)
// chunk; rows past the problem are pointed at a valid row by the caller.
struct NwSrc {
    const uint8_t* a;       // fp16 A, row pitch 2K bytes
    const uint8_t* b;       // B codes, row pitch K/2
    const uint8_t* s;       // B E4M3 bytes, row pitch K/16
    const uint8_t* ac;      // A codes (pitch K/2) and E4M3 bytes (pitch K/16)
    const uint8_t* as;
    uint32_t aoff[4], boff[4], soff[2];
    uint32_t acoff, asoff;
};

__device__ __forceinline__ int nw_wave() { return (int)(threadIdx.x >> 6); }
template <int TM>
__device__ __forceinline__ int nw_a_row(int q) {
    return (TM / 8) * nw_wave() + 4 * q + (int)((threadIdx.x & 63) >> 4);
}
__device__ __forceinline__ uint32_t nw_a_chunk(int row) { return ((threadIdx.x & 15u) ^ (uint32_t)(row & 15)) << 4; }
__device__ __forceinline__ int nw_b_row(int q) { return 64 * nw_wave() + 16 * q + (int)((threadIdx.x & 63) >> 2); }
__device__ __forceinline__ uint32_t nw_swz(int row) { return (uint32_t)((row >> 1) ^ (row >> 3)) & 3u; }
__device__ __forceinline__ uint32_t nw_b_chunk(int row) { return ((threadIdx.x & 3u) ^ nw_swz(row)) << 4; }
__device__ __forceinline__ int nw_s_row(int j) { return 64 * nw_wave() + 32 * j + (int)((threadIdx.x & 63) >> 1); }
__device__ __forceinline__ uint32_t nw_s_col() { return (threadIdx.x & 1u) << 2; }
// A given as codes: TM = 64 copies its codes with waves 0-3 (16 rows each) and
// its scales with waves 4-5 (32 rows each); TM = 128 with all 8 waves and waves
// 4-7.
template <int TM>
__device__ __forceinline__ int nw_ac_row() {
    return 16 * (TM == 64 ? (nw_wave() & 3) : nw_wave()) + (int)((threadIdx.x & 63) >> 2);
}
__device__ __forceinline__ uint32_t nw_ac_chunk() { return (threadIdx.x & 3u) << 4; }
template <int TM>
__device__ __forceinline__ int nw_as_row() {
    return 32 * (TM == 64 ? (nw_wave() & 1) : (nw_wave() & 3)) + (int)((threadIdx.x & 63) >> 1);
}

// Copies of K step ks into one stage.  Every wave issues the same copies each
// step (TM/32 + 6; with A as codes and TM = 64, 7 for waves 0-5 and 6 for waves
// 6-7): the three-stage waits count on it.
template <int TM, bool ACODES>
__device__ __forceinline__ void nw_issue(NwStage<TM, ACODES>& st, const NwSrc& S, int ks) {
    const int wave = __builtin_amdgcn_readfirstlane(nw_wave());
    if constexpr (ACODES && TM == 64) {
        if (wave < 4)
            dma16(S.ac + (int64_t)ks * kNwBRow, S.acoff, lds_addr(st.ac) + wave * 1024);
        else if (wave < 6)
            dma4(S.as + (int64_t)ks * kNwSRow, S.asoff, lds_addr(st.as) + (wave - 4) * 256);
    } else if constexpr (ACODES) {
        dma16(S.ac + (int64_t)ks * kNwBRow, S.acoff, lds_addr(st.ac) + wave * 1024);
        if (wave >= 4) dma4(S.as + (int64_t)ks * kNwSRow, S.asoff, lds_addr(st.as) + (wave - 4) * 256);
    } else {
        const uint8_t* a = S.a + (int64_t)ks * kNwARow;
        const uint32_t la = lds_addr(st.a) + wave * (TM / 32) * 1024;
#pragma unroll
        for (int q = 0; q < TM / 32; ++q) dma16(a, S.aoff[q], la + q * 1024);
    }
    const uint8_t* b = S.b + (int64_t)ks * kNwBRow;
    const uint32_t lb = lds_addr(st.b) + wave * 4096;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(b, S.boff[q], lb + q * 1024);
    const uint8_t* sp = S.s + (int64_t)ks * kNwSRow;
    const uint32_t ls = lds_addr(st.s) + wave * 512;
    dma4(sp, S.soff[0], ls);
    dma4(sp, S.soff[1], ls + 256);
}

// Three stages: wait until this wave's copies of the current step have landed,
// leaving those of the next step in flight.
template <int TM, bool ACODES>
__device__ __forceinline__ void nw_wait_current() {
    static_assert(TM == 64, "the copy counts below are those of 64-row tiles");
    if constexpr (ACODES) {
        if (__builtin_amdgcn_readfirstlane(nw_wave()) < 6)
            asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    }
}

// A given as codes: each thread expands one 16-group per 64 rows (TM x 8
// groups) to fp16 into the shared A buffer, in the swizzled layout the
// fragment reads use.
template <int TM>
__device__ __forceinline__ void nw_expand_a(const NwStage<TM, true>& st, uint8_t* a16) {
#pragma unroll
    for (int h = 0; h < TM / 64; ++h) {
        const int row = h * 64 + (int)(threadIdx.x >> 3), g = (int)(threadIdx.x & 7);
        const uint2 c = *reinterpret_cast<const uint2*>(&st.ac[row * kNwBRow + g * 8]);
        const _Float16 sg = nv_scale_pair(st.as[row * kNwSRow + g])[0];
        *reinterpret_cast<h8_t*>(&a16[row * kNwARow + (((2 * g) ^ (row & 15)) << 4)]) = nv_expand8(c.x, sg);
        *reinterpret_cast<h8_t*>(&a16[row * kNwARow + (((2 * g + 1) ^ (row & 15)) << 4)]) = nv_expand8(c.y, sg);
    }
}

__device__ __forceinline__ uint32_t nw_word(const uint4& c, int i) {
    return i == 0 ? c.x : (i == 1 ? c.y : (i == 2 ? c.z : c.w));
}

// Full K loop of one TM x 512 tile for the MF A fragments (16 rows each) that
// hold rows of the problem.  acc[mf][nf]: A rows mf*16 .., B rows
// wave*64 + nf*16 ..; D row = A row, D column = B row.  Every wave takes part
// in the copies, the A expansion and the barriers whatever its MF.  The copies
// of step ks + NS - 1 are issued at step ks into the stage step ks - 1 used.
template <int TM, int NS, bool ACODES, int MF>
__device__ __forceinline__ void nw_mainloop(NwSmem<TM, NS, ACODES>& sm, const NwSrc& S, int nsteps,
                                            v4f acc[TM / 16][4]) {
    const int lane = threadIdx.x & 63, wave = nw_wave();
    const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nsteps) nw_issue<TM, ACODES>(sm.st[p], S, p);
    int cur = 0;
    for (int ks = 0; ks < nsteps; ++ks) {
        if constexpr (NS == 3) {
            if (ks + 1 < nsteps)
                nw_wait_current<TM, ACODES>();
            else
                wait_vm_zero();
        } else {
            wait_vm_zero();
        }
        __syncthreads();
        const int nxt = cur == 0 ? NS - 1 : cur - 1;     // (ks + NS - 1) % NS
        if (ks + NS - 1 < nsteps) nw_issue<TM, ACODES>(sm.st[nxt], S, ks + NS - 1);
        const NwStage<TM, ACODES>& st = sm.st[cur];
        cur = cur + 1 == NS ? 0 : cur + 1;
        if constexpr (ACODES) {
            nw_expand_a<TM>(st, sm.a16);
            __syncthreads();
        }
        if (MF == 0) continue;
        const uint8_t* ab = ACODES ? sm.a16 : st.a;
        // B: the lane's 32 codes of its row in each of the wave's fragments
        uint4 c[4];
        h2_t sp[4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) {
            const int row = wave * 64 + nf * 16 + lr;
            c[nf] = *reinterpret_cast<const uint4*>(&st.b[row * kNwBRow + ((lq ^ nw_swz(row)) << 4)]);
            sp[nf] = nv_scale_pair(*reinterpret_cast<const uint16_t*>(&st.s[row * kNwSRow + lq * 2]));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // the sub-step's A fragment reads go out first and land while B is expanded
            h8_t a[MF > 0 ? MF : 1];
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
                const int row = mf * 16 + lr;
                a[mf] = *reinterpret_cast<const h8_t*>(&ab[row * kNwARow + (((4 * lq + i) ^ (row & 15)) << 4)]);
            }
            h8_t bx[4];
#pragma unroll
            for (int nf = 0; nf < 4; ++nf) bx[nf] = nv_expand8(nw_word(c[nf], i), sp[nf][i >> 1]);
#pragma unroll
            for (int mf = 0; mf < MF; ++mf)
#pragma unroll
                for (int nf = 0; nf < 4; ++nf)
                    acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mf], bx[nf], acc[mf][nf], 0, 0, 0);
        }
    }
}

template <int TM, int NS, bool ACODES>
__device__ __forceinline__ void nw_mainloop_rows(NwSmem<TM, NS, ACODES>& sm, const NwSrc& S, int nsteps,
                                                 v4f acc[TM / 16][4], int64_t rows) {
    constexpr int kMaxMf = TM / 16;
    const int mf = rows <= 0 ? 0 : (rows >= TM ? kMaxMf : (int)((rows + 15) >> 4));
    switch (__builtin_amdgcn_readfirstlane(mf)) {
        case 8: if constexpr (kMaxMf >= 8) nw_mainloop<TM, NS, ACODES, 8>(sm, S, nsteps, acc); break;
        case 7: if constexpr (kMaxMf >= 7) nw_mainloop<TM, NS, ACODES, 7>(sm, S, nsteps, acc); break;
        case 6: if constexpr (kMaxMf >= 6) nw_mainloop<TM, NS, ACODES, 6>(sm, S, nsteps, acc); break;
        case 5: if constexpr (kMaxMf >= 5) nw_mainloop<TM, NS, ACODES, 5>(sm, S, nsteps, acc); break;
        case 4: nw_mainloop<TM, NS, ACODES, 4>(sm, S, nsteps, acc); break;
        case 3: nw_mainloop<TM, NS, ACODES, 3>(sm, S, nsteps, acc); break;
        case 2: nw_mainloop<TM, NS, ACODES, 2>(sm, S, nsteps, acc); break;
        case 1: nw_mainloop<TM, NS, ACODES, 1>(sm, S, nsteps, acc); break;
        default: nw_mainloop<TM, NS, ACODES, 0>(sm, S, nsteps, acc); break;
    }
}

}  // namespace fp4
