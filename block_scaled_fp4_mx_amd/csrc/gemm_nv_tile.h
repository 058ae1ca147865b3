// LDS-staged NVFP4 block tile for gfx950: 32 rows of A (fp16) x 256 rows of B
// (NVFP4 codes + E4M3 group scales), K advancing 256 values per step through
// three stages; 512 threads, 8 waves, each wave all 32 A rows x 32 B rows (two
// 16-row fragments).  Used by the decode-sized MoE grouped GEMMs: few rows per
// expert, the expert weights stream from HBM, and the third stage keeps two K
// steps of weights in flight per workgroup.
//
// NVFP4 group scales are not a matrix-core scale format, so B is expanded in
// registers to the exact fp16 values code * s_g (at most 6 significant bits,
// inside fp16's normal range for every E4M3 scale) and fed to
// v_mfma_f32_16x16x32_f16; the tensor scales multiply the fp32 result.  The
// expansion costs two instructions per pair of codes: v_cvt_scalef32_pk_f16_fp4
// (scale 1) converts the codes, and a packed fp16 multiply by s_g (two group
// bytes go to fp16 in one v_cvt_scalef32_pk_f16_fp8) finishes the exact value.
//
// Stage layout per K step: A TM rows x 512 B (16-byte chunk c of row r at
// c ^ nv_a_swz(r)), B codes 256 rows x 128 B (chunk c of row r at c ^ (r & 7)), B
// scales 256 rows x 16 B.  All of it goes from global memory straight into LDS
// (global_load_lds_dwordx4 / _dword), as in the MX tile.
#pragma once

#include "gemm_mx_tile.h"

namespace fp4 {

constexpr int kNvTileN = 256, kNvThreads = 512;
constexpr int kNvARow = 512;        // bytes of one A row per step (256 fp16)
constexpr int kNvBRow = 128;        // code bytes of one B row per step
constexpr int kNvSRow = 16;         // scale bytes of one B row per step

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

template <int TM>
struct NvStageT {
    uint8_t a[TM * kNvARow];                        // fp16 A
    uint8_t b[kNvTileN * kNvBRow];
    uint8_t s[kNvTileN * kNvSRow];
};
template <int TM, int NS>
struct NvSmemT {
    static_assert(TM == 32 && NS == 3, "the copy counts below are those of 32 A rows in three stages");
    NvStageT<TM> st[NS];
};

// Sources of one tile, as per-lane byte offsets from bases that are the same
// for the whole workgroup.  A (fp16): DMA q of a lane fills 1 KiB block
// wave * (TM/16) + q, i.e. row nv_a_row<TM>(q), LDS chunk lane % 32, from global
// chunk (lane % 32) ^ nv_a_swz(row); aoff[q] is that row's byte offset plus the
// chunk.  B codes: DMA q fills rows (wave * 4 + q) * 8 + lane / 8 as in the MX
// tile (boff[q]).  B scales: every wave fills its 512 bytes with two 4-byte
// DMAs (sdw[j]: byte wave*512 + j*256 + 4*lane of the scale slab).
struct NvSrc {
    const uint8_t* a;       // fp16 activations
    const uint8_t* b;       // codes, row pitch K/2
    const uint8_t* s;       // E4M3 bytes, row pitch K/16
    uint32_t aoff[4], boff[4], sdw[2];
};

template <int TM>
__device__ __forceinline__ int nv_a_row(int q) {
    return 2 * ((int)(threadIdx.x >> 6) * (TM / 16) + q) + (int)((threadIdx.x & 63) >> 5);
}
// fp16 A rows: 16-byte chunk c of row r sits at slot c ^ nv_a_swz(r).  With
// the plain mask r & 15, the fragment reads of lanes (r, lq) and (r ^ 4, lq ^ 1)
// of one instruction land on the same banks (measured with the LDS bank-conflict
// counter: one stall cycle per access); this mask, linear in r, pairs no two
// lanes of a fragment read that way.
__device__ __forceinline__ int nv_a_swz(int row) { return ((row & 7) << 1) | ((row >> 3) & 1); }

__device__ __forceinline__ uint32_t nv_a_chunk(int row) {
    return (((threadIdx.x & 31) ^ (uint32_t)nv_a_swz(row)) * 16);
}
// Three-stage scale DMA j of this lane: slab row, and byte within the row's 16.
__device__ __forceinline__ int nv_sdw_row(int j) {
    return ((int)(threadIdx.x >> 6) * 512 + j * 256 + 4 * (int)(threadIdx.x & 63)) >> 4;
}
__device__ __forceinline__ uint32_t nv_sdw_col() { return (uint32_t)((4 * (threadIdx.x & 63)) & 15); }

__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t off, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "s"(lds)
                 : "memory", "m0");
}

// DMA instructions each wave issues per K step (A 2, B codes 4, B scales 2):
// the count the waits rely on.
constexpr int kNvDmaPerStep = 8;

// Copies of one K step: every wave issues the same fixed number of copies.
template <int TM>
__device__ __forceinline__ void nv_issue(NvStageT<TM>& sm, const NvSrc& S, int ks) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint8_t* b = S.b + (int64_t)ks * kNvBRow;
    const uint32_t lb = lds_addr(sm.b) + wave * 4 * 1024;
    constexpr int QA = TM / 16;
    const uint8_t* a = S.a + (int64_t)ks * kNvARow;
    const uint32_t la = lds_addr(sm.a) + wave * QA * 1024;
#pragma unroll
    for (int q = 0; q < QA; ++q) dma16(a, S.aoff[q], la + q * 1024);   // block = 2 rows
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(b, S.boff[q], lb + q * 1024);
#pragma unroll
    for (int j = 0; j < 2; ++j) dma4(S.s + (int64_t)ks * kNvSRow, S.sdw[j], lds_addr(sm.s) + wave * 512 + j * 256);
}

// Two E4M3 group bytes (bits 15:0 of g2) -> the fp16 pair {s_g0, s_g1}.  Every
// E4M3 value, subnormals included, is an fp16 normal number, so the conversion
// (v_cvt_scalef32_pk_f16_fp8 with scale 1) is exact.
__device__ __forceinline__ h2_t nv_scale_pair(uint32_t g2) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(g2, 1.0f, false);
}

// Eight codes (one word) of one group -> 8 exact fp16 values code * s_g.  The
// codes convert exactly (scale 1); the product of an E2M1 and an E4M3 value has
// at most 6 significant bits and lies in [2^-10, 2688] (or is zero), so the
// packed fp16 multiply rounds nothing.
__device__ __forceinline__ h8_t nv_expand8(uint32_t w, _Float16 s) {
    const h2_t s2 = {s, s};
    const h2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const h2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const h2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const h2_t d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    return h8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Full K loop of one TM x 256 tile for the MF A fragments (16 rows each) that
// hold rows of the problem.  acc[mf][nf]: A rows mf*16 .., B rows of the wave's
// fragment nf (wave * 32 + nf * 16 ..); D row = A row, D column = B row.
// Every wave takes part in the copies and barriers.  The copies of step
// ks + NS - 1 are issued at step ks; the wait at step ks leaves the copies of
// the later steps in flight.
template <int TM, int NS, int MF>
__device__ __forceinline__ void nv_tile_mainloop(NvSmemT<TM, NS>& sm, const NvSrc& S, int nsteps, v4f acc[4][2]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nsteps) nv_issue<TM>(sm.st[p], S, p);
    int cur = 0;
    for (int ks = 0; ks < nsteps; ++ks) {
        if (ks + 1 < nsteps)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kNvDmaPerStep) : "memory");   // step ks + 1 may still land
        else
            wait_vm_zero();
        __syncthreads();
        const int nxt = cur == 0 ? NS - 1 : cur - 1;    // (ks + NS - 1) % NS
        if (ks + NS - 1 < nsteps) nv_issue<TM>(sm.st[nxt], S, ks + NS - 1);
        const NvStageT<TM>& st = sm.st[cur];
        cur = cur + 1 == NS ? 0 : cur + 1;
        if (MF == 0) continue;
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            // B: the lane's 32 codes (K hs*128 + 32 lq ..) of its row in each fragment
            h8_t bx[2][4];
#pragma unroll
            for (int nf = 0; nf < 2; ++nf) {
                const int row = wave * 32 + nf * 16 + lr;
                const uint4 c = *reinterpret_cast<const uint4*>(&st.b[row * kNvBRow + (((hs * 4 + lq) ^ (row & 7)) * 16)]);
                const uint32_t sg = *reinterpret_cast<const uint16_t*>(&st.s[row * kNvSRow + hs * 8 + lq * 2]);
                const h2_t sp = nv_scale_pair(sg);
                bx[nf][0] = nv_expand8(c.x, sp[0]);
                bx[nf][1] = nv_expand8(c.y, sp[0]);
                bx[nf][2] = nv_expand8(c.z, sp[1]);
                bx[nf][3] = nv_expand8(c.w, sp[1]);
            }
            // A: fp16 rows, chunk hs*16 + 4 lq + i of each row
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
                const int row = mf * 16 + lr;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ch = (hs * 16 + lq * 4 + i) ^ nv_a_swz(row);
                    const h8_t a = *reinterpret_cast<const h8_t*>(&st.a[row * kNvARow + ch * 16]);
#pragma unroll
                    for (int nf = 0; nf < 2; ++nf)
                        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bx[nf][i], acc[mf][nf], 0, 0, 0);
                }
            }
        }
    }
}

template <int TM, int NS>
__device__ __forceinline__ void nv_tile_mainloop_rows(NvSmemT<TM, NS>& sm, const NvSrc& S, int nsteps, v4f acc[4][2],
                                                      int64_t rows) {
    constexpr int kMaxMf = TM / 16;
    const int mf = rows <= 0 ? 0 : (rows >= TM ? kMaxMf : (int)((rows + 15) >> 4));
    switch (__builtin_amdgcn_readfirstlane(mf)) {
        case 4: if constexpr (kMaxMf >= 4) nv_tile_mainloop<TM, NS, 4>(sm, S, nsteps, acc); break;
        case 3: if constexpr (kMaxMf >= 3) nv_tile_mainloop<TM, NS, 3>(sm, S, nsteps, acc); break;
        case 2: nv_tile_mainloop<TM, NS, 2>(sm, S, nsteps, acc); break;
        case 1: nv_tile_mainloop<TM, NS, 1>(sm, S, nsteps, acc); break;
        default: nv_tile_mainloop<TM, NS, 0>(sm, S, nsteps, acc); break;
    }
}

}  // namespace fp4
