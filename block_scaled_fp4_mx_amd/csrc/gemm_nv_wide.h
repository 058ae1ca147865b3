// Wide LDS-staged NVFP4 tile for gfx950: 128 rows of A x 512 rows of B, both
// given as NVFP4 codes + E4M3 group scales, K advancing 128 values per step;
// 512 threads, 8 waves, wave w computes all 128 A rows x B rows w*64 .. w*64 + 63
// (8 x 4 accumulator fragments of 16 x 16).  Used by the dense NV GEMM and by
// the prefill-sized MoE grouped GEMMs (A rows gathered per routed slot).
//
// NVFP4 group scales are not a matrix-core scale format, so both operands are
// expanded to the exact fp16 values code * s_g (an E2M1 value times an E4M3
// value has at most 6 significant bits and lies inside fp16's normal range) and
// multiplied on v_mfma_f32_16x16x32_f16; the tensor scales multiply the fp32
// result.  B is expanded in registers by each wave for its own rows; A is
// expanded once per step by the whole workgroup into an fp16 buffer in LDS that
// every wave reads.
//
// Why this shape: each fp16 A fragment read from LDS (1 KiB per wave) feeds
// four MFMAs, so A costs 1/64 LDS byte per flop; each B fragment is expanded
// once per wave and feeds eight MFMAs; every weight byte fetched serves 128 rows,
// and A arrives as codes, a quarter of the bytes of its fp16 form.
//
// Pipeline (one barrier per step).  Three two-slot rings in LDS:
//   B stages   (codes + scales of 512 rows)  2 slots, step ks in slot ks & 1;
//   A stages   (codes + scales of 128 rows)  2 slots, step ks in slot ks & 1;
//   fp16 A     (expanded)                    2 slots, step ks in slot ks & 1.
// At step ks, after the wait for this wave's copies and the barrier, the
// workgroup issues the copies of A(ks + 2), reads B(ks) into registers,
// expands A(ks + 1) into its fp16 slot, issues the copies of B(ks + 2) into
// the B slot just read, and multiplies A(ks) by B(ks).  A slots (codes and
// fp16) are shared: every one written in step ks was last read in step ks - 1,
// which the barrier closes, and every one read in step ks was filled before
// it.  B slots are private to a wave (wave w copies and reads only B rows
// w*64 .. w*64 + 63), so a B slot is refilled as soon as the wave's own reads
// of it have finished, and the weights get two steps of copy time.  The
// expansion needs no barrier of its own: the next step's barrier orders it
// before the fragment reads.
//
// Stage layout per K step (128 values):
//   fp16 A  128 rows x 256 B, 16-byte chunk c of row r at slot c ^ nv_a_swz(r);
//   B codes 512 rows x 64 B in blocks of 16 rows (1 KiB), chunk-major inside a
//           block: chunk c of row r at (r & ~15) * 64 + c * 256 + (r & 15) * 16,
//           so a fragment read (lane = 16 * chunk + row within the block) is one
//           contiguous KiB;
//   B E4M3  512 rows x 8 B, row-major;
//   A codes 128 rows x 64 B and A E4M3 128 rows x 8 B, row-major.
// Every stage arrives by global_load_lds DMA (dwordx4 for codes, dword for the
// scale bytes).
//
// K permutation: within a step, lane group lq (= lane / 16) of every fragment
// holds K values 32 lq .. 32 lq + 31, word i of them (8 codes) going to
// sub-step i; the fp16 A chunk 4 lq + i holds the same K values.  A and B use
// the same permutation, so each MFMA pairs equal K indices.
#pragma once

#include "gemm_nv_tile.h"

namespace fp4 {

constexpr int kNwM = 128, kNwN = 512, kNwK = 128;
constexpr int kNwMf = kNwM / 16;     // A fragments of a full tile
constexpr int kNwARow = kNwK * 2;    // fp16 A bytes of one row per step
constexpr int kNwBRow = kNwK / 2;    // code bytes of one row per step
constexpr int kNwSRow = kNwK / 16;   // E4M3 bytes of one row per step

struct NwBStage {
    uint8_t b[kNwN * kNwBRow];
    uint8_t s[kNwN * kNwSRow];
};
struct NwAStage {
    uint8_t c[kNwM * kNwBRow];
    uint8_t s[kNwM * kNwSRow];
};
struct NwSmem {
    NwBStage b[2];
    NwAStage a[2];
    uint8_t a16[2][kNwM * kNwARow];
};
static_assert(sizeof(NwSmem) <= 160 * 1024, "the wide tile exceeds the LDS of one workgroup");

// Sources of one tile as per-lane byte offsets from workgroup-uniform bases.
//   B codes: DMA q (0..3) of wave w fills rows nw_b_row(q) (one 16-row block
//     per KiB, lane l taking chunk l / 16 of row l % 16 of the block);
//   B scales: dword DMA j (0..1) of wave w fills rows nw_s_row(j), 4 of the
//     row's 8 bytes (nw_s_col);
//   A codes: one DMA per wave, rows nw_ac_row() (16 rows per KiB);
//   A scales: one dword DMA for each of waves 4-7, rows nw_as_row().
// Each offset is the row's byte offset at K step 0 plus the lane's (swizzled)
// chunk; rows past the problem are pointed at a valid row by the caller.
struct NwSrc {
    const uint8_t* b;       // B codes, row pitch K/2
    const uint8_t* s;       // B E4M3 bytes, row pitch K/16
    const uint8_t* ac;      // A codes, row pitch K/2
    const uint8_t* as;      // A E4M3 bytes, row pitch K/16
    uint32_t boff[4], soff[2];
    uint32_t acoff, asoff;
};

__device__ __forceinline__ int nw_wave() { return (int)(threadIdx.x >> 6); }
__device__ __forceinline__ int nw_b_row(int q) { return 64 * nw_wave() + 16 * q + (int)(threadIdx.x & 15); }
__device__ __forceinline__ uint32_t nw_b_chunk(int row) {
    (void)row;
    return ((threadIdx.x & 63u) >> 4) << 4;
}

__device__ __forceinline__ int nw_s_row(int j) { return 64 * nw_wave() + 32 * j + (int)((threadIdx.x & 63) >> 1); }
__device__ __forceinline__ uint32_t nw_s_col() { return (threadIdx.x & 1u) << 2; }
__device__ __forceinline__ int nw_ac_row() { return 16 * nw_wave() + (int)((threadIdx.x & 63) >> 2); }
__device__ __forceinline__ uint32_t nw_ac_chunk() { return (threadIdx.x & 3u) << 4; }
__device__ __forceinline__ int nw_as_row() { return 32 * (nw_wave() & 3) + (int)((threadIdx.x & 63) >> 1); }

// Copies of B for K step ks.
__device__ __forceinline__ void nw_issue_b(NwBStage& st, const NwSrc& S, int ks) {
    const int wave = __builtin_amdgcn_readfirstlane(nw_wave());
    const uint8_t* b = S.b + (int64_t)ks * kNwBRow;
    const uint32_t lb = lds_addr(st.b) + wave * 4096;
#pragma unroll
    for (int q = 0; q < 4; ++q) dma16(b, S.boff[q], lb + q * 1024);
    const uint8_t* sp = S.s + (int64_t)ks * kNwSRow;
    const uint32_t ls = lds_addr(st.s) + wave * 512;
    dma4(sp, S.soff[0], ls);
    dma4(sp, S.soff[1], ls + 256);
}

// Copies of A (codes and scales) for K step ks.
__device__ __forceinline__ void nw_issue_a(NwAStage& st, const NwSrc& S, int ks) {
    const int wave = __builtin_amdgcn_readfirstlane(nw_wave());
    dma16(S.ac + (int64_t)ks * kNwBRow, S.acoff, lds_addr(st.c) + wave * 1024);
    if (wave >= 4) dma4(S.as + (int64_t)ks * kNwSRow, S.asoff, lds_addr(st.s) + (wave - 4) * 256);
}

// Wait until at most one step of B copies (6 per wave) is in flight.
__device__ __forceinline__ void nw_wait_b_in_flight() { asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); }


// Half h (rows 64 h .. 64 h + 63) of one step's A expanded to fp16: each thread
// expands one 16-group, in the swizzled layout the fragment reads use.  The
// load (codes and the group's E4M3 byte) and the store (expansion and write)
// are separate calls so that the loop can issue them groups apart.
__device__ __forceinline__ void nw_load_a_half(const NwAStage& st, int h, uint2& code, uint32_t& scale) {
    const int row = h * 64 + (int)(threadIdx.x >> 3), g = (int)(threadIdx.x & 7);
    code = *reinterpret_cast<const uint2*>(&st.c[row * kNwBRow + g * 8]);
    scale = st.s[row * kNwSRow + g];
}
__device__ __forceinline__ void nw_store_a_half(uint8_t* a16, int h, uint2 code, uint32_t scale) {
    const int row = h * 64 + (int)(threadIdx.x >> 3), g = (int)(threadIdx.x & 7);
    const _Float16 sg = nv_scale_pair(scale)[0];
    *reinterpret_cast<h8_t*>(&a16[row * kNwARow + (((2 * g) ^ nv_a_swz(row)) << 4)]) = nv_expand8(code.x, sg);
    *reinterpret_cast<h8_t*>(&a16[row * kNwARow + (((2 * g + 1) ^ nv_a_swz(row)) << 4)]) = nv_expand8(code.y, sg);
}
__device__ __forceinline__ void nw_expand_a_half(const NwAStage& st, uint8_t* a16, int h) {
    uint2 code;
    uint32_t scale;
    nw_load_a_half(st, h, code, scale);
    nw_store_a_half(a16, h, code, scale);
}

__device__ __forceinline__ uint32_t nw_word(const uint4& c, int i) {
    return i == 0 ? c.x : (i == 1 ? c.y : (i == 2 ? c.z : c.w));
}

// A fragments 2g and 2g + 1 (those below MF) of sub-step i, from the step's
// fp16 A slot.
template <int MF>
__device__ __forceinline__ void nw_read_pair(h8_t (&a)[2], const uint8_t* ab, int i, int g, int lr, int lq) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int mf = 2 * g + u;
        if (mf < MF) {
            const int row = mf * 16 + lr;
            a[u] = *reinterpret_cast<const h8_t*>(&ab[row * kNwARow + (((4 * lq + i) ^ nv_a_swz(row)) << 4)]);
        }
    }
}

// The lane's 32 codes of its row in each of the wave's B fragments of one
// step, and the row's two E4M3 group scales as fp16.
__device__ __forceinline__ void nw_read_b(const NwBStage& st, uint4 (&c)[4], h2_t (&sp)[4], int wave, int lr, int lq) {
#pragma unroll
    for (int nf = 0; nf < 4; ++nf) {
        const int row = wave * 64 + nf * 16 + lr;
        c[nf] = *reinterpret_cast<const uint4*>(&st.b[(row & ~15) * kNwBRow + lq * 256 + lr * 16]);
        sp[nf] = nv_scale_pair(*reinterpret_cast<const uint16_t*>(&st.s[row * kNwSRow + lq * 2]));
    }
}

constexpr int kNwAhead = 2;   // groups by which A fragment reads run ahead of their MFMAs

// Full K loop of one tile for the MF A fragments (16 rows each) that hold rows
// of the problem.  acc[mf][nf]: A rows mf*16 .., B rows wave*64 + nf*16 ..;
// D row = A row, D column = B row.  Every wave takes part in the copies, the A
// expansion and the barriers; A rows of fragments past MF are not expanded.
// MF is the same for the whole workgroup (a tile without rows does nothing).
//
// Inside a step the wave works through T = 4 * NG groups (sub-step i, pair g
// of A fragments: 8 MFMAs each for a full pair).  A group's A fragments are
// read from LDS two groups ahead (a ring of three register pairs), so the read
// latency hides behind the MFMAs of the two groups before it; each sub-step's
// B fragments are expanded during the groups of the sub-step before it (two
// register sets).  Group boundaries are scheduling barriers, which keeps the
// compiler from pulling the reads back next to their MFMAs.  The step's extra
// work rides in its first groups: group 0 also reads the codes of the next
// step's A, group 1 expands them into the other fp16 slot and, once every LDS
// read issued so far has returned (the wave's reads of its B slot among them),
// issues the copies of B(ks + 2) into that slot.
template <int MF>
__device__ __forceinline__ void nw_mainloop(NwSmem& sm, const NwSrc& S, int nsteps, v4f acc[kNwMf][4]) {
    const int lane = threadIdx.x & 63, wave = nw_wave();
    const int lr = lane & 15, lq = lane >> 4;
    static_assert(MF >= 1 && MF <= kNwMf, "fragment count");
    constexpr int kHalves = MF > 4 ? 2 : 1;   // expanded 64-row halves of A
    constexpr int NG = (MF + 1) / 2;          // A fragment pairs per sub-step
    constexpr int T = 4 * NG;                 // groups per step
    // copy order A(0), B(0), A(1), B(1), then per step A(ks + 2), B(ks + 2): the
    // wait at the top of step ks (for B(ks) and A(ks + 1)) leaves B(ks + 1) in flight
    nw_issue_a(sm.a[0], S, 0);
    nw_issue_b(sm.b[0], S, 0);
    nw_wait_b_in_flight();                             // A(0)
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kHalves; ++h) nw_expand_a_half(sm.a[0], sm.a16[0], h);
    if (nsteps > 1) {
        nw_issue_a(sm.a[1], S, 1);
        nw_issue_b(sm.b[1], S, 1);
    }
    for (int ks = 0; ks < nsteps; ++ks) {
        if (ks + 1 < nsteps)
            nw_wait_b_in_flight();
        else
            wait_vm_zero();
        __syncthreads();
        const int cur = ks & 1, nxt = cur ^ 1;
        const bool more = ks + 1 < nsteps;
        if (ks + 2 < nsteps) nw_issue_a(sm.a[cur], S, ks + 2);
        const uint8_t* ab = sm.a16[cur];
        uint4 c[4];
        h2_t sp[4];
        nw_read_b(sm.b[cur], c, sp, wave, lr, lq);
        h8_t af[kNwAhead + 1][2];
#pragma unroll
        for (int t = 0; t < kNwAhead; ++t) nw_read_pair<MF>(af[t], ab, t / NG, t % NG, lr, lq);
        h8_t bx[2][4];
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) bx[0][nf] = nv_expand8(c[nf].x, sp[nf][0]);
        __builtin_amdgcn_sched_barrier(0);
        uint2 acode[kHalves];
        uint32_t ascale[kHalves];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int i = t / NG, g = t % NG;
            if (t == 1 && ks + 2 < nsteps) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                nw_issue_b(sm.b[cur], S, ks + 2);
            }
            if (t + kNwAhead < T)
                nw_read_pair<MF>(af[(t + kNwAhead) % (kNwAhead + 1)], ab, (t + kNwAhead) / NG, (t + kNwAhead) % NG,
                                 lr, lq);
            if (t == 0 && more) {
#pragma unroll
                for (int h = 0; h < kHalves; ++h) nw_load_a_half(sm.a[nxt], h, acode[h], ascale[h]);
            }
            if (t == 1 && more) {
#pragma unroll
                for (int h = 0; h < kHalves; ++h) nw_store_a_half(sm.a16[nxt], h, acode[h], ascale[h]);
            }
            if (i + 1 < 4) {
#pragma unroll
                for (int nf = 0; nf < 4; ++nf)
                    if (nf % NG == g)
                        bx[(i + 1) & 1][nf] = nv_expand8(nw_word(c[nf], i + 1), sp[nf][(i + 1) >> 1]);
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int mf = 2 * g + u;
                if (mf < MF)
#pragma unroll
                    for (int nf = 0; nf < 4; ++nf)
                        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[t % (kNwAhead + 1)][u], bx[i & 1][nf],
                                                                             acc[mf][nf], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

__device__ __forceinline__ void nw_mainloop_rows(NwSmem& sm, const NwSrc& S, int nsteps, v4f acc[kNwMf][4],
                                                 int64_t rows) {
    const int mf = rows <= 0 ? 0 : (rows >= kNwM ? kNwMf : (int)((rows + 15) >> 4));
    switch (__builtin_amdgcn_readfirstlane(mf)) {
        case 8: nw_mainloop<8>(sm, S, nsteps, acc); break;
        case 7: nw_mainloop<7>(sm, S, nsteps, acc); break;
        case 6: nw_mainloop<6>(sm, S, nsteps, acc); break;
        case 5: nw_mainloop<5>(sm, S, nsteps, acc); break;
        case 4: nw_mainloop<4>(sm, S, nsteps, acc); break;
        case 3: nw_mainloop<3>(sm, S, nsteps, acc); break;
        case 2: nw_mainloop<2>(sm, S, nsteps, acc); break;
        case 1: nw_mainloop<1>(sm, S, nsteps, acc); break;
        default: break;                                   // no rows: nothing to copy or multiply
    }
}

}  // namespace fp4
