// fa_bwd.hip - bf16 attention backward for gfx950 (MI355X, CDNA4).
//
// Gradients of O = softmax(scale * Q K^T) V (optionally causal) with respect
// to Q, K and V, given dO and the forward's O and per-row log-sum-exp.  The
// backward pass the pages describe keeps no N x N matrix either: it recomputes
// the scores block by block from Q, K and the stored row statistics
// ("PagedAttention vs FlashAttention: key differences", training section;
// "LLM study notes", DEVOCEAN tech blog, FlashAttention core principles:
// recomputation).  With P = exp(S - LSE) recomputed per tile:
//     dV = P^T dO,   dP = dO V^T,   dS = P o (dP - delta),  delta_i = dO_i . O_i
//     dQ = scale dS K,   dK = scale dS^T Q
// (delta_i equals sum_j P_ij dP_ij: the softmax Jacobian's row term).
//
// Two launches, no atomics, so results are deterministic:
//  1. bwd_dq_kernel: a work group owns 128 queries (32 per wave, Q and dO rows
//     in registers) and streams K / V tiles, as the forward does: S^T = K Q^T,
//     dP^T = V dO^T (lane = one query, so lse2 and delta are per-lane scalars),
//     dS^T in registers, dQ^T += K^T dS^T.  Its prologue forms each row's
//     statistics, lse2 = LSE log2(e) and delta, from the dO fragments it holds
//     and the O row, and stores them per 32-row block into a small workspace
//     (256 bytes per block: one LDS DMA load for the next kernel).
//  2. dK and dV: a work group owns 128 keys and streams the Q / dO rows
//     through LDS (HBM -> LDS without registers), in one of two layouts:
//     bwd_dkdv_kernel (d = 128): each 32-key slice is worked by a pair of
//     waves on one SIMD, one holding the K rows and dV^T (S = Q K^T, P,
//     dV^T += dO^T P), the other the V rows and dK^T (dP = dO V^T,
//     dS = P (dP - delta) with P passed through LDS, dK^T += Q^T dS);
//     bwd_dkdv1_kernel (d = 64): one wave per slice does all four products
//     (small enough at d = 64 for two waves per SIMD).  Transposed operands
//     are read by ds_read_b64_tr_b16.
// Recomputing S and dP in both (1) and (2) costs 14 N^2 d flops per head
// instead of 10 N^2 d, the price of having no atomic dQ accumulation.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>

#include "fa_gfx950.h"
#include "fa_kernels.h"

namespace {

using namespace fa_gfx950;

constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr int BQ = 64;                 // query rows per Q / dO tile of the one-wave dK/dV kernel
constexpr int BKV = 64;                // key rows per tile in the dQ kernel
constexpr int BM = NWAVES * 32;        // queries per dQ work group
constexpr int BK = 128;                // keys per dK/dV work group
constexpr int SB = 32;                 // query rows per statistics block
constexpr int SB_FLOATS = 2 * SB;      // per 32-row block: lse2[32], delta[32] (256 bytes)

// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// 2a. dK, dV at d = 64: one wave per key slice.
//
// A work group owns 128 keys (32 per wave, K and V rows held in registers as
// MFMA B operands) and streams 64-row Q / dO tiles through LDS
// (double-buffered).  Per tile a wave computes S = Q K^T and dP = dO V^T
// (lane = one key, 16 queries per 32-row block), P and dS in registers, then
// dV^T += dO^T P and dK^T += Q^T dS.  At d = 64 a wave needs about 240
// registers, so two waves share a SIMD (two work groups per CU).
constexpr int STATS_KIB_FLOATS = 256;  // LDS room for a tile's statistics (1 KiB)
template <int D>
constexpr int dkdv1_stage_elems() {                       // Q, dO, stats (1 KiB), in uint16
    return 2 * BQ * D + 2 * STATS_KIB_FLOATS;
}

// dK, dV of the BK keys from k0 of head bh.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv1_block(uint16_t* smem0, uint16_t* smem1,
                                           const uint16_t* __restrict__ Q,
                                           const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V,
                                           const uint16_t* __restrict__ dO,
                                           const float* __restrict__ stats,
                                           uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                           int N, float scale_log2, float scale, int bh, int k0) {
    constexpr int TILE = BQ * D;                          // elements of a Q or dO tile
    constexpr int LPW = TILE * 2 / 1024 / NWAVES;         // 1 KiB loads per wave per tensor
    constexpr int NKC = D / 16;
    constexpr int ND = D / 32;
    const size_t base = (size_t)bh * (size_t)N * D;
    const uint16_t* __restrict__ Qh = Q + base;
    const uint16_t* __restrict__ dOh = dO + base;
    const int n_qt = (N + BQ - 1) / BQ;
    const int n_sb = (N + SB - 1) / SB;
    const float* st_h = stats + (size_t)bh * n_sb * SB_FLOATS;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wk0 = k0 + 32 * wave;            // first key of this wave
    const int key = wk0 + l32;                 // this lane's key (MFMA column)

    // K and V rows of this wave's keys: B operands of S = Q K^T and dP = dO V^T
    bf16x8 kop[NKC], vop[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        kop[kc] = row_operand<D>(K + base, key, N, 2 * kc + g, 0u);
        vop[kc] = row_operand<D>(V + base, key, N, 2 * kc + g, 0u);
    }
    f32x16 dvacc[ND], dkacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dvacc[db][r] = 0.f; dkacc[db][r] = 0.f; }

    int gofs[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) gofs[i] = tile_load_offset<D>(wave * LPW + i, lane);
    auto load_tile = [&](int qt, uint16_t* stage) __device__ __attribute__((always_inline)) {
        const int bytes = N * D * 2;
        const int tb = qt * BQ * D * 2;
        load_tile_lds<LPW>(Qh, bytes, tb, &gofs[0], stage, wave * LPW);
        load_tile_lds<LPW>(dOh, bytes, tb, &gofs[0], stage + TILE, wave * LPW);
        // the two 32-row statistics blocks of the tile (and 512 bytes more,
        // unused), the offset in the range-checked per-lane part: zeros past
        // the end of the head's statistics
        if (wave == 0) {
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)st_h, (short)0, n_sb * SB_FLOATS * 4, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + 2 * TILE), 16,
                                                     qt * 2 * SB_FLOATS * 4 + lane * 16, 0, 0, 0);
        }
    };

    int rofs[NKC];                             // row-major fragment: query row l32, chunk 2kc+g
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) rofs[kc] = frag_offset<D>(l32, 2 * kc + g);
    int tofs[2][ND];                           // transposed fragment, d rows db*32 ..
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int db = 0; db < ND; ++db) tofs[hl][db] = trfrag_offset<D>(lane, hl, db * 32);

    auto tile_step = [&](int qt, uint16_t* cur, uint16_t* nxt, auto mask_tag) __device__
        __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): this wave's loads have landed
        __syncthreads();
        if (qt + 1 < n_qt) load_tile(qt + 1, nxt);
        // keep the dV / dK accumulators in AGPRs for the whole loop (an empty
        // asm with an AGPR operand; it emits no instruction)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            asm volatile("" : "+a"(dvacc[db]));
            asm volatile("" : "+a"(dkacc[db]));
        }
        const int q0 = qt * BQ;
        if (MASK && CAUSAL && q0 + BQ - 1 < wk0) return;   // every query precedes every key
        const uint16_t* qs = cur;
        const uint16_t* dos = cur + TILE;
        const float* sts = reinterpret_cast<const float*>(cur + 2 * TILE);

        // The tile is worked as a two-stage software pipeline over its two
        // 32-query blocks, so that one block's softmax (VALU) overlaps the
        // other block's matrix products:
        //   A: S, dP of block 0
        //   B: S, dP of block 1         | P, dS of block 0
        //   C: dV, dK from block 0      | P, dS of block 1
        //   D: dV, dK from block 1
        // Each phase ends in a scheduling fence.  At one wave per SIMD nothing
        // hides a wait on an LDS read, so the phases without softmax work (A,
        // D) issue all their operand reads first, and B and C keep 12 / 24
        // reads ahead while spreading the VALU work between the MFMAs
        // (measured: about 2-4% faster than reading 4 MFMAs ahead).
        using H0 = std::integral_constant<int, 0>;
        using H1 = std::integral_constant<int, 1>;
        f32x16 sacc[2], pacc[2];
        bf16x8 pop[2][2], dsop[2][2];

        // S = Q K^T and dP = dO V^T of one 32-query block (16 MFMAs)
        auto scores = [&](auto hbt) __device__ __attribute__((always_inline)) {
            constexpr int hb = decltype(hbt)::value;
#pragma unroll
            for (int r = 0; r < 16; ++r) { sacc[hb][r] = 0.f; pacc[hb][r] = 0.f; }
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(qs + hb * 32 * D + rofs[kc]));
                sacc[hb] = mfma(a, kop[kc], sacc[hb]);
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(dos + hb * 32 * D + rofs[kc]));
                pacc[hb] = mfma(b, vop[kc], pacc[hb]);
            }
        };

        // P and dS of one block; lane holds key `key` and queries
        // q0 + 32hb + 8i + 4g + j in register r = 4i + j.  Masked: keys after
        // the query (causal) and queries past N.
        const int lo = CAUSAL ? key - (q0 + 4 * g) : INT_MIN;
        const int hi = N - 1 - (q0 + 4 * g);
        auto softmax = [&](auto hbt) __device__ __attribute__((always_inline)) {
            constexpr int hb = decltype(hbt)::value;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 l4 = *reinterpret_cast<const float4*>(sts + 2 * SB * hb + 8 * i + 4 * g);
                const float4 d4 =
                    *reinterpret_cast<const float4*>(sts + 2 * SB * hb + SB + 8 * i + 4 * g);
                const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                const float dv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * i + j;
                    float p = fast_exp2(fmaf(sacc[hb][r], scale_log2, -lv[j]));
                    if constexpr (MASK) {
                        const int qrel = 32 * hb + 8 * i + j;
                        if (qrel < lo || qrel > hi) p = 0.f;
                    }
                    const float ds = p * (pacc[hb][r] - dv[j]);
                    pop[hb][r >> 3][r & 7] = (__bf16)p;
                    dsop[hb][r >> 3][r & 7] = (__bf16)ds;
                }
            }
        };

        // dV^T += dO^T P and dK^T += Q^T dS over the block's two chunks of 16
        // queries (16 MFMAs); the query order inside a chunk matches the
        // registers of P and dS
        auto grads = [&](auto hbt) __device__ __attribute__((always_inline)) {
            constexpr int hb = decltype(hbt)::value;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int rb = (32 * hb + 16 * cc) * D;
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const bf16x8 a = tr_operand(dos + rb + tofs[0][db], dos + rb + tofs[1][db]);
                    dvacc[db] = mfma(a, pop[hb][cc], dvacc[db]);
                    const bf16x8 b = tr_operand(qs + rb + tofs[0][db], qs + rb + tofs[1][db]);
                    dkacc[db] = mfma(b, dsop[hb][cc], dkacc[db]);
                }
            }
        };

        constexpr int NM = 2 * NKC;            // MFMAs per phase (= 4 ND)
        // A
        scores(H0{});
        __builtin_amdgcn_sched_group_barrier(0x100, NM, 0);   // every operand read first
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
        __builtin_amdgcn_sched_barrier(0);
        // B
        scores(H1{});
        softmax(H0{});
        __builtin_amdgcn_sched_group_barrier(0x100, 12, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
        // C
        grads(H0{});
        softmax(H1{});
        __builtin_amdgcn_sched_group_barrier(0x100, 24, 2);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 2);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        // D
        grads(H1{});
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * NM, 3);
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 3);
    };

    // query tiles: the two tiles that straddle the diagonal (causal), then the
    // unmasked ones, then the ragged last tile
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    uint16_t* const stage0 = smem0;
    uint16_t* const stage1 = smem1;
    const int qt_begin = CAUSAL ? k0 / BQ : 0;
    const int qt_diag_end = CAUSAL ? min(n_qt, (k0 + BK) / BQ) : 0;
    const int n_full = N / BQ;
    // tile qt lives in stage (qt - qt_begin) & 1 and every call names its
    // stages statically.  The diagonal tiles (at most two) come first, so the
    // unmasked pairs start on stage 0 (qt_diag_end - qt_begin is 0 or 2
    // whenever an unmasked tile exists), and the rest (an odd last full tile,
    // the ragged tile: at most two) start on stage 0 again.  The mask hides
    // nothing in a full tile past the diagonal.
    load_tile(qt_begin, stage0);
    int qt = qt_begin;
    if (qt < qt_diag_end) tile_step(qt++, stage0, stage1, Mask{});
    if (qt < qt_diag_end) tile_step(qt++, stage1, stage0, Mask{});
    for (; qt + 1 < n_full; qt += 2) {
        tile_step(qt, stage0, stage1, NoMask{});
        tile_step(qt + 1, stage1, stage0, NoMask{});
    }
    if (qt < n_qt) tile_step(qt++, stage0, stage1, Mask{});
    if (qt < n_qt) tile_step(qt++, stage1, stage0, Mask{});

    // epilogue: lane holds key `key`, d = db*32 + 8i + 4g + j in register 4i + j
    store_o_row<ND>(dV + base + (size_t)key * D, dvacc, 1.f, g, key < N);
    store_o_row<ND>(dK + base + (size_t)key * D, dkacc, scale, g, key < N);
}

// ---------------------------------------------------------------------------
// 2b. dK, dV at d = 128: a pair of waves per key slice.
//
// A work group owns BK = 128 keys as four slices of 32 keys, and each slice
// is worked by two waves that share a SIMD (waves w and w + 4):
//  * the P wave holds the slice's K rows (MFMA B operands) and dV^T.  Per
//    32-query block it computes S = Q K^T, P = 2^(S c - lse2) (masked), puts P
//    (fp32) in LDS for its partner and adds dV^T += dO^T P;
//  * the dS wave holds the slice's V rows and dK^T.  It computes dP = dO V^T,
//    reads P back, forms dS = P (dP - delta) and adds dK^T += Q^T dS.
// A wave then keeps 32 + 64 VGPRs of operands and accumulators (d = 128), two
// waves fit on a SIMD, and one wave's exponentials or dS arithmetic run
// beside the other's matrix products.  The 32-query blocks are worked in
// segments that end in one barrier: in segment s the P wave adds block s's
// dV and computes block s+1's P, the dS wave adds block s's dK (the P of
// block s was published by the barrier before) and computes block s+1's dP.
// A block's Q and dO rows and statistics stream through four LDS stages,
// loaded three segments before their first use; P goes through two LDS
// buffers (block parity).  Both waves of a pair have the same lane layout for
// S and dP (lane = one key, 16 queries), so a lane reads back exactly the P
// values its partner lane wrote.
constexpr int DKDV_WAVES = 8;
constexpr int DKDV_THREADS = DKDV_WAVES * 64;
constexpr int PBUF_FLOATS = 4 * 1024;  // fp32 P of a 32 x 32 block, four slices (16 KiB)

template <int D>
constexpr int dkdv_stage_elems() {     // Q and dO rows of a 32-query block, statistics (uint16)
    return 2 * SB * D + 2 * SB_FLOATS;
}
// buffer -> LDS loads a wave issues per block: its 1 KiB region(s) of the Q
// and dO rows, and the 256 bytes of statistics
template <int D>
constexpr int dkdv_loads_per_block() { return D == 128 ? 3 : 2; }

// Position of a segment in the four-stage rotation: the stages of block s
// (gradient products) and block s+1 (scores) are s % 4 and (s+1) % 4, and
// the segment loads block s+3 into stage (s+3) % 4.  FIRST: no block s
// (segment -1); LAST: no block s+1 and no load; MASK: block s+1's P takes the
// causal mask.
template <int POS_, bool FIRST_, bool LAST_, bool MASK_ = false>
struct SegPos {
    static constexpr int SA = (POS_ + 4) % 4, SB = (POS_ + 5) % 4, SL = (POS_ + 7) % 4;
    static constexpr bool FIRST = FIRST_, LAST = LAST_, MASK = MASK_;
};

// dK, dV of the BK keys from k0 of head bh.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_block(uint16_t* st0, uint16_t* st1, uint16_t* st2,
                                           uint16_t* st3, float* pb0, float* pb1,
                                           const uint16_t* __restrict__ Q,
                                           const uint16_t* __restrict__ K,
                                           const uint16_t* __restrict__ V,
                                           const uint16_t* __restrict__ dO,
                                           const float* __restrict__ stats,
                                           uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                           int N, float scale_log2, float scale, int bh, int k0) {
    constexpr int BLK = SB * D;                           // elements of a block's Q or dO rows
    constexpr int NKC = D / 16;
    constexpr int ND = D / 32;
    constexpr int LPB = dkdv_loads_per_block<D>();
    const size_t base = (size_t)bh * (size_t)N * D;
    const uint16_t* __restrict__ Qh = Q + base;
    const uint16_t* __restrict__ dOh = dO + base;
    const int n_sb = (N + SB - 1) / SB;
    const float* st_h = stats + (size_t)bh * n_sb * SB_FLOATS;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slice = wave & 3;
    const bool pwave = wave < 4;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int key = k0 + 32 * slice + l32;     // this lane's key (MFMA column)

    // K rows (P wave) or V rows (dS wave) of the slice: B operands of the
    // score products S = Q K^T / dP = dO V^T
    bf16x8 kv[NKC];
    {
        const uint16_t* src = (pwave ? K : V) + base;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) kv[kc] = row_operand<D>(src, key, N, 2 * kc + g, 0u);
    }
    f32x16 acc[ND];                            // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    // operand offsets: the score product's A rows come from Q (P wave) or dO,
    // the gradient product's transposed A from dO (P wave) or Q
    const int xoff = pwave ? 0 : BLK;
    const int yoff = pwave ? BLK : 0;
    int rofs[NKC];                             // byte offsets within a stage
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) rofs[kc] = 2 * (frag_offset<D>(l32, 2 * kc + g) + xoff);
    int tofs[2][ND];
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int db = 0; db < ND; ++db)
            tofs[hl][db] = 2 * (trfrag_offset<D>(lane, hl, db * 32) + yoff);
    const int pofs = slice * 1024 + lane * 4;  // this lane's P floats (register 4i + j at + 256 i + j)

    // 32-query blocks b = 0 .. nb-1 of this key block: from the first that
    // holds a query at or after its first key (causal) to the last
    const int qb_begin = CAUSAL ? k0 / SB : 0;
    const int nb = n_sb - qb_begin;

    // Block b into `stage`.  Every wave issues the same number of loads per
    // block (LPB: its 1 KiB region of the Q rows and of the dO rows at
    // d = 128, of either at d = 64, and the 256 bytes of statistics, which all
    // eight waves write with the same bytes), so a wait for the loads of all
    // blocks but the last issued is vmcnt(LPB).  The whole byte offset goes in
    // the per-lane offset, which the buffer range check covers: rows past N
    // arrive as zeros, and so does every row of a block past the last (b >= nb:
    // the range is empty).  Zero Q and dO rows with zero statistics give
    // P = 1, dP = 0, dS = 0 and add nothing to dV or dK, so only the causal
    // diagonal needs a mask.
    auto load_block = [&](int b, uint16_t* stage) __device__ __attribute__((always_inline)) {
        const int qb = qb_begin + min(b, nb - 1);
        const bool real = b < nb;
        const int bytes = real ? N * D * 2 : 0;
        const int tb = qb * SB * D * 2;
        if constexpr (D == 128) {
            const int go = tile_load_offset<D>(wave, lane) + tb;
            load_tile_lds<1>(Qh, bytes, 0, &go, stage, wave);
            load_tile_lds<1>(dOh, bytes, 0, &go, stage + BLK, wave);
        } else {
            const int go = tile_load_offset<D>(wave & 3, lane) + tb;
            load_tile_lds<1>(pwave ? Qh : dOh, bytes, 0, &go, stage + (wave >> 2) * BLK, wave & 3);
        }
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)st_h, (short)0, real ? n_sb * SB_FLOATS * 4 : 0, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(stage + 2 * BLK), 4,
                                                 qb * SB_FLOATS * 4 + lane * 4, 0, 0, 0);
    };
    auto stage_ptr = [&](auto idx) __device__ __attribute__((always_inline)) -> uint16_t* {
        constexpr int i = decltype(idx)::value;
        if constexpr (i == 0) return st0;
        else if constexpr (i == 1) return st1;
        else if constexpr (i == 2) return st2;
        else return st3;
    };

    // S (P wave) or dP (dS wave) of the block in `stage` (8 MFMAs at
    // d = 128): lane holds key `key` and the block's queries 8i + 4g + j in
    // register 4i + j
    auto scores = [&](const uint16_t* stage) __device__ __attribute__((always_inline)) {
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const bf16x8 a = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(stage) + rofs[kc]));
            s = mfma(a, kv[kc], s);
        }
        return s;
    };
    // dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS wave) over the block's two
    // chunks of 16 queries; the query order inside a chunk matches the
    // registers of P and dS
    auto grads = [&](const uint16_t* stage, const bf16x8* o) __device__
        __attribute__((always_inline)) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const char* sc = reinterpret_cast<const char*>(stage + 16 * cc * D);
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const bf16x8 a = tr_operand(reinterpret_cast<const uint16_t*>(sc + tofs[0][db]),
                                            reinterpret_cast<const uint16_t*>(sc + tofs[1][db]));
                acc[db] = mfma(a, o[cc], acc[db]);
            }
        }
    };
    auto read_lse = [&](const uint16_t* stage, float4* l4) __device__
        __attribute__((always_inline)) {
        const float* sts = reinterpret_cast<const float*>(stage + 2 * BLK);
#pragma unroll
        for (int i = 0; i < 4; ++i) l4[i] = *reinterpret_cast<const float4*>(sts + 8 * i + 4 * g);
    };
    // P of block b from its scores (P wave): into LDS as fp32 and into o as
    // bf16.  `mask`: the block holds queries before keys of the work group
    // (causal, blocks 0-3), and P is zero where the key follows the query.
    auto make_p = [&](const f32x16& s, const float4* l4, float* pb, int b, bf16x8* o,
                      auto mask_tag) __device__ __attribute__((always_inline)) {
        constexpr bool mask = decltype(mask_tag)::value;
        const int lo = key - ((qb_begin + b) * SB + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lv[4] = {l4[i].x, l4[i].y, l4[i].z, l4[i].w};
            float pv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * i + j;
                float p = fast_exp2(fmaf(s[r], scale_log2, -lv[j]));
                const int qrel = 8 * i + j;
                if constexpr (mask)
                    if (qrel < lo) p = 0.f;
                pv[j] = p;
                o[r >> 3][r & 7] = (__bf16)p;
            }
            *reinterpret_cast<float4*>(pb + pofs + 256 * i) = make_float4(pv[0], pv[1], pv[2], pv[3]);
        }
    };
    // dS = P (dP - delta) of a block (dS wave): P read back from LDS, delta
    // from the block's statistics (read_pd), then the arithmetic (make_ds)
    auto read_pd = [&](const uint16_t* stage, const float* pb, float4* p4, float4* d4) __device__
        __attribute__((always_inline)) {
        const float* sts = reinterpret_cast<const float*>(stage + 2 * BLK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p4[i] = *reinterpret_cast<const float4*>(pb + pofs + 256 * i);
            d4[i] = *reinterpret_cast<const float4*>(sts + SB + 8 * i + 4 * g);
        }
    };
    auto make_ds = [&](const f32x16& dp, const float4* p4, const float4* d4, bf16x8* o) __device__
        __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float dv[4] = {d4[i].x, d4[i].y, d4[i].z, d4[i].w};
            const float pv[4] = {p4[i].x, p4[i].y, p4[i].z, p4[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * i + j;
                o[r >> 3][r & 7] = (__bf16)(pv[j] * (dp[r] - dv[j]));
            }
        }
    };

    // End of a segment: this wave's P writes are done and the loads of block
    // s+2 (read from the next segment on) have landed, those of block s+3 may
    // stay in flight (vmcnt(LPB), lgkmcnt(0)); then the barrier.  Written out
    // because __syncthreads() would also wait for the loads still in flight.
    // The empty asm with a memory clobber keeps LDS accesses on their side.
    auto seg_barrier = [&]() __device__ __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0070 | LPB);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
    };

    // Scheduling patterns (sched_group_barrier masks: 0x008 MFMA, 0x100 DS
    // read, 0x002 VALU).  sched_scores: `pre` reads (the P wave's statistics,
    // the dS wave's P and delta) and kAhead operand reads first, then per
    // score MFMA one read (and, in the dS wave, kVpS vector instructions).
    // sched_grads: kTrAhead operands (two transposed reads each) first, then
    // per gradient MFMA one operand and `vpm` vector instructions.
    constexpr int kAhead = 4;
    constexpr int kTrAhead = 2;
    constexpr int kVpS = 5;
    constexpr int kVpP = 9;
    constexpr int GM = 2 * ND;                 // gradient MFMAs per block
    auto sched_scores = [&](auto idt, int pre) __device__ __attribute__((always_inline)) {
        constexpr int id = decltype(idt)::value;
        if (pre == 8) __builtin_amdgcn_sched_group_barrier(0x100, 8, id);
        else __builtin_amdgcn_sched_group_barrier(0x100, 4, id);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, id);
#pragma unroll
        for (int i = 0; i < NKC; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, id);
            if (i + kAhead < NKC) __builtin_amdgcn_sched_group_barrier(0x100, 1, id);
            if (pre == 8) __builtin_amdgcn_sched_group_barrier(0x002, kVpS, id);
        }
    };
    auto sched_grads = [&](auto idt, int vpm) __device__ __attribute__((always_inline)) {
        constexpr int id = decltype(idt)::value;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * kTrAhead, id);
#pragma unroll
        for (int i = 0; i < GM; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, id);
            if (i + kTrAhead < GM) __builtin_amdgcn_sched_group_barrier(0x100, 2, id);
            if (vpm == kVpP) __builtin_amdgcn_sched_group_barrier(0x002, kVpP, id);
        }
    };

    // The segment stream of one role.
    auto run = [&](auto role) __device__ __attribute__((always_inline)) {
        constexpr bool PW = decltype(role)::value;
        bf16x8 op[2];                          // P wave: bf16 P of block s
        f32x16 pacc;                           // dS wave: dP of block s
        auto segment = [&](int s, auto pos) __device__ __attribute__((always_inline)) {
            using P = decltype(pos);
            // The operand offsets are redefined (no instruction) at every
            // segment, so that stage base + offset is formed per segment and
            // the base folds into the DS instructions' immediate offsets
            // (hoisted out of the loop, each stage would hold its own copy of
            // every offset in VGPRs).
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) asm volatile("" : "+v"(rofs[kc]));
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                for (int db = 0; db < ND; ++db) asm volatile("" : "+v"(tofs[hl][db]));
            uint16_t* sa = stage_ptr(std::integral_constant<int, P::SA>{});
            uint16_t* sb = stage_ptr(std::integral_constant<int, P::SB>{});
            float* pba = (P::SA & 1) ? pb1 : pb0;    // block s's P (by its parity)
            float* pbb = (P::SB & 1) ? pb1 : pb0;    // block s+1's P
            if constexpr (!P::LAST) load_block(s + 3, stage_ptr(std::integral_constant<int, P::SL>{}));
            f32x16 sn;
            // Instruction order (full segments): the score MFMAs with their
            // A operands read kAhead ahead, then the gradient MFMAs with two
            // transposed operands ahead and the wave's vector work between
            // them.  Each phase ends in a scheduling fence.
            constexpr bool FULL = !P::FIRST && !P::LAST;
            if constexpr (PW) {
                // scores of block s+1 | block s's dV and block s+1's P
                float4 l4[4];
                if constexpr (!P::LAST) read_lse(sb, l4);
                if constexpr (!P::LAST) sn = scores(sb);
                if constexpr (FULL) sched_scores(std::integral_constant<int, 0>{}, 4);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!P::FIRST) grads(sa, op);
                if constexpr (!P::LAST)
                    make_p(sn, l4, pbb, s + 1, op, std::integral_constant<bool, P::MASK>{});
                if constexpr (FULL) sched_grads(std::integral_constant<int, 1>{}, kVpP);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                // block s+1's dP and block s's dS | block s's dK
                bf16x8 ds[2];
                float4 p4[4], d4[4];
                if constexpr (!P::FIRST) read_pd(sa, pba, p4, d4);
                if constexpr (!P::LAST) sn = scores(sb);
                if constexpr (!P::FIRST) make_ds(pacc, p4, d4, ds);
                if constexpr (FULL) sched_scores(std::integral_constant<int, 0>{}, 8);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!P::FIRST) grads(sa, ds);
                if constexpr (FULL) sched_grads(std::integral_constant<int, 1>{}, 0);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (!P::LAST) pacc = sn;
            }
            if constexpr (!P::LAST) seg_barrier();
        };
        // segment -1: block 0's scores; block 2 is loaded
        segment(-1, SegPos<3, true, false, CAUSAL>{});
        // segments 0 .. 4 ceil(nb/4) - 1, in groups of four (the segments
        // past nb-1, at most three and none when N is a multiple of 128, work
        // all-zero blocks).  Under the causal mask blocks 0-3 hold queries
        // before some key of the work group: their P, formed in segments -1
        // to 2, is masked; the first group is written out for that.
        segment(0, SegPos<0, false, false, CAUSAL>{});
        segment(1, SegPos<1, false, false, CAUSAL>{});
        segment(2, SegPos<2, false, false, CAUSAL>{});
        segment(3, SegPos<3, false, false>{});
        for (int s = 4; s < nb; s += 4) {
            segment(s, SegPos<0, false, false>{});
            segment(s + 1, SegPos<1, false, false>{});
            segment(s + 2, SegPos<2, false, false>{});
            segment(s + 3, SegPos<3, false, false>{});
        }
    };
    // blocks 0 and 1 in flight, wait for block 0
    load_block(0, st0);
    load_block(1, st1);
    seg_barrier();
    if (pwave) run(std::true_type{});
    else run(std::false_type{});
    __builtin_amdgcn_s_waitcnt(0x0F70);        // the last (repeated) loads have landed

    // epilogue: lane holds key `key`, d = db*32 + 8i + 4g + j in register 4i + j
    store_o_row<ND>((pwave ? dV : dK) + base + (size_t)key * D, acc, pwave ? 1.f : scale, g,
                    key < N);
}

// Causal work balance (both gradient kernels): under the causal mask key
// block b of n meets about n - b query tiles (and query block b about b + 1
// key tiles), so work group p of a head takes blocks p and n-1-p (one block
// when they coincide) and all work groups carry about the same work.
__host__ __device__ constexpr int causal_groups(int n_blocks) { return (n_blocks + 1) / 2; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2)
void bwd_dkdv1_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ stats, uint16_t* __restrict__ dK,
                     uint16_t* __restrict__ dV, int N, int n_kblocks, float scale_log2,
                     float scale) {
    // two stages as separate arrays, so that reads of one stage are known not
    // to alias the asynchronous loads into the other (no wait for those loads)
    __shared__ __attribute__((aligned(1024))) uint16_t smem0[dkdv1_stage_elems<D>()];
    __shared__ __attribute__((aligned(1024))) uint16_t smem1[dkdv1_stage_elems<D>()];

    // work group -> (b*h, p), XCD-aware as in the forward; p is the key block,
    // or under the causal mask the blocks p (the longer) and n-1-p
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    const int per_head = CAUSAL ? causal_groups(n_kblocks) : n_kblocks;
    const int bh = wg / per_head;
    const int p = wg - bh * per_head;
    const int n_blocks = (CAUSAL && p < n_kblocks - 1 - p) ? 2 : 1;
    for (int i = 0; i < n_blocks; ++i) {
        if (i > 0) __syncthreads();            // the first block's last tile is read
        dkdv1_block<D, CAUSAL>(smem0, smem1, Q, K, V, dO, stats, dK, dV, N, scale_log2, scale, bh,
                              (i == 0 ? p : n_kblocks - 1 - p) * BK);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(DKDV_THREADS, 1)
void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ stats, uint16_t* __restrict__ dK,
                     uint16_t* __restrict__ dV, int N, int n_kblocks, float scale_log2,
                     float scale) {
    // four stages and two P buffers, separate arrays, so that reads of one
    // stage are known not to alias the asynchronous loads into another; the
    // stages come first, so that every stage offset fits a DS instruction's
    // 16-bit immediate
    __shared__ __attribute__((aligned(256))) uint16_t st0[dkdv_stage_elems<D>()];
    __shared__ __attribute__((aligned(256))) uint16_t st1[dkdv_stage_elems<D>()];
    __shared__ __attribute__((aligned(256))) uint16_t st2[dkdv_stage_elems<D>()];
    __shared__ __attribute__((aligned(256))) uint16_t st3[dkdv_stage_elems<D>()];
    __shared__ __attribute__((aligned(256))) float pb0[PBUF_FLOATS];
    __shared__ __attribute__((aligned(256))) float pb1[PBUF_FLOATS];

    // work group -> (b*h, p), XCD-aware as in the forward; p is the key block,
    // or under the causal mask the blocks p (the longer) and n-1-p
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    const int per_head = CAUSAL ? causal_groups(n_kblocks) : n_kblocks;
    const int bh = wg / per_head;
    const int p = wg - bh * per_head;
    const int n_blocks = (CAUSAL && p < n_kblocks - 1 - p) ? 2 : 1;
    for (int i = 0; i < n_blocks; ++i) {
        if (i > 0) __syncthreads();            // the first block's last stages are read
        dkdv_block<D, CAUSAL>(st0, st1, st2, st3, pb0, pb1, Q, K, V, dO, stats, dK, dV, N,
                              scale_log2, scale, bh, (i == 0 ? p : n_kblocks - 1 - p) * BK);
    }
}

// ---------------------------------------------------------------------------
// 3. dQ.
// dQ of the BM queries from q0 of head bh.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dq_block(uint16_t* smem0, uint16_t* smem1,
                                         const uint16_t* __restrict__ Q,
                                         const uint16_t* __restrict__ K,
                                         const uint16_t* __restrict__ V,
                                         const uint16_t* __restrict__ dO,
                                         const uint16_t* __restrict__ O,
                                         const float* __restrict__ LSE,
                                         float* __restrict__ stats,
                                         uint16_t* __restrict__ dQ, int N, float scale_log2,
                                         float scale, int bh, int q0) {
    constexpr int TILE = BKV * D;
    constexpr int LPW = TILE * 2 / 1024 / NWAVES;
    constexpr int NKC = D / 16;
    constexpr int ND = D / 32;
    const size_t base = (size_t)bh * (size_t)N * D;
    const uint16_t* __restrict__ Kh = K + base;
    const uint16_t* __restrict__ Vh = V + base;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wq0 = q0 + 32 * wave;
    const int qrow = wq0 + l32;                // this lane's query (MFMA column)

    bf16x8 qop[NKC], doop[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        qop[kc] = row_operand<D>(Q + base, qrow, N, 2 * kc + g, 0u);
        doop[kc] = row_operand<D>(dO + base, qrow, N, 2 * kc + g, 0u);
    }
    // the row's statistics: lse2 = LSE log2(e) and delta = dO . O in fp32,
    // formed once the first K / V tile is in flight (below)
    float lse2 = 0.f, delta = 0.f;
    u32x4 orow[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        orow[kc] = __builtin_bit_cast(u32x4, row_operand<D>(O + base, qrow, N, 2 * kc + g, 0u));
    const float lse_row = LSE[(size_t)bh * N + min(qrow, N - 1)];   // used for rows < N only
    f32x16 dqacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

    int gofs[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) gofs[i] = tile_load_offset<D>(wave * LPW + i, lane);
    auto load_tile = [&](int kt, uint16_t* stage) __device__ __attribute__((always_inline)) {
        const int bytes = N * D * 2;
        const int tb = kt * BKV * D * 2;
        load_tile_lds<LPW>(Kh, bytes, tb, &gofs[0], stage, wave * LPW);
        load_tile_lds<LPW>(Vh, bytes, tb, &gofs[0], stage + TILE, wave * LPW);
    };
    int rofs[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) rofs[kc] = frag_offset<D>(l32, 2 * kc + g);
    int tofs[2][ND];
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int db = 0; db < ND; ++db) tofs[hl][db] = trfrag_offset<D>(lane, hl, db * 32);

    const int n_kt_all = (N + BKV - 1) / BKV;
    const int n_kt = CAUSAL ? min(n_kt_all, (q0 + BM + BKV - 1) / BKV) : n_kt_all;
    const int n_full = CAUSAL ? min(N / BKV, q0 / BKV) : N / BKV;

    auto tile_step = [&](int kt, uint16_t* cur, uint16_t* nxt, auto mask_tag) __device__
        __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (kt + 1 < n_kt) load_tile(kt + 1, nxt);
        const int k0 = kt * BKV;
        if (MASK && CAUSAL && k0 > wq0 + 31) return;      // every key follows every query
        const uint16_t* ks = cur;
        const uint16_t* vs = cur + TILE;

        // S^T = K Q^T and dP^T = V dO^T for two 32-key blocks
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) { sacc[kb][r] = 0.f; pacc[kb][r] = 0.f; }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(ks + kb * 32 * D + rofs[kc]));
                sacc[kb] = mfma(a, qop[kc], sacc[kb]);
                const bf16x8 b = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(vs + kb * 32 * D + rofs[kc]));
                pacc[kb] = mfma(b, doop[kc], pacc[kb]);
            }

        // dS^T; lane holds query qrow and keys k0 + 32kb + 8(r/4) + 4g + r%4
        const int lim = (CAUSAL ? min(N - 1, qrow) : N - 1) - (k0 + 4 * g);
        bf16x8 dsop[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(sacc[kb][r], scale_log2, -lse2));
                if constexpr (MASK)
                    if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) p = 0.f;
                dsop[kb][r >> 3][r & 7] = (__bf16)(p * (pacc[kb][r] - delta));
            }

        // dQ^T += K^T dS^T
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint16_t* kbase = ks + (kb * 32 + cc * 16) * D;
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const bf16x8 a = tr_operand(kbase + tofs[0][db], kbase + tofs[1][db]);
                    dqacc[db] = mfma(a, dsop[kb][cc], dqacc[db]);
                }
            }
    };

    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    uint16_t* const stage0 = smem0;
    uint16_t* const stage1 = smem1;
    load_tile(0, stage0);
    {
        // each lane sums the half of the row its dO fragments hold (elements
        // kc*16 + 8g .. +8), lane l + 32 the other half.  Stored per 32-row
        // block (lse2 of its rows, then delta) for the dK/dV kernel, which
        // runs after this one; rows past N get lse2 = delta = 0, which makes
        // the padded rows of the last Q / dO block contribute exactly zero
        // there (their Q and dO rows are zero as well).
        float dot = 0.f;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            const u32x4 b = __builtin_bit_cast(u32x4, doop[kc]);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                dot = fmaf(__uint_as_float(orow[kc][w] << 16), __uint_as_float(b[w] << 16), dot);
                dot = fmaf(__uint_as_float(orow[kc][w] & 0xFFFF0000u),
                           __uint_as_float(b[w] & 0xFFFF0000u), dot);
            }
        }
        dot += __shfl_xor(dot, 32);
        if (qrow < N) {
            lse2 = lse_row * kLog2e;
            delta = dot;
        }
        const int n_sb = (N + SB - 1) / SB;
        if (g == 0 && qrow / SB < n_sb) {
            float* st = stats + ((size_t)bh * n_sb + qrow / SB) * SB_FLOATS;
            st[qrow % SB] = lse2;
            st[SB + qrow % SB] = delta;
        }
    }
    int kt = 0;
    for (; kt < n_full; kt += 2) {
        tile_step(kt, stage0, stage1, NoMask{});
        if (kt + 1 < n_full) tile_step(kt + 1, stage1, stage0, NoMask{});
    }
    kt = n_full;
    if (kt < n_kt && (kt & 1)) tile_step(kt++, stage1, stage0, Mask{});
    for (; kt < n_kt; kt += 2) {
        tile_step(kt, stage0, stage1, Mask{});
        if (kt + 1 < n_kt) tile_step(kt + 1, stage1, stage0, Mask{});
    }

    store_o_row<ND>(dQ + base + (size_t)qrow * D, dqacc, scale, g, qrow < N);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2)
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const uint16_t* __restrict__ O, const float* __restrict__ LSE,
                   float* __restrict__ stats, uint16_t* __restrict__ dQ, int N,
                   int n_qblocks, float scale_log2, float scale) {
    // two stages (K tile, V tile), separate arrays as in the dK/dV kernel
    __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * BKV * D];
    __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * BKV * D];

    // work group -> (b*h, p); causal: the query blocks n-1-p (the longer) and p
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    const int per_head = CAUSAL ? causal_groups(n_qblocks) : n_qblocks;
    const int bh = wg / per_head;
    const int p = wg - bh * per_head;
    const int first = CAUSAL ? n_qblocks - 1 - p : p;
    const int n_blocks = (CAUSAL && p < first) ? 2 : 1;
    for (int i = 0; i < n_blocks; ++i) {
        if (i > 0) __syncthreads();            // the first block's last tile is read
        dq_block<D, CAUSAL>(smem0, smem1, Q, K, V, dO, O, LSE, stats, dQ, N, scale_log2, scale,
                            bh, (i == 0 ? first : p) * BM);
    }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, int B, int H, int N,
                      float scale, float* stats, hipStream_t stream) {
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k);
    const uint16_t* vp = static_cast<const uint16_t*>(v);
    const uint16_t* op = static_cast<const uint16_t*>(o);
    const uint16_t* gp = static_cast<const uint16_t*>(dout);
    uint16_t* dqp = static_cast<uint16_t*>(dq);
    uint16_t* dkp = static_cast<uint16_t*>(dk);
    uint16_t* dvp = static_cast<uint16_t*>(dv);
    const float* lp = lse;
    const float* sp = stats;
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    const unsigned bh = (unsigned)B * (unsigned)H;

    // dQ first: its prologue stores the row statistics the dK/dV kernel reads
    int n_qblocks = (N + BM - 1) / BM;
    const unsigned g3 = (unsigned)(CAUSAL ? causal_groups(n_qblocks) : n_qblocks);
    void* a3[] = {&qp, &kp, &vp, &gp, &op, &lp, &stats, &dqp, &N, &n_qblocks, &scale_log2, &scale};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<D, CAUSAL>),
                                   dim3(bh * g3), dim3(NTHREADS), a3, 0, stream);
    if (e != hipSuccess) return e;

    int n_kblocks = (N + BK - 1) / BK;
    const unsigned g2 = (unsigned)(CAUSAL ? causal_groups(n_kblocks) : n_kblocks);
    void* a2[] = {&qp, &kp, &vp, &gp, &sp, &dkp, &dvp, &N, &n_kblocks, &scale_log2, &scale};
    if constexpr (D == 64)
        return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv1_kernel<D, CAUSAL>),
                               dim3(bh * g2), dim3(NTHREADS), a2, 0, stream);
    else
        return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, CAUSAL>),
                               dim3(bh * g2), dim3(DKDV_THREADS), a2, 0, stream);
}

}  // namespace

hipError_t fa_launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int H, int N, int d, int causal, float scale, void* workspace,
                              hipStream_t stream) {
    float* stats = static_cast<float*>(workspace);
    if (d == 128)
        return causal ? launch_bwd<128, true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, scale, stats, stream)
                      : launch_bwd<128, false>(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, scale, stats, stream);
    if (d == 64)
        return causal ? launch_bwd<64, true>(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, scale, stats, stream)
                      : launch_bwd<64, false>(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, scale, stats, stream);
    return hipErrorInvalidValue;
}
