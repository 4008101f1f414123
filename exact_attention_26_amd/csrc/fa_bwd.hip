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
// Three launches, no atomics, so results are deterministic:
//  1. bwd_prep_kernel: per 64-row tile of a head, lse2 = LSE log2(e) and
//     delta, into a small workspace (1 KiB per tile: one LDS DMA load).
//  2. bwd_dkdv_kernel: a work group owns 128 keys (32 per wave, K and V rows
//     held in registers as MFMA B operands) and streams 64-row Q / dO tiles
//     through LDS (double-buffered, HBM -> LDS without registers).  Per tile a
//     wave computes S = Q K^T and dP = dO V^T (lane = one key, 16 queries per
//     32-row block), P and dS in registers, then dV^T += dO^T P and
//     dK^T += Q^T dS with the transposed operands read by ds_read_b64_tr_b16.
//  3. bwd_dq_kernel: a work group owns 128 queries (32 per wave, Q and dO rows
//     in registers) and streams K / V tiles, as the forward does: S^T = K Q^T,
//     dP^T = V dO^T (lane = one query, so lse2 and delta are per-lane scalars),
//     dS^T in registers, dQ^T += K^T dS^T.
// Recomputing S and dP in both (2) and (3) costs 14 N^2 d flops per head
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
constexpr int BQ = 64;                 // query rows per tile in the dK/dV kernel; stats tile
constexpr int BKV = 64;                // key rows per tile in the dQ kernel
constexpr int BK = NWAVES * 32;        // keys per dK/dV work group
constexpr int BM = NWAVES * 32;        // queries per dQ work group
constexpr int STATS_FLOATS = 256;      // per 64-row tile: lse2[64], delta[64], 128 unused

// ---------------------------------------------------------------------------
// 1. Row statistics.  One work group per (b*h, 64-row tile); four lanes per
//    row, each summing a quarter of dO_i . O_i in fp32.  Rows past N get
//    lse2 = delta = 0, which makes the padded rows of the last Q / dO tile
//    contribute exactly zero (their Q and dO rows are zero as well).
template <int D>
__global__ __launch_bounds__(NTHREADS)
void bwd_prep_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
                     const float* __restrict__ LSE, float* __restrict__ stats, int N, int n_tiles) {
    constexpr int PART = D / 4;                // elements per lane
    const int wg = blockIdx.x;
    const int bh = wg / n_tiles;
    const int t = wg - bh * n_tiles;
    const int r = threadIdx.x >> 2;
    const int part = threadIdx.x & 3;
    const int row = t * BQ + r;
    float dot = 0.f, l2 = 0.f;
    if (row < N) {
        const size_t off = ((size_t)bh * N + row) * D + part * PART;
        const u32x4* op = reinterpret_cast<const u32x4*>(O + off);
        const u32x4* gp = reinterpret_cast<const u32x4*>(dO + off);
#pragma unroll
        for (int c = 0; c < PART / 8; ++c) {
            const u32x4 a = op[c];
            const u32x4 b = gp[c];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                dot = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), dot);
                dot = fmaf(__uint_as_float(a[w] & 0xFFFF0000u), __uint_as_float(b[w] & 0xFFFF0000u), dot);
            }
        }
        l2 = LSE[(size_t)bh * N + row] * kLog2e;
    }
    dot += __shfl_xor(dot, 1);
    dot += __shfl_xor(dot, 2);
    if (part == 0) {
        float* st = stats + (size_t)wg * STATS_FLOATS;
        st[r] = l2;
        st[BQ + r] = dot;
    }
}

// ---------------------------------------------------------------------------
// 2. dK, dV.
template <int D>
constexpr int dkdv_stage_elems() {                        // Q, dO, stats (1 KiB), in uint16
    return 2 * BQ * D + 2 * STATS_FLOATS;
}

// dK, dV of the BK keys from k0 of head bh.
template <int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_block(uint16_t* smem0, uint16_t* smem1,
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
    const float* st_h = stats + (size_t)bh * n_qt * STATS_FLOATS;

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
        if (wave == 0) load_kib_lds(st_h, n_qt * STATS_FLOATS * 4, qt * STATS_FLOATS * 4,
                                    stage + 2 * TILE, lane);
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
                const float4 l4 = *reinterpret_cast<const float4*>(sts + 32 * hb + 8 * i + 4 * g);
                const float4 d4 = *reinterpret_cast<const float4*>(sts + BQ + 32 * hb + 8 * i + 4 * g);
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
    if (key < N) {
        uint16_t* dvrow = dV + base + (size_t)key * D;
        uint16_t* dkrow = dK + base + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int col = db * 32 + 8 * i + 4 * g;
                *reinterpret_cast<bf16x4*>(dvrow + col) =
                    to_bf16x4(dvacc[db][4 * i], dvacc[db][4 * i + 1], dvacc[db][4 * i + 2],
                              dvacc[db][4 * i + 3]);
                *reinterpret_cast<bf16x4*>(dkrow + col) =
                    to_bf16x4(scale * dkacc[db][4 * i], scale * dkacc[db][4 * i + 1],
                              scale * dkacc[db][4 * i + 2], scale * dkacc[db][4 * i + 3]);
            }
    }
}

// Causal work balance (both gradient kernels): under the causal mask key
// block b of n meets about n - b query tiles (and query block b about b + 1
// key tiles), so work group p of a head takes blocks p and n-1-p (one block
// when they coincide) and all work groups carry about the same work.
__host__ __device__ constexpr int causal_groups(int n_blocks) { return (n_blocks + 1) / 2; }

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 1)
void bwd_dkdv_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                     const float* __restrict__ stats, uint16_t* __restrict__ dK,
                     uint16_t* __restrict__ dV, int N, int n_kblocks, float scale_log2,
                     float scale) {
    // two stages as separate arrays, so that reads of one stage are known not
    // to alias the asynchronous loads into the other (no wait for those loads)
    __shared__ __attribute__((aligned(1024))) uint16_t smem0[dkdv_stage_elems<D>()];
    __shared__ __attribute__((aligned(1024))) uint16_t smem1[dkdv_stage_elems<D>()];

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
        dkdv_block<D, CAUSAL>(smem0, smem1, Q, K, V, dO, stats, dK, dV, N, scale_log2, scale, bh,
                              (i == 0 ? p : n_kblocks - 1 - p) * BK);
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
                                         const float* __restrict__ stats,
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
    float lse2 = 0.f, delta = 0.f;
    if (qrow < N) {
        const float* st = stats + ((size_t)bh * ((N + BQ - 1) / BQ) + qrow / BQ) * STATS_FLOATS;
        lse2 = st[qrow % BQ];
        delta = st[BQ + qrow % BQ];
    }
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

    if (qrow < N) {
        uint16_t* dqrow = dQ + base + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<bf16x4*>(dqrow + db * 32 + 8 * i + 4 * g) =
                    to_bf16x4(scale * dqacc[db][4 * i], scale * dqacc[db][4 * i + 1],
                              scale * dqacc[db][4 * i + 2], scale * dqacc[db][4 * i + 3]);
    }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2)
void bwd_dq_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                   const float* __restrict__ stats, uint16_t* __restrict__ dQ, int N,
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
        dq_block<D, CAUSAL>(smem0, smem1, Q, K, V, dO, stats, dQ, N, scale_log2, scale, bh,
                            (i == 0 ? first : p) * BM);
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

    int n_tiles = (N + BQ - 1) / BQ;
    void* a1[] = {&op, &gp, &lp, &stats, &N, &n_tiles};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_prep_kernel<D>),
                                   dim3(bh * (unsigned)n_tiles), dim3(NTHREADS), a1, 0, stream);
    if (e != hipSuccess) return e;

    int n_kblocks = (N + BK - 1) / BK;
    const unsigned g2 = (unsigned)(CAUSAL ? causal_groups(n_kblocks) : n_kblocks);
    void* a2[] = {&qp, &kp, &vp, &gp, &sp, &dkp, &dvp, &N, &n_kblocks, &scale_log2, &scale};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv_kernel<D, CAUSAL>),
                        dim3(bh * g2), dim3(NTHREADS), a2, 0, stream);
    if (e != hipSuccess) return e;

    int n_qblocks = (N + BM - 1) / BM;
    const unsigned g3 = (unsigned)(CAUSAL ? causal_groups(n_qblocks) : n_qblocks);
    void* a3[] = {&qp, &kp, &vp, &gp, &sp, &dqp, &N, &n_qblocks, &scale_log2, &scale};
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq_kernel<D, CAUSAL>),
                           dim3(bh * g3), dim3(NTHREADS), a3, 0, stream);
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
