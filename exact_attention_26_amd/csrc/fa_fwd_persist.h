// fa_fwd_persist.h - the persistent ping-pong forward (non-causal, d = 128).
//
// The ping-pong block of fa_fwd_block.h (256 query rows, eight waves in two
// groups of four that alternate matrix and vector phases half a tile apart),
// run by one work group per CU over all the blocks it is given, as one stream
// of key tiles.  The per-block arithmetic is that of the single-block code:
// the tiled online softmax of "Flash Attention" (velog @myungum, section 2 and
// its pseudocode), each work group owning its rows of O ("FlashAttention-2 GPU
// work partitioning", iPLEX blog, section 3).
//
// Tile t of the stream is tile t % n_kt of block t / n_kt.  Iteration k:
// the first group's matrix phase (PV of tile k-1, then the scores of tile k,
// one stream of 32 MFMAs) while the second group runs the softmax of tile
// k-1; then the groups swap (one barrier per iteration, at its top: the
// groups keep the offset between their phases by themselves).  What differs
// from one block per work group:
//  - no block start or end stalls the CU: at a block boundary the matrix
//    phase computes the new block's first scores right after the old block's
//    last PV, then finishes the old block (normalise, store O and LSE: the
//    stores drain under the next phases) and resets the accumulator; the new
//    block's query rows were loaded into the operand registers right after
//    the old block's last scores, one iteration ahead;
//  - the K and V tiles are loaded by the first group alone, spread through
//    its MFMA stream, so the softmax waves never stall on a load issue;
//  - the matrix waves raise their priority for their MFMA stream: when both
//    waves of a SIMD are ready, the MFMA issues first and the matrix unit
//    stays busy, the softmax wave filling the cycles in between;
//  - the first and last iterations (no PV, no scores) are peeled, so the
//    middle iterations carry no branch between their products;
//  - a finished block's O goes through LDS (a region per wave), so each
//    store instruction writes whole rows.
#pragma once

#include "fa_fwd_block.h"

namespace fa_gfx950 {

constexpr int kPersistBM = 256;                // query rows per block (8 waves x 32)
// N must be a multiple of the 64-key tile (no tile needs a mask, which keeps
// the loop within its registers); shorter sequences, whose blocks have few
// tiles, run on the per-block grid.
constexpr int kPersistMinTiles = 11;
// LDS of one wave for a finished block's O rows on their way to HBM: 32 rows
// of 256 bytes, each padded to 272 (writes at most two-way bank conflicts)
constexpr int kOStageRow = 272;
constexpr int kOStageBytes = 32 * kOStageRow;

// Work units of a (sequence, head): a block each, or (causal) pairs of a
// long and a short block, (n + 1) / 2 of them.
template <bool CAUSAL>
__host__ __device__ constexpr int units_per_head(int n_qblocks) {
    return CAUSAL ? (n_qblocks + 1) / 2 : n_qblocks;
}

// Units of work group `wg` of `G`: i * G + slot, i = 0, 1, ...  With G a
// multiple of 8, the work groups of one XCD (wg % 8, the hardware's
// round-robin) take a contiguous range of G / 8 blocks in every round, so the
// blocks of a head share that XCD's L2.
__device__ __forceinline__ int persist_slot(int wg, int G) {
    return (G & 7) == 0 ? (wg & 7) * (G >> 3) + (wg >> 3) : wg;
}

// ROPE: the query rows are rotated (rotate_pairs, the angle of the row's
// position in its head) when their block starts; K arrives rotated.
template <int D, bool CAUSAL, bool ROPE = false, int AHEAD = 4>
__device__ __forceinline__ void fwd_pingpong_persistent(
    uint16_t* kb0, uint16_t* kb1, uint16_t* vb0, uint16_t* vb1,
    const uint16_t* Q, const uint16_t* K, const uint16_t* V, uint16_t* O, float* LSE, int N,
    int n_qblocks, int total_units, float scale_log2, uint16_t* ostage,
    const float* rope_cos = nullptr, const float* rope_sin = nullptr) {
    static_assert(D == 128, "the O store path assumes 256-byte rows");
    constexpr int W = 8;
    constexpr int BM = kPersistBM;
    using Sh = FwdShape<D, W>;
    constexpr int NKC = Sh::NKC;
    constexpr int ND = Sh::ND;
    constexpr int LPW = Sh::LPW;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // as in fwd_block: p = 2^(c*s - c*m), c = |scale| log2(e) (2^-100 for 0)
    const float c = fmaxf(fabsf(scale_log2), 7.888609052210118e-31f);
    const uint32_t qflip = (scale_log2 < 0.f) ? 0x80008000u : 0u;
    const float tau_raw = (c > 0.f) ? kRescaleThreshold / c : __builtin_inff();

    const int bytes = N * D * 2;                   // N % 64 == 0
    const int G = gridDim.x;
    const int slot = persist_slot(blockIdx.x, G);
    // work units: non-causal, one block; causal, blocks n_qblocks-1-p and p of
    // a head (one block when they coincide), about the same number of key
    // tiles for every unit.  Unit j of this work group is u = j * G + slot.
    const int per_head = units_per_head<CAUSAL>(n_qblocks);
    const int nu = (slot < total_units) ? (total_units - slot + G - 1) / G : 0;
    if (nu == 0) return;
    // key tiles of query block qb: all of them, or (causal) those up to its
    // last row
    auto tiles_of = [&](int qb) __attribute__((always_inline)) {
        return (CAUSAL ? min(N, (qb + 1) * BM) : N) / kFwdBN;
    };
    // a tile's place in the stream, advanced one tile per iteration
    struct Pos {
        int j;                                     // unit (nu when past the end)
        int m;                                     // block of the unit (causal: 0 long, 1 short)
        int kt;                                    // key tile of the block
        int n_kt;                                  // key tiles of the block
        int q0;                                    // first query row of the block
        int bh;                                    // (b, h) of the block
    };
    // the block of p.j / p.m (past the end: tile 0, 1, ... of head 0, in bounds)
    auto set_block = [&](Pos& p) __attribute__((always_inline)) {
        if (p.j < nu) {
            const int u = p.j * G + slot;
            const int bh = u / per_head;
            const int pp = u - bh * per_head;
            const int qb = (CAUSAL && p.m == 0) ? n_qblocks - 1 - pp : pp;
            p.bh = bh;
            p.q0 = qb * BM;
            p.n_kt = tiles_of(qb);
        } else {
            p.bh = 0;
            p.q0 = 0;
            p.n_kt = 1 << 30;
        }
    };
    auto advance = [&](Pos p) __attribute__((always_inline)) {
        if (++p.kt == p.n_kt) {
            p.kt = 0;
            const int pp = (p.j * G + slot) % per_head;
            if (CAUSAL && p.m == 0 && 2 * pp != n_qblocks - 1) {
                p.m = 1;                           // the short block of the pair
            } else {
                p.m = 0;
                ++p.j;
            }
            set_block(p);
        }
        return p;
    };
    auto head_of = [&](const Pos& p) __attribute__((always_inline)) {
        return (size_t)p.bh * N * D;
    };
    // tiles of the stream
    int T = 0;
    for (int j = 0; j < nu; ++j) {
        const int pp = (j * G + slot) % per_head;
        if (CAUSAL) {
            T += tiles_of(n_qblocks - 1 - pp);
            if (2 * pp != n_qblocks - 1) T += tiles_of(pp);
        } else {
            T += tiles_of(pp);
        }
    }

    // the K and V tiles are loaded by the four waves of the first group
    // alone (2 * LPW regions of each per wave), inside their matrix phase:
    // the softmax waves issue no loads
    constexpr int LPW4 = 2 * LPW;
    int gofs[LPW4];
#pragma unroll
    for (int i = 0; i < LPW4; ++i) gofs[i] = tile_load_offset<D>((wave & 3) * LPW4 + i, lane);
    // the tile at `p` (K or V) into LDS `dst`
    auto load_kv = [&](const uint16_t* X, const Pos& p, uint16_t* dst)
                       __attribute__((always_inline)) {
        load_tile_lds<LPW4>(X + head_of(p), bytes, p.kt * kFwdBN * D * 2, &gofs[0], dst,
                            (wave & 3) * LPW4);
    };
    bf16x8 qop[NKC];
    // the query fragments for this lane of the block at `p`, raw (the sign of
    // a negative scale and rows past N are applied when that block starts),
    // into the registers of the block before, dead after its last scores
    auto load_q_next = [&](const Pos& p) __attribute__((always_inline)) {
        const int row = min(p.q0 + wave * 32 + l32, N - 1);
        const uint16_t* qr = Q + head_of(p) + (size_t)row * D + g * 8;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
            qop[kc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + kc * 16));
    };

    // ---- the first block: K_0 in flight during its query loads
    Pos cur{0, 0, 0, 0, 0, 0};                     // tile k of iteration k
    set_block(cur);
    Pos prv = cur;                                 // tile k - 1
    Pos nxt = advance(cur);                        // tile k + 1
    load_kv(K, cur, kb0);
    {
        QRows qr0;
        qr0.Q = Q + head_of(cur);
        qr0.stride = D;
        qr0.rows = N;
        qr0.rope_cos = rope_cos;
        qr0.rope_sin = rope_sin;
        qr0.pos0 = 0;
        load_q_operand<D, ROPE>(qr0, cur.q0 + wave * 32 + l32, g, qflip, qop);
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    int kofs[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kofs[kc] = frag_offset<D>(l32, 2 * kc + g);
    int vofs[2][ND];
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int db = 0; db < ND; ++db) vofs[hl][db] = trfrag_offset<D>(lane, hl, db * 32);

    f32x16 sacc[2];
    bf16x8 pop[2][2];

    // finish block i: O = O_acc / l, LSE = m + ln l (as in fwd_block)
    auto finish = [&](const Pos& p) __attribute__((always_inline)) {
        const int row = p.q0 + wave * 32 + l32;
        const size_t bh = (size_t)p.bh;
        const float l_tot = pair_sum(l_run);
        if (row < N) {
            const bool empty = !(l_tot > 0.f);
            const float inv = empty ? 0.f : 1.0f / l_tot;
            // through this wave's LDS region (rows padded to 272 bytes), so
            // that each store writes four whole rows: lane (l, g) puts its
            // pieces of row l there, then lane t reads 16 bytes of row
            // 4s + t / 16 for store s.  Stored straight from the registers
            // (8 bytes per lane, 32 rows per instruction) the blocks' O cost
            // 2.5-4 % more time at B=8 H=16 N=2048.
            char* ob = reinterpret_cast<char*>(ostage) + wave * kOStageBytes;
            char* wr = ob + l32 * kOStageRow + 8 * g;
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    *reinterpret_cast<bf16x4*>(wr + (db * 4 + j) * 16) =
                        to_bf16x4(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                                  oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
            const char* rd = ob + (lane >> 4) * kOStageRow + (lane & 15) * 16;
            uint16_t* ost_g = O + (bh * N + p.q0 + wave * 32 + (lane >> 4)) * D + (lane & 15) * 8;
#pragma unroll
            for (int st = 0; st < 8; ++st)
                *reinterpret_cast<u32x4*>(ost_g + 4 * st * D) =
                    *reinterpret_cast<const u32x4*>(rd + 4 * st * kOStageRow);
            if (LSE != nullptr && g == 0) {
                const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
                LSE[bh * N + row] = empty ? kNegInf : (mc + __log2f(l_tot)) * kLn2;
            }
        }
    };

    // PV of the tile in `vs` (probabilities of the tile before)
    auto pv_products = [&](const uint16_t* vs) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint16_t* vb = vs + (kb * 32 + cc * 16) * D;
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const bf16x8 a = tr_operand(vb + vofs[0][db], vb + vofs[1][db]);
                    oacc[db] = mfma(a, pop[kb][cc], oacc[db]);
                }
            }
    };
    // scores of the tile in `ks`
    auto score_products = [&](const uint16_t* ks) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(ks + kb * 32 * D + kofs[kc]));
                sacc[kb] = mfma(a, qop[kc], sacc[kb]);
            }
    };
    constexpr int kPV = 4 * ND;                    // PV products per tile (two reads each)
    constexpr int kS = 2 * NKC;                    // score products per tile (one read each)
    constexpr int kAhead = AHEAD;                  // MFMAs whose operands are read ahead

    // M(k) of a middle iteration, one stream of MFMAs: PV of tile k-1 with
    // four operands (eight transposing reads) in flight, the first four K
    // fragments read under the last PV products, the scores of tile k.  At a
    // block boundary the block that tile k-1 ended is finished after the
    // stream (the scores of the next block do not touch the accumulator).
    auto m_middle = [&](auto with_loads, const uint16_t* ks, const uint16_t* vs, uint16_t* knext,
                        uint16_t* vcur) __attribute__((always_inline)) {
        constexpr bool LD = decltype(with_loads)::value;
        const bool boundary = cur.kt == 0;
        if (boundary && (ROPE || qflip != 0u || cur.q0 + BM > N)) {
            // rare: the rotation, a negative scale, or rows past N in the new
            // block (the rows were loaded from min(row, N - 1))
            const int row = cur.q0 + wave * 32 + l32;
            const uint32_t keep = (row < N) ? 0xFFFFFFFFu : 0u;
            u32x4 xq[NKC];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) xq[kc] = __builtin_bit_cast(u32x4, qop[kc]);
            if constexpr (ROPE) {
                // elements kc*16 + 8g .. +8 are pairs kc*8 + 4g .. +4
                const int64_t t0 = (int64_t)min(row, N - 1) * (D / 2) + g * 4;
                float4 cq[NKC], sq[NKC];
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    cq[kc] = *reinterpret_cast<const float4*>(rope_cos + t0 + kc * 8);
                    sq[kc] = *reinterpret_cast<const float4*>(rope_sin + t0 + kc * 8);
                }
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) xq[kc] = rotate_pairs(xq[kc], cq[kc], sq[kc]);
            }
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
                qop[kc] = __builtin_bit_cast(bf16x8, (xq[kc] & keep) ^ qflip);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the matrix wave of each SIMD issues first when both waves are ready:
        // an MFMA then starts as soon as the unit frees, the softmax wave
        // fills the cycles between
        __builtin_amdgcn_s_setprio(1);
        pv_products(vs);
        score_products(ks);
        if constexpr (LD) {
            load_kv(K, nxt, knext);
            load_kv(V, cur, vcur);
        }
        // reads for MFMA j + kAhead issued right after MFMA j (two per PV
        // product, one per score product); the eight tile loads after PV
        // products 1, 4, 7 and 10
        // (the builtin takes constants only: the branches fold away once the
        // loops are unrolled)
#pragma unroll
        for (int j = 0; j < kAhead; ++j) {
            if (j < kPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int j = 0; j < kPV + kS; ++j) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (j + kAhead < kPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            else if (j + kAhead < kPV + kS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (LD && j < 12 && j % 3 == 1) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        if (boundary) {
            finish(prv);
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
            m_run = kNegInf;
            l_run = 0.f;
        }
        if (cur.kt == cur.n_kt - 1 && nxt.j < nu) load_q_next(nxt);
    };
    // M(0): the scores of the first tile only
    auto m_first = [&](const uint16_t* ks) __attribute__((always_inline)) {
        score_products(ks);
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < kS - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    // M(T): PV of the last tile only
    auto m_last = [&](const uint16_t* vs) __attribute__((always_inline)) {
        pv_products(vs);
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < kPV - 4; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    };
    // V: online softmax of the scores of the tile at `t` (non-causal: every
    // key of every tile exists, N being a multiple of the tile).  Causal: on
    // a tile that reaches past this wave's first row, key k0 + off of the
    // lane's row is hidden when off > row - k0, off = 32kb + 8(r/4) + 4g +
    // r%4 for sacc[kb][r].  The mask is arithmetic, min(s, +-inf) with the
    // sign of lim - off: no compare results to keep in scalar registers.
    auto v_phase = [&](const Pos& t) __attribute__((always_inline)) {
        if constexpr (CAUSAL) {
            const int k0 = t.kt * kFwdBN;
            if (k0 + kFwdBN - 1 > t.q0 + wave * 32) {
                const int lim = (t.q0 + wave * 32 + l32) - (k0 + 4 * g);
                const uint32_t sign = 0x80000000u, inf = 0x7f800000u;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int off = 32 * kb + 8 * (r >> 2) + (r & 3);
                        // s = min(s, +inf or, when lim - off < 0, -inf): the
                        // bound from the sign bit, then the minimum, in one
                        // block the compiler cannot rewrite into a select
                        float out;
                        asm("v_and_or_b32 %0, %1, %2, %3\n\tv_min_f32 %0, %4, %0"
                            : "=&v"(out)
                            : "v"(lim - off), "v"(sign), "v"(inf), "v"(sacc[kb][r]));
                        sacc[kb][r] = out;
                    }
            }
        }
        softmax_tile<ND, 2>(sacc, m_run, l_run, oacc, pop, c, tau_raw);
        // the probabilities and the row sum exist here: without this use the
        // compiler may sink their arithmetic into the next matrix phase,
        // next to the products that read them, which undoes the alternation
        asm volatile("" ::"v"(pop[0][0]), "v"(pop[0][1]), "v"(pop[1][0]), "v"(pop[1][1]),
                     "v"(l_run));
    };

    // iteration k: the first group loads K_{k+1} and V_k (inside its matrix
    // phase, or at its head in the peeled iterations), then the two halves.
    // `stage`: 0 for k = 0 (no PV, group B has no softmax), 1 for 0 < k < T,
    // 2 for k = T (no scores, group A has no softmax).  The loads are issued
    // in every iteration, also past the end of the stream (a position there
    // is tile 0 or 1 of the first head, in bounds, and lands in a buffer
    // nobody reads again), so the middle iterations carry no branch.
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): K_0 has landed
    auto iter = [&](auto group_b, auto stage, uint16_t* kcur, uint16_t* knext, uint16_t* vcur,
                    uint16_t* vprev) __attribute__((always_inline)) {
        constexpr bool B = decltype(group_b)::value;
        constexpr int ST = decltype(stage)::value;
        auto m_phase = [&]() __attribute__((always_inline)) {
            if constexpr (ST == 0) m_first(kcur);
            else if constexpr (ST == 1)
                m_middle(std::integral_constant<bool, !B>{}, kcur, vprev, knext, vcur);
            else m_last(vprev);
        };
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();                           // last iteration's reads done, its loads landed
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!B && ST != 1) {             // loads at the head of the first and last
            load_kv(K, nxt, knext);
            load_kv(V, cur, vcur);
        }
        if constexpr (!B) m_phase();
        else if constexpr (ST != 0) v_phase(prv);  // softmax of tile k-1
        // no barrier between the halves: the top barrier orders every reuse of
        // an LDS buffer, and the groups keep their half-iteration offset by
        // themselves (A starts with its MFMAs, B with its softmax, and the
        // MFMA wave of a SIMD issues first): a barrier here cost 1.5-2.5 %
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!B) {
            if constexpr (ST != 2) v_phase(cur);   // softmax of tile k
        } else {
            m_phase();
        }
        __builtin_amdgcn_sched_barrier(0);
        // the first group: its tile loads (and the next block's query loads,
        // issued with its last scores in the first half) have landed.  The
        // second group issues no tile loads; its query loads (issued at the
        // end of its matrix phase) stay in flight into the next iteration.
        if constexpr (!B) __builtin_amdgcn_s_waitcnt(0x0F70);
        if constexpr (ST != 2) {                   // after the last one prv stays tile T-1
            prv = cur;
            cur = nxt;
            nxt = advance(nxt);
        }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    // k = 0, then 1 .. T-1 two at a time (odd k uses buffers 1), then k = T
    auto run = [&](auto g) __attribute__((always_inline)) {
        iter(g, S0{}, kb0, kb1, vb0, vb1);
        int k = 1;
        for (; k + 1 <= T - 1; k += 2) {
            iter(g, S1{}, kb1, kb0, vb1, vb0);
            iter(g, S1{}, kb0, kb1, vb0, vb1);
        }
        if (k <= T - 1) {
            iter(g, S1{}, kb1, kb0, vb1, vb0);
            ++k;
        }
        if (k & 1) iter(g, S2{}, kb1, kb0, vb1, vb0);
        else iter(g, S2{}, kb0, kb1, vb0, vb1);
    };
    if (wave < 4) run(std::integral_constant<bool, false>{});
    else run(std::integral_constant<bool, true>{});
    finish(prv);                                   // the block of the last tile
}

}  // namespace fa_gfx950
