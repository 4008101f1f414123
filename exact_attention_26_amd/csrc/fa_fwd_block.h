// fa_fwd_block.h - the bf16 attention forward of one block of 128 query rows
// against one head's keys, for gfx950.  Used by the dense forward
// (fa_fwd_bf16.hip), the paged prefill and the draft-tree verification
// (fa_prefill.hip) and the forward with rotary embeddings (fa_rope.hip); they
// differ only in where the query rows and the K/V tiles live, which a "K/V
// source" (DenseKV, PagedKV) and a few row pointers describe, in the mask
// (none, causal, tree) and in whether the query rows are rotated on load.
//
// Per block: O = softmax(scale * Q K^T) V over the keys each query may see and
// the natural-log log-sum-exp of every row, with the tiled online softmax of
// "Flash Attention" (velog @myungum, section 2 and its pseudocode): key/value
// tiles staged through on-chip memory, a running row maximum and row sum
// rescaling the output accumulator, the score matrix never leaving the chip.
// The work group owns its 128 rows of O ("FlashAttention-2 GPU work
// partitioning", iPLEX blog, section 3).
//
// gfx950 mapping
//  * 32 query rows per wave, 4 or 8 waves per work group (the K/V source's
//    kWaves).  All of a wave's state fits in 256 VGPRs, so two waves share
//    each SIMD and one wave's softmax overlaps the other's MFMAs.
//  * K and V tiles (64 keys) go HBM -> LDS with buffer_load ... lds (no
//    register staging), double-buffered in two separate LDS arrays, one
//    barrier per tile; rows are stored with their 16-byte chunks XOR-swizzled
//    (swz), which makes the K reads and the transposed V reads conflict-free.
//    The next tile's K loads go out at the top of a tile and its V loads
//    after the score MFMAs: the K and V tiles of one index are often a large
//    power of two apart in memory, and requesting both at once made them
//    collide (about 15% slower when K and V sit exactly 64 MiB apart).
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
//    Q in registers as the B operand): a lane holds one query and 16 keys, so
//    row max / row sum are in-lane plus one v_permlane32_swap.
//  * O^T += V^T P^T: the probabilities, converted to bf16, are already the B
//    operand; V^T comes from the row-major V tile via ds_read_b64_tr_b16.
//  * p = 2^(c*s - c*m) with c = |scale| log2(e) in one FMA; the accumulator
//    is rescaled only when a row maximum grows by more than 2^8 (a
//    wave-uniform branch), and normalised once at the end.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_gfx950.h"

namespace fa_gfx950 {

constexpr int kFwdBN = TILE_ROWS;              // keys per tile
constexpr int kFwdWaves = 4;
constexpr int kFwdThreads = kFwdWaves * 64;
constexpr int kFwdBM = kFwdWaves * 32;         // query rows per work group
constexpr float kRescaleThreshold = 8.0f;      // log2 units

template <int D, int W = kFwdWaves>
struct FwdShape {
    static constexpr int TILE = kFwdBN * D;                       // elements per K or V tile
    static constexpr int LPW = TILE * 2 / 1024 / W;               // 1 KiB loads per wave per tensor
    static constexpr int NKC = D / 16;                            // S^T MFMAs along d
    static constexpr int ND = D / 32;                             // 32-row blocks of O^T
};

// K/V of one head stored densely, [rows][D]; tile kt = rows 64kt .. 64kt+63,
// loaded by the W waves of the work group.  Buffer resources span the head,
// so rows past the end arrive as zeros.
template <int D, int W = kFwdWaves>
struct DenseKV {
    static constexpr bool kPaged = false;
    static constexpr int kWaves = W;
    const uint16_t* K;
    const uint16_t* V;
    int len;                                   // keys
    int gofs[FwdShape<D, W>::LPW];             // this lane's byte offset in the tile, per load

    __device__ __forceinline__ void setup(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < FwdShape<D, W>::LPW; ++i)
            gofs[i] = tile_load_offset<D>(wave * FwdShape<D, W>::LPW + i, lane);
    }
    // Issue tile kt's K loads into `stage`.  Returns the tile's pages that
    // must be hidden (none here).
    __device__ __forceinline__ uint32_t load_k(int kt, uint16_t* stage, int wave) {
        constexpr int LPW = FwdShape<D, W>::LPW;
        load_tile_lds<LPW>(K, len * D * 2, kt * kFwdBN * D * 2, &gofs[0], stage, wave * LPW);
        return 0u;
    }
    // Issue tile kt's V loads into `stage` (after load_k of the same tile).
    __device__ __forceinline__ void load_v(int kt, uint16_t* stage, int wave) {
        constexpr int LPW = FwdShape<D, W>::LPW;
        load_tile_lds<LPW>(V, len * D * 2, kt * kFwdBN * D * 2, &gofs[0],
                           stage + FwdShape<D>::TILE, wave * LPW);
    }
};

// K/V of one head of one sequence in a paged cache [num_blocks][H][16][D],
// logical page p of the sequence at physical page table[p].  A 64-key tile is
// 4 pages and wave w loads page w of it (its LPW loads cover exactly 16 rows).
// Slots past the sequence's length are never read (the buffer resource of a
// page ends at its last valid row: the rest arrives as zeros), and a table
// entry outside [0, num_blocks) is not followed: the page arrives as zeros
// and the caller hides its keys.  STREAM: the pages are read by this work
// group only (one block of query rows per sequence and head), so the loads
// are non-temporal; with several query blocks per sequence they are not (the
// blocks re-read the same pages through L2).
template <int D, bool STREAM = false>
struct PagedKV {
    static constexpr bool kPaged = true;
    static constexpr int kWaves = kFwdWaves;   // one page of a tile per wave
    static constexpr int kPage = 16;
    const uint16_t* Kc;
    const uint16_t* Vc;
    const int32_t* table;                      // this sequence's row of the block table
    int64_t num_blocks;
    int64_t page_stride;                       // elements per physical page (H * 16 * D)
    int64_t head_off;                          // elements to this head inside a page (h * 16 * D)
    int len;                                   // keys (cached tokens of the sequence)
    int gofs[FwdShape<D>::LPW];                // byte offset inside this wave's page, per load
    int n_pages;
    int sub;                                   // lane % 4
    // The table entries of the tile load_k loads next, read one call ahead:
    // lane l holds entry 4 kt + l % 4.  A vector load, so that the wait for it
    // is the vmcnt(0) a tile already waits for its K/V loads (a scalar load
    // would be waited with every LDS read of the tile).  Entries past the
    // sequence's last page read that page's entry again (in bounds) and are
    // not used.
    int32_t nidv;

    __device__ __forceinline__ void prefetch(int kt) {
        const int last = max(n_pages - 1, 0);
        nidv = table[min(4 * kt + sub, last)];
    }
    __device__ __forceinline__ void setup(int wave, int lane) {
#pragma unroll
        for (int i = 0; i < FwdShape<D>::LPW; ++i)
            gofs[i] = tile_load_offset<D>(wave * FwdShape<D>::LPW + i, lane) - wave * kPage * D * 2;
        n_pages = (len + kPage - 1) / kPage;
        sub = lane & 3;
        prefetch(0);
    }
    int64_t cur_off = 0;                       // this wave's page of the tile being loaded
    int cur_bytes = 0;
    // Issue tile kt's K loads (kt: 0, then each tile after the one before).
    // Logical page 4 kt + w of the tile is the entry in lane w of nidv; a
    // page past the sequence is not loaded, and one whose entry lies outside
    // [0, num_blocks) is not followed and is reported in the returned mask.
    __device__ __forceinline__ uint32_t load_k(int kt, uint16_t* stage, int wave) {
        constexpr int LPW = FwdShape<D>::LPW;
        uint32_t hide = 0u;
        int64_t mine = -1;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int p = 4 * kt + w;
            const int64_t raw = __builtin_amdgcn_readlane(nidv, w);
            const bool ok = p < n_pages && raw >= 0 && raw < num_blocks;
            if (p < n_pages && !ok) hide |= 1u << w;
            if (w == wave) mine = ok ? raw : -1;
        }
        prefetch(kt + 1);
        const int rows = (mine < 0) ? 0 : min(kPage, len - (4 * kt + wave) * kPage);
        cur_off = (mine < 0 ? 0 : mine) * page_stride + head_off;
        cur_bytes = rows * D * 2;
        load_tile_lds<LPW, STREAM ? kLoadNT : 0>(Kc + cur_off, cur_bytes, 0, &gofs[0], stage, wave * LPW);
        return hide;
    }
    __device__ __forceinline__ void load_v(int kt, uint16_t* stage, int wave) {
        constexpr int LPW = FwdShape<D>::LPW;
        load_tile_lds<LPW, STREAM ? kLoadNT : 0>(Vc + cur_off, cur_bytes, 0, &gofs[0], stage + FwdShape<D>::TILE,
                           wave * LPW);
    }
};

// Waves per work group of the dense forwards: 8 without the mask (256 query
// rows share every K/V tile in LDS: half the HBM -> LDS traffic per flop, one
// work group per CU; measured about 2 % faster than 4), 4 under the causal
// mask (two work groups per CU; with 256-row blocks the diagonal tiles and
// the balance of the grid cost more than the shared tiles save).
template <bool CAUSAL>
__host__ __device__ constexpr int dense_fwd_waves() { return CAUSAL ? 4 : 8; }

// The ping-pong block (fwd_block_pingpong) serves the non-causal dense
// forwards at d = 128: same-box A/B 253-254 -> 246-248 us at B=8 H=16 N=2048;
// at d = 64 it was 8-20 % slower than fwd_block.
template <int D, bool CAUSAL>
__host__ __device__ constexpr bool use_pingpong() { return D == 128 && !CAUSAL; }

// Causal work balance: under the causal mask query block b of n sees about
// b + 1 key tiles, so work group p of a (sequence, head) takes blocks n-1-p
// and p (one block when they coincide); every work group then sees about the
// same number of tiles and no long block is left for the end of the grid.
__host__ __device__ constexpr int causal_groups(int n_qblocks) { return (n_qblocks + 1) / 2; }

// Query rows of the block: row r (0-based in the sequence / head) at
// Q + r * stride; O the same; LSE at lse + r * lse_stride (lse may be null).
struct QRows {
    const uint16_t* Q;
    uint16_t* O;
    float* lse;
    int64_t stride;                            // elements between consecutive rows
    int64_t lse_stride;
    int rows;                                  // valid rows
    // RoPE mode only: cosine / sine tables [positions][D/2] and the position
    // of row 0 (row r is at position pos0 + r)
    const float* rope_cos = nullptr;
    const float* rope_sin = nullptr;
    int pos0 = 0;
};

// Largest draft tree of the tree mode (one 64-bit path mask per node).
constexpr int kMaxTreeNodes = 64;

// Online softmax of one 64-key score tile (masked keys already -inf): the
// tile maximum (in-lane, then the partner lane of the query), a rescale of
// (O, l) only when the row maximum grows by more than the threshold (m_run
// is the reference maximum of O and l), then p = 2^(c*s - c*m) into the bf16
// operand of O^T += V^T P^T and the fp32 row sum.  The maximum and the sum
// run as CH independent chains (CH = 1 or 2 or 4: a single chain waits on
// each dependent result; more chains hold more registers).
template <int ND, int CH = 2>
__device__ __forceinline__ void softmax_tile(f32x16 (&sacc)[2], float& m_run, float& l_run,
                                             f32x16 (&oacc)[ND], bf16x8 (&pop)[2][2], float c,
                                             float tau_raw) {
    static_assert(CH == 1 || CH == 2 || CH == 4, "chains");
    float mq[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) mq[i] = sacc[0][i];
#pragma unroll
    for (int i = CH; i < 32; ++i) mq[i % CH] = fmaxf(mq[i % CH], sacc[i >> 4][i & 15]);
#pragma unroll
    for (int w = CH / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) mq[i] = fmaxf(mq[i], mq[i + w]);
    const float mt = pair_max(mq[0]);
    if (__any(mt > m_run + tau_raw)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
    }
    const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
    constexpr int CS = CH < 2 ? 2 : CH;            // partial sums
    float ps[CS];
#pragma unroll
    for (int i = 0; i < CS; ++i) ps[i] = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(sacc[kb][r], c, -mc));
            ps[r % CS] += p;
            pop[kb][r >> 3][r & 7] = (__bf16)p;
        }
#pragma unroll
    for (int w = CS / 2; w >= 1; w /= 2)
#pragma unroll
        for (int i = 0; i < w; ++i) ps[i] += ps[i + w];
    l_run += ps[0];                                // row sum from the fp32 probabilities
}

// S^T = K Q^T for the tile's two 32-key blocks: K fragments read from the
// swizzled LDS tile `ks`, four reads (DS read, 0x100) kept in flight ahead of
// the MFMAs (0x008).
template <int D>
__device__ __forceinline__ void score_mfmas(f32x16 (&sacc)[2], const uint16_t* ks,
                                            const int* kofs, const bf16x8* qop) {
    constexpr int NKC = FwdShape<D>::NKC;
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
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 2 * NKC - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Query fragments of one lane: row qrow, elements kc*16 + 8g .. +8 for every
// kc, as the B operand of S^T = K Q^T, sign bits flipped by qflip (a negative
// scale); rows past qr.rows are zero.  Branch-free: such rows load the last
// row (qr.rows >= 1 whenever a block runs) and are zeroed afterwards.  ROPE:
// the rows are rotated on load, all table loads in flight together.
template <int D, bool ROPE>
__device__ __forceinline__ void load_q_operand(const QRows& qr, int qrow, int g, uint32_t qflip,
                                               bf16x8* qop) {
    constexpr int NKC = FwdShape<D>::NKC;
    const int qld = min(qrow, qr.rows - 1);
    const uint32_t keep = (qrow < qr.rows) ? 0xFFFFFFFFu : 0u;
    u32x4 xq[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc)
        xq[kc] = *reinterpret_cast<const u32x4*>(qr.Q + qld * qr.stride + kc * 16 + g * 8);
    if constexpr (ROPE) {
        // elements kc*16 + 8g .. +8 are pairs kc*8 + 4g .. +4
        float4 cq[NKC], sq[NKC];
        const int64_t t0 = (int64_t)(qr.pos0 + qld) * (D / 2) + g * 4;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            cq[kc] = *reinterpret_cast<const float4*>(qr.rope_cos + t0 + kc * 8);
            sq[kc] = *reinterpret_cast<const float4*>(qr.rope_sin + t0 + kc * 8);
        }
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) xq[kc] = rotate_pairs(xq[kc], cq[kc], sq[kc]);
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) qop[kc] = __builtin_bit_cast(bf16x8, (xq[kc] & keep) ^ qflip);
}

// One block of 32 x KV::kWaves query rows (one wave per 32 rows) starting at
// row q0.  Causal: row r sees the
// keys 0 .. shift + r (shift = 0 for square attention; for the last n tokens
// of a sequence of kv.len tokens, shift = kv.len - n, however many of those
// n rows are computed).  TREE: the rows
// are the nodes of a draft tree whose K/V are the last `rows` keys; row r
// sees the keys before `shift` (the committed tokens) and the tree keys of
// the nodes on its path from the root, found by walking `parents` (node r's
// parent among the rows, or -1; parents come first).  A row that sees no key
// gets O = 0 and LSE = -inf.  ROPE: the query rows are rotated on load
// (rotate_pairs, consecutive pairs, the angle of the row's position).
template <int D, bool CAUSAL, class KV, bool TREE = false, bool ROPE = false>
__device__ __forceinline__ void fwd_block(uint16_t* smem0, uint16_t* smem1, const QRows& qr,
                                          KV& kv, int q0, int shift, float scale_log2,
                                          const int32_t* parents = nullptr) {
    static_assert(!(CAUSAL && TREE), "the tree mask replaces the causal mask");
    using Sh = FwdShape<D>;
    constexpr int TILE = Sh::TILE;
    constexpr int NKC = Sh::NKC;
    constexpr int ND = Sh::ND;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wq0 = q0 + wave * 32;            // first query row of this wave
    const int qrow = wq0 + l32;                // this lane's query row
    const int N = kv.len;

    // Scores are kept raw: p = 2^(c*s - c*m).  c = 0 (scale 0) is replaced by
    // 2^-100: every finite c*s then rounds to 0 in the exponent, so all visible
    // keys get p = 1 exactly as with c = 0, while hidden keys (s = -inf) still
    // get p = 0 without a separate test.
    const float c = fmaxf(fabsf(scale_log2), 7.888609052210118e-31f);
    const uint32_t qflip = (scale_log2 < 0.f) ? 0x80008000u : 0u;   // fold a negative scale into Q
    const float tau_raw = (c > 0.f) ? kRescaleThreshold / c : __builtin_inff();

    // ---- tiles: causal blocks stop at the last key their last row sees;
    //      tiles before n_full need no mask (every key exists and is seen by
    //      every row of the block)
    const int n_kt_all = (N + kFwdBN - 1) / kFwdBN;
    int n_kt = n_kt_all, n_full = N / kFwdBN;
    if (TREE) n_full = min(n_full, max(shift, 0) / kFwdBN);   // tiles of committed tokens only
    if (CAUSAL) {
        const int last = shift + min(qr.rows, q0 + 32 * KV::kWaves) - 1;   // last key any row sees
        n_kt = last < 0 ? 0 : min(n_kt_all, last / kFwdBN + 1);
        const int first = shift + q0;                             // last key the first row sees
        n_full = first < kFwdBN - 1 ? 0 : min(n_full, (first + 1) / kFwdBN);
    }
    n_full = min(n_full, n_kt);

    // ---- tree mode: the parent indices of the (at most kMaxTreeNodes)
    //      nodes are loaded first, one per lane of the first wave, and staged
    //      in LDS below, so that each row's walk up its path reads LDS rather
    //      than waiting on one global load per step
    int par_mine = -1;
    if constexpr (TREE) {
        if (threadIdx.x < qr.rows && threadIdx.x < kMaxTreeNodes) par_mine = parents[threadIdx.x];
    }

    // ---- the first K/V tile's HBM -> LDS loads go out before anything else,
    //      so their latency overlaps the query loads below
    kv.setup(wave, lane);
    uint32_t hide_next = 0u;                   // pages of the next tile to hide (paged)
    if (n_kt > 0) {
        hide_next = kv.load_k(0, smem0, wave);
        kv.load_v(0, smem0, wave);
    }

    // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
    bf16x8 qop[NKC];
    load_q_operand<D, ROPE>(qr, qrow, g, qflip, qop);

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    // ---- tree mode: bit j of `path` = this row may see tree node j (itself
    //      and its ancestors; the walk ends because parents precede children)
    uint64_t path = 0;
    if constexpr (TREE) {
        __shared__ int par_lds[kMaxTreeNodes];
        if (threadIdx.x < kMaxTreeNodes) par_lds[threadIdx.x] = par_mine;
        // the LDS writes are visible to every wave after this barrier; the
        // tile and query loads in flight are not waited for (no fence: the
        // empty asm statements keep the compiler from moving memory accesses
        // across the barrier)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0xC07F);    // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (qrow < qr.rows && qrow < kMaxTreeNodes) {
            path = 1ull << qrow;
            int cur = qrow;
            int p = par_lds[qrow];
            while (p >= 0 && p < cur) {
                path |= 1ull << p;
                cur = p;
                p = par_lds[p];
            }
        }
    }



    // ---- per-lane LDS offsets (elements) of the MFMA operand reads; the row
    //      offsets 32kb (+16cc, +8) do not change the swizzle, so they and the
    //      stage offset are immediates.
    int kofs[NKC];                             // K fragment, key row l32, chunk 2kc+g
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kofs[kc] = frag_offset<D>(l32, 2 * kc + g);
    int vofs[2][ND];                           // V transpose read, key row 4g+li/4 (+8)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int db = 0; db < ND; ++db) vofs[hl][db] = trfrag_offset<D>(lane, hl, db * 32);

    // ---- one key tile: wait for its loads, sync (all loads landed, everyone
    //      is done with the other buffer), start the next tile's loads into
    //      the other buffer, then scores, online softmax and PV on this one.
    auto tile_step = [&](int kt, uint16_t* cur, uint16_t* nxt, auto mask_tag)
                         __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const uint16_t* ks = cur;
        const uint16_t* vs = cur + TILE;
        const uint32_t hide = hide_next;
        __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): this wave's loads have landed
        __syncthreads();
        if (kt + 1 < n_kt) hide_next = kv.load_k(kt + 1, nxt, wave);
        const int k0 = kt * kFwdBN;
        // a wave with nothing to compute here (no row of it exists, or the tile
        // lies after all of its keys) still issues its share of the next V tile
        if (wq0 >= qr.rows || (MASK && CAUSAL && k0 > shift + wq0 + 31)) {
            if (kt + 1 < n_kt) kv.load_v(kt + 1, nxt, wave);
            return;
        }

        // ---- S^T = K Q^T for 2 blocks of 32 keys
        f32x16 sacc[2];
        score_mfmas<D>(sacc, ks, kofs, qop);
        if (kt + 1 < n_kt) kv.load_v(kt + 1, nxt, wave);   // the next tile's V, staggered

        // ---- online softmax; lane holds query qrow and keys
        //      k0 + 32kb + 8(r/4) + 4g + r%4 (page 2kb + r/8 of the tile)
        if constexpr (KV::kPaged) {
            if (hide != 0u) {                  // rare: a page the table does not resolve
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if ((hide >> (2 * kb + (r >> 3))) & 1u) sacc[kb][r] = kNegInf;
            }
        }
        if constexpr (MASK) {                  // ragged end of the keys or causal diagonal:
            // hide key k0 + 4g + off(kb, r) when it is past this row's last key
            const int lim = (CAUSAL ? min(N - 1, shift + qrow) : N - 1) - (k0 + 4 * g);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = kNegInf;
            if constexpr (TREE) {              // tree keys: only the row's path
                const int t0 = k0 + 4 * g - shift;     // tree node of the lane's first key
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int t = t0 + kb * 32 + 8 * (r >> 2) + (r & 3);
                        if (t >= 0 && (t >= kMaxTreeNodes || !((path >> t) & 1ull)))
                            sacc[kb][r] = kNegInf;
                    }
            }
        }
        bf16x8 pop[2][2];
        softmax_tile<ND>(sacc, m_run, l_run, oacc, pop, c, tau_raw);

        // ---- O^T += V^T P^T.  Fragment for d rows db*32 .. +32 and keys
        //      32kb + 16cc + {4g..4g+3, 8+4g..8+4g+3}: two transpose loads.
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

    // ---- tile loops: unmasked tiles unrolled by two (each body's LDS stage is
    //      named statically), then the few masked tiles (ragged end, causal
    //      diagonal); tile kt lives in stage kt & 1.
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    int kt = 0;
    for (; kt < n_full; kt += 2) {
        tile_step(kt, smem0, smem1, NoMask{});
        if (kt + 1 < n_full) tile_step(kt + 1, smem1, smem0, NoMask{});
    }
    kt = n_full;
    if (kt < n_kt && (kt & 1)) tile_step(kt++, smem1, smem0, Mask{});
    for (; kt < n_kt; kt += 2) {
        tile_step(kt, smem0, smem1, Mask{});
        if (kt + 1 < n_kt) tile_step(kt + 1, smem1, smem0, Mask{});
    }

    // ---- epilogue: O = O_acc / l (bf16, round to nearest even), LSE = ln l + m;
    //      a row that saw no key (l = 0) gets O = 0, LSE = -inf
    const float l_tot = pair_sum(l_run);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    store_o_row<ND>(qr.O + (int64_t)qrow * qr.stride, oacc, inv, g, qrow < qr.rows);
    if (qrow < qr.rows) {
        if (qr.lse != nullptr && g == 0) {
            const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
            qr.lse[qrow * qr.lse_stride] = empty ? kNegInf : (mc + __log2f(l_tot)) * kLn2;
        }
    }
}

// ---- ping-pong block: the non-causal dense forward at d = 128 ----
//
// 256 query rows, 8 waves sharing every K/V tile, as fwd_block with 8 waves,
// but the waves are two groups of four (waves 0-3: A, 4-7: B; every SIMD
// holds one wave of each) that work half a tile apart.  Each wave alternates
//   M(k): O += V_{k-1} P_{k-1}, then S_k = K_k Q^T        (matrix cores, LDS)
//   V(k): online softmax of S_k into P_k                  (vector ALU)
// and the groups run A: M(k) V(k), B: V(k-1) M(k), so in each half of an
// iteration one wave of every SIMD issues MFMAs while the other one computes
// exponentials: the two units overlap instead of both waves of a SIMD
// waiting on the same phase.  Two barriers per iteration keep the groups
// half an iteration apart; scheduling barriers keep the compiler from moving
// MFMAs across them.  K and V tiles have two LDS buffers each: K_k and V_k
// live in buffer k & 1, and the loads of K_{k+1} and V_k go out at the top
// of iteration k, into buffers the previous iteration finished reading.
// Every wave performs the same arithmetic in the same order as fwd_block, so
// the results are bit-identical.  At d = 64 the matrix phase is half as long
// and the barriers cost more than the overlap gains; fwd_block is used there.
template <int D, bool ROPE = false>
__device__ __forceinline__ void fwd_block_pingpong(uint16_t* kb0, uint16_t* kb1, uint16_t* vb0,
                                                   uint16_t* vb1, const QRows& qr,
                                                   const uint16_t* K, const uint16_t* V, int N,
                                                   int q0, float scale_log2) {
    constexpr int W = 8;
    using Sh = FwdShape<D, W>;
    constexpr int NKC = Sh::NKC;
    constexpr int ND = Sh::ND;
    constexpr int LPW = Sh::LPW;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int qrow = q0 + wave * 32 + l32;

    // as in fwd_block: p = 2^(c*s - c*m), c = |scale| log2(e) (2^-100 for 0)
    const float c = fmaxf(fabsf(scale_log2), 7.888609052210118e-31f);
    const uint32_t qflip = (scale_log2 < 0.f) ? 0x80008000u : 0u;
    const float tau_raw = (c > 0.f) ? kRescaleThreshold / c : __builtin_inff();

    const int n_kt = (N + kFwdBN - 1) / kFwdBN;
    const int n_full = N / kFwdBN;             // tiles without keys past the end
    const int bytes = N * D * 2;

    int gofs[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) gofs[i] = tile_load_offset<D>(wave * LPW + i, lane);
    auto load = [&](const uint16_t* X, int kt, uint16_t* dst) __attribute__((always_inline)) {
        load_tile_lds<LPW>(X, bytes, kt * kFwdBN * D * 2, &gofs[0], dst, wave * LPW);
    };

    load(K, 0, kb0);                           // in flight during the query loads

    bf16x8 qop[NKC];
    load_q_operand<D, ROPE>(qr, qrow, g, qflip, qop);

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

    // M(k): O += V_{k-1} P_{k-1} (k >= 1), then S_k = K_k Q^T (k < n_kt).  P
    // is dead before S is started, so the two never hold registers together.
    auto m_phase = [&](int k, const uint16_t* ks, const uint16_t* vs)
                       __attribute__((always_inline)) {
        if (k >= 1) {
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
            // two operands (four transposed reads, DS read 0x100) ahead of the
            // MFMAs (0x008)
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 4 * ND - 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        if (k < n_kt) score_mfmas<D>(sacc, ks, kofs, qop);
    };

    // V(k): online softmax of S_k into P_k (0 <= k < n_kt), as in fwd_block;
    // lane holds query qrow and keys 64k + 32kb + 8(r/4) + 4g + r%4
    auto v_phase = [&](int k) __attribute__((always_inline)) {
        if (k < 0 || k >= n_kt) return;
        if (k >= n_full) {                     // the ragged last tile
            const int lim = N - 1 - (k * kFwdBN + 4 * g);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[kb][r] = kNegInf;
        }
        softmax_tile<ND>(sacc, m_run, l_run, oacc, pop, c, tau_raw);
    };

    // iteration k (k = 0 .. n_kt): loads of K_{k+1} and V_k, then the two
    // halves.  Each group runs its own loop (code of the two orders never
    // meets at a join) and both execute the same barriers; the loop body is
    // unrolled by two so that every LDS buffer is named statically.
    __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): K_0 has landed
    auto iter = [&](auto group_b, int k, uint16_t* kcur, uint16_t* knext, uint16_t* vcur,
                    uint16_t* vprev) __attribute__((always_inline)) {
        constexpr bool B = decltype(group_b)::value;
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();                       // last iteration's reads done, its loads landed
        __builtin_amdgcn_sched_barrier(0);
        if (k + 1 < n_kt) load(K, k + 1, knext);
        if (k < n_kt) load(V, k, vcur);
        if constexpr (!B) m_phase(k, kcur, vprev);
        else v_phase(k - 1);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();          // half an iteration: the groups swap units
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!B) v_phase(k);
        else m_phase(k, kcur, vprev);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): this wave's loads have landed
    };
    if (wave < 4) {
        using GroupA = std::integral_constant<bool, false>;
        for (int k = 0; k <= n_kt; k += 2) {
            iter(GroupA{}, k, kb0, kb1, vb0, vb1);
            if (k + 1 <= n_kt) iter(GroupA{}, k + 1, kb1, kb0, vb1, vb0);
        }
    } else {
        using GroupB = std::integral_constant<bool, true>;
        for (int k = 0; k <= n_kt; k += 2) {
            iter(GroupB{}, k, kb0, kb1, vb0, vb1);
            if (k + 1 <= n_kt) iter(GroupB{}, k + 1, kb1, kb0, vb1, vb0);
        }
    }

    // ---- epilogue, as in fwd_block
    const float l_tot = pair_sum(l_run);
    const bool empty = !(l_tot > 0.f);
    const float inv = empty ? 0.f : 1.0f / l_tot;
    store_o_row<ND>(qr.O + (int64_t)qrow * qr.stride, oacc, inv, g, qrow < qr.rows);
    if (qrow < qr.rows) {
        if (qr.lse != nullptr && g == 0) {
            const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
            qr.lse[qrow * qr.lse_stride] = empty ? kNegInf : (mc + __log2f(l_tot)) * kLn2;
        }
    }
}

}  // namespace fa_gfx950
