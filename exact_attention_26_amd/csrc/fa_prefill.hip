// fa_prefill.hip - bf16 prefill of new tokens, and verification of a draft
// token tree, against a paged KV cache, gfx950.
//
// A batch of sequences of different lengths: sequence s has seq_lens[s]
// cached tokens in fixed-size pages reached through its row of the block
// table ("LLM study notes", DEVOCEAN tech blog, section "Paged attention"),
// and its last n_s tokens are new, with their queries packed at rows
// cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1.  Every new query attends to the
// cached tokens it may see (causal: those up to its own position), computed
// FlashAttention-style: paged memory with flash compute, the combination
// "PagedAttention vs FlashAttention: key differences" recommends.  The block
// computation is fwd_block (fa_fwd_block.h) over a paged K/V source: each
// 64-key tile is 4 pages, one per wave, loaded HBM -> LDS through per-page
// buffer resources that end at the sequence's last token.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_block.h"
#include "fa_kernels.h"

namespace {

using namespace fa_gfx950;

// Batches of up to this many sequences are taken heaviest first.
constexpr int kSortedSeqs = kFwdThreads;

// The sequence of rank t among the S <= kSortedSeqs sequences ordered by
// decreasing work of their new rows (ties: lower index first): the
// (query, key) pairs they see, n (2L - n + 1) / 2 under the causal mask, n L
// without, for n new and L cached tokens.  Computed by every work group for
// itself; called by all threads of the group.
template <bool CAUSAL>
__device__ __forceinline__ int seq_by_work_rank(const int32_t* __restrict__ seq_lens,
                                                const int32_t* __restrict__ cu_q, int S,
                                                int max_len, int t, float* key_sh, int* pick) {
    const int i = threadIdx.x;
    float key = 0.f;
    if (i < S) {
        const float L = (float)max(0, min(seq_lens[i], max_len));
        const float n = (float)min(max(0, cu_q[i + 1] - cu_q[i]), max_len);
        key = CAUSAL ? n * (2.f * L - n + 1.f) : n * L;
        key_sh[i] = key;
    }
    __syncthreads();
    if (i < S) {
        int rank = 0;
        for (int j = 0; j < S; ++j) {
            const float v = key_sh[j];
            rank += (v > key || (v == key && j < i)) ? 1 : 0;
        }
        if (rank == t) *pick = i;
    }
    __syncthreads();
    return *pick;
}

// The sequence of rank t among the S <= kSortedSeqs sequences ordered by
// decreasing cached length (ties: lower index first), computed by every work
// group for itself: thread i reads sequence i's length and counts the
// sequences ahead of it.  Called by all threads of the group.
__device__ __forceinline__ int seq_by_length_rank(const int32_t* __restrict__ seq_lens, int S,
                                                  int max_len, int t, int* len_sh, int* pick) {
    const int i = threadIdx.x;
    int len = 0;
    if (i < S) {
        len = max(0, min(seq_lens[i], max_len));
        len_sh[i] = len;
    }
    __syncthreads();
    if (i < S) {
        int rank = 0;
        for (int j = 0; j < S; ++j) {
            const int v = len_sh[j];
            rank += (v > len || (v == len && j < i)) ? 1 : 0;
        }
        if (rank == t) *pick = i;
    }
    __syncthreads();
    return *pick;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kFwdThreads, 2)
void prefill_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                         const uint16_t* __restrict__ Vc, const int32_t* __restrict__ table,
                         const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
                         uint16_t* __restrict__ O, float* __restrict__ LSE, int H, int max_blocks,
                         int64_t num_blocks, int total_q, int n_qblocks, int n_units,
                         float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * FwdShape<D>::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * FwdShape<D>::TILE];

    // work group -> (sequence, head, query block).  Work groups are dealt to
    // the 8 XCDs round-robin (XCD = blockIdx % 8).  Unit u = (sequence of
    // rank u / H, head u % H) goes to XCD u % 8, its query blocks one after
    // another there (they share the unit's K/V through that XCD's L2); so
    // every XCD gets the same share of every sequence, however unequal the
    // sequences are.  The sequences come heaviest first (up to kSortedSeqs of
    // them), so that no long one is left for the end of the grid; causal:
    // longest rows first within a unit.
    __shared__ float key_sh[kSortedSeqs];
    __shared__ int pick;
    const int x = blockIdx.x & 7;
    const int k = blockIdx.x >> 3;             // k-th work group on XCD x
    const int j = k / n_qblocks;
    const int u = 8 * j + x;
    if (u >= n_units) return;                  // padding of the grid
    const int t = u / H;
    const int h = u - t * H;
    const int n_seq = n_units / H;
    const int s = (n_seq <= kSortedSeqs)
                      ? seq_by_work_rank<CAUSAL>(seq_lens, cu_q, n_seq,
                                                 max_blocks * PagedKV<D>::kPage, t, key_sh, &pick)
                      : t;
    int qb = k - j * n_qblocks;
    if (CAUSAL) qb = n_qblocks - 1 - qb;

    // this sequence's new tokens (their positions follow from n_new), of
    // which the rows inside [0, total_q) are computed
    const int qbeg = cu_q[s];
    const int n_new = max(0, cu_q[s + 1] - qbeg);
    int rows = n_new;
    if (qbeg < 0 || qbeg >= total_q) rows = 0;
    rows = max(0, min(rows, total_q - qbeg));
    const int q0 = qb * kFwdBM;
    if (q0 >= rows) return;                    // whole work group: no row here
    const int L = max(0, min(seq_lens[s], max_blocks * PagedKV<D>::kPage));

    PagedKV<D> kv;
    kv.Kc = Kc;
    kv.Vc = Vc;
    kv.table = table + (size_t)s * max_blocks;
    kv.num_blocks = num_blocks;
    kv.page_stride = (int64_t)H * PagedKV<D>::kPage * D;
    kv.head_off = (int64_t)h * PagedKV<D>::kPage * D;
    kv.len = L;
    QRows qr;
    qr.Q = Q + ((int64_t)qbeg * H + h) * D;
    qr.O = O + ((int64_t)qbeg * H + h) * D;
    qr.lse = LSE != nullptr ? LSE + (int64_t)qbeg * H + h : nullptr;
    qr.stride = (int64_t)H * D;
    qr.lse_stride = H;
    qr.rows = rows;
    // the new tokens are the last n_new of the L cached ones; row r stands at
    // position L - n_new + r whether or not later rows are computed
    fwd_block<D, CAUSAL>(smem0, smem1, qr, kv, q0, L - n_new, scale_log2);
}

// Draft-tree verification ("LLM study notes", speculative decoding section:
// the target model computes every node of the draft tree in one pass with
// tree attention): the rows of sequence s are the nodes of its draft tree,
// whose K/V are the last n_s cached tokens; node i sees the committed tokens
// and the nodes on its path from the root.  One work group per (sequence,
// head); at most kMaxTreeNodes nodes, rows past that are not written.
template <int D>
__global__ __launch_bounds__(kFwdThreads, 2)
void tree_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ Kc,
                      const uint16_t* __restrict__ Vc, const int32_t* __restrict__ table,
                      const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cu_q,
                      const int32_t* __restrict__ parents, uint16_t* __restrict__ O,
                      float* __restrict__ LSE, int H, int max_blocks, int64_t num_blocks,
                      int total_q, float scale_log2) {
    __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * FwdShape<D>::TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * FwdShape<D>::TILE];

    __shared__ int len_sh[kSortedSeqs];
    __shared__ int pick;

    // consecutive work groups (the heads of one sequence) go to different
    // XCDs, so every XCD gets the same share of every sequence (nothing is
    // reused across work groups that an L2 could keep), and the sequences
    // come longest first (up to kSortedSeqs of them), so that no long one is
    // left for the end of the grid
    const int n_seq = gridDim.x / H;
    const int t = blockIdx.x / H;
    const int h = blockIdx.x - t * H;
    const int s = (n_seq <= kSortedSeqs)
                      ? seq_by_length_rank(seq_lens, n_seq, max_blocks * PagedKV<D>::kPage, t,
                                           len_sh, &pick)
                      : t;

    // the tree's nodes (their positions follow from n_nodes), of which the
    // first kMaxTreeNodes inside [0, total_q) are computed
    const int qbeg = cu_q[s];
    const int n_nodes = max(0, cu_q[s + 1] - qbeg);
    int rows = n_nodes;
    if (qbeg < 0 || qbeg >= total_q) rows = 0;
    rows = max(0, min(min(rows, total_q - qbeg), kMaxTreeNodes));
    if (rows == 0) return;
    const int L = max(0, min(seq_lens[s], max_blocks * PagedKV<D>::kPage));

    // one work group reads this (sequence, head)'s pages: streaming loads
    PagedKV<D, true> kv;
    kv.Kc = Kc;
    kv.Vc = Vc;
    kv.table = table + (size_t)s * max_blocks;
    kv.num_blocks = num_blocks;
    kv.page_stride = (int64_t)H * PagedKV<D>::kPage * D;
    kv.head_off = (int64_t)h * PagedKV<D>::kPage * D;
    kv.len = L;
    QRows qr;
    qr.Q = Q + ((int64_t)qbeg * H + h) * D;
    qr.O = O + ((int64_t)qbeg * H + h) * D;
    qr.lse = LSE != nullptr ? LSE + (int64_t)qbeg * H + h : nullptr;
    qr.stride = (int64_t)H * D;
    qr.lse_stride = H;
    qr.rows = rows;
    // the tree's K/V are the last n_nodes of the L cached tokens (keys of
    // nodes past kMaxTreeNodes are hidden: no computed node has them on its path)
    fwd_block<D, false, PagedKV<D, true>, true>(smem0, smem1, qr, kv, 0, L - n_nodes, scale_log2,
                                                parents + qbeg);
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* table,
                  const int32_t* seq_lens, const int32_t* cu_q, void* o, float* lse, int S, int H,
                  int max_blocks, int64_t num_blocks, int total_q, int max_q_len, float scale,
                  hipStream_t stream) {
    const int n_qblocks = (max_q_len + kFwdBM - 1) / kFwdBM;
    int n_units = S * H;                       // (sequence, head) pairs, dealt to 8 XCDs
    const unsigned nwg = (unsigned)((n_units + 7) / 8) * 8u * (unsigned)n_qblocks;
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k_cache);
    const uint16_t* vp = static_cast<const uint16_t*>(v_cache);
    uint16_t* op = static_cast<uint16_t*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, (void*)&table, (void*)&seq_lens, (void*)&cu_q, &op, &lse,
                    &H, &max_blocks, &num_blocks, &total_q, (void*)&n_qblocks, &n_units,
                    &scale_log2};
    return hipLaunchKernel(reinterpret_cast<const void*>(&prefill_bf16_kernel<D, CAUSAL>),
                           dim3(nwg), dim3(kFwdThreads), args, 0, stream);
}

}  // namespace

hipError_t fa_launch_tree_decode(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* cu_seqlens_q, const int32_t* parents, void* o,
                                 float* lse, int S, int H, int d, int max_blocks,
                                 int64_t num_blocks, int total_q, float scale,
                                 hipStream_t stream) {
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k_cache);
    const uint16_t* vp = static_cast<const uint16_t*>(v_cache);
    uint16_t* op = static_cast<uint16_t*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, (void*)&block_table, (void*)&seq_lens, (void*)&cu_seqlens_q,
                    (void*)&parents, &op, &lse, &H, &max_blocks, &num_blocks, &total_q,
                    &scale_log2};
    const dim3 grid((unsigned)S * (unsigned)H);
    if (d == 128)
        return hipLaunchKernel(reinterpret_cast<const void*>(&tree_bf16_kernel<128>), grid,
                               dim3(kFwdThreads), args, 0, stream);
    if (d == 64)
        return hipLaunchKernel(reinterpret_cast<const void*>(&tree_bf16_kernel<64>), grid,
                               dim3(kFwdThreads), args, 0, stream);
    return hipErrorInvalidValue;
}

hipError_t fa_launch_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* cu_seqlens_q, void* o, float* lse, int S, int H,
                                   int d, int max_blocks, int64_t num_blocks, int total_q,
                                   int max_q_len, int causal, float scale, hipStream_t stream) {
    if (d == 128)
        return causal ? launch<128, true>(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q,
                                          o, lse, S, H, max_blocks, num_blocks, total_q, max_q_len,
                                          scale, stream)
                      : launch<128, false>(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q,
                                           o, lse, S, H, max_blocks, num_blocks, total_q, max_q_len,
                                           scale, stream);
    if (d == 64)
        return causal ? launch<64, true>(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q,
                                         o, lse, S, H, max_blocks, num_blocks, total_q, max_q_len,
                                         scale, stream)
                      : launch<64, false>(q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q,
                                          o, lse, S, H, max_blocks, num_blocks, total_q, max_q_len,
                                          scale, stream);
    return hipErrorInvalidValue;
}
