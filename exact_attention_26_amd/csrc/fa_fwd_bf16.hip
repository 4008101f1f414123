// fa_fwd_bf16.hip - bf16 attention forward for gfx950 (MI355X, CDNA4), the hot path.
//
// Computes, per (batch, head), O = softmax(scale * Q K^T) V (optionally causal)
// and the natural-log log-sum-exp of every row, exactly as defined for scaled
// dot-product attention ("LLM study notes", DEVOCEAN tech blog, self-attention
// section), with the tiled online softmax of "Flash Attention" (velog
// @myungum, section 2).  Work is split over batch, heads and blocks of 256
// query rows (128 under the causal mask, dense_fwd_waves); every work group
// owns its rows of O ("FlashAttention-2 GPU work partitioning", iPLEX blog,
// section 3).  Under the causal mask a work group takes two blocks, a long
// one and a short one (causal_groups), so that all work groups carry about
// the same number of key tiles.  The block itself is fwd_block
// (fa_fwd_block.h) over a dense K/V source, or, without the mask at d = 128,
// fwd_block_pingpong (its two wave groups alternate matrix and vector work).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_block.h"
#include "fa_fwd_persist.h"
#include "fa_kernels.h"

namespace {

using namespace fa_gfx950;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * dense_fwd_waves<CAUSAL>(), 8 / dense_fwd_waves<CAUSAL>())
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, int N, int n_qblocks, float scale_log2) {
    // work group -> (batch*head, query block); XCD-aware remap (work groups are
    // dealt round-robin to 8 XCDs: give each XCD a contiguous range so the query
    // blocks of a head share one L2)
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    // causal: work group p of a head takes query blocks n_qblocks-1-p and p
    const int per_head = CAUSAL ? causal_groups(n_qblocks) : n_qblocks;
    const int bh = wg / per_head;
    const int p = wg - bh * per_head;
    const size_t base = (size_t)bh * (size_t)N * D;

    constexpr int W = dense_fwd_waves<CAUSAL>();
    constexpr int BM = 32 * W;                 // query rows per block
    QRows qr;
    qr.Q = Q + base;
    qr.O = O + base;
    qr.lse = LSE != nullptr ? LSE + (size_t)bh * N : nullptr;
    qr.stride = D;
    qr.lse_stride = 1;
    qr.rows = N;
    constexpr int TILE = FwdShape<D>::TILE;
    if constexpr (use_pingpong<D, CAUSAL>()) {
        // separate arrays for the two K and two V buffers (the compiler then
        // knows reads of one do not alias loads into another)
        __shared__ __attribute__((aligned(1024))) uint16_t kb0[TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t kb1[TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t vb0[TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t vb1[TILE];
        fwd_block_pingpong<D>(kb0, kb1, vb0, vb1, qr, K + base, V + base, N, p * BM, scale_log2);
    } else {
        // two stages, each a K tile followed by a V tile, as separate arrays
        __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * TILE];
        DenseKV<D, W> kv;
        kv.K = K + base;
        kv.V = V + base;
        kv.len = N;
        if constexpr (!CAUSAL) {
            fwd_block<D, CAUSAL>(smem0, smem1, qr, kv, p * BM, 0, scale_log2);
        } else {
            const int qb_heavy = n_qblocks - 1 - p;
            const int n_blocks = (p < qb_heavy) ? 2 : 1;
            for (int i = 0; i < n_blocks; ++i) {
                if (i > 0) __syncthreads();    // the first block's last tile is read
                fwd_block<D, CAUSAL>(smem0, smem1, qr, kv, (i == 0 ? qb_heavy : p) * BM, 0,
                                     scale_log2);
            }
        }
    }
}

// The d = 128 forward as a persistent grid: one work group per CU walks its
// blocks of 256 query rows as one stream of key tiles (fa_fwd_persist.h).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1)
void fwd_bf16_persist_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                             const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                             float* __restrict__ LSE, int N, int n_qblocks, int total_units,
                             float scale_log2) {
    constexpr int TILE = FwdShape<D>::TILE;
    __shared__ __attribute__((aligned(1024))) uint16_t kb0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t kb1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vb0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vb1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t ost[8 * kOStageBytes / 2];
    fwd_pingpong_persistent<D, CAUSAL, false>(kb0, kb1, vb0, vb1, Q, K, V, O, LSE, N,
                                              n_qblocks, total_units, scale_log2, ost);
}

}  // namespace

// Compute units of the current device (queried once per device).
int fa_cu_count() {
    static int counts[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (counts[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        counts[dev] = n;
    }
    return counts[dev];
}

namespace {

template <int D, bool CAUSAL>
hipError_t launch_persist(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int N, float scale, hipStream_t stream) {
    const int n_qblocks = (N + kPersistBM - 1) / kPersistBM;
    const int total = B * H * units_per_head<CAUSAL>(n_qblocks);
    const int grid = total < fa_cu_count() ? total : fa_cu_count();
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k);
    const uint16_t* vp = static_cast<const uint16_t*>(v);
    uint16_t* op = static_cast<uint16_t*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qblocks, (void*)&total, &scale_log2};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_persist_kernel<D, CAUSAL>),
                           dim3(grid), dim3(512), args, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int N, float scale, hipStream_t stream) {
    constexpr int W = dense_fwd_waves<CAUSAL>();
    const int n_qblocks = (N + 32 * W - 1) / (32 * W);
    const int per_head = CAUSAL ? causal_groups(n_qblocks) : n_qblocks;
    const unsigned nwg = (unsigned)B * (unsigned)H * (unsigned)per_head;
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k);
    const uint16_t* vp = static_cast<const uint16_t*>(v);
    uint16_t* op = static_cast<uint16_t*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qblocks, &scale_log2};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, CAUSAL>),
                           dim3(nwg), dim3(64 * W), args, 0, stream);
}

}  // namespace

hipError_t fa_launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int d, int causal, float scale,
                              hipStream_t stream) {
    if (d == 128) {
        // the persistent stream has no ragged tile; short sequences (blocks
        // of few tiles) stay on the per-block grid
        const bool persist = N % kFwdBN == 0 && N >= kPersistMinTiles * kFwdBN;
        if (causal)
            return persist ? launch_persist<128, true>(q, k, v, o, lse, B, H, N, scale, stream)
                           : launch<128, true>(q, k, v, o, lse, B, H, N, scale, stream);
        return persist ? launch_persist<128, false>(q, k, v, o, lse, B, H, N, scale, stream)
                       : launch<128, false>(q, k, v, o, lse, B, H, N, scale, stream);
    }
    if (d == 64)
        return causal ? launch<64, true>(q, k, v, o, lse, B, H, N, scale, stream)
                      : launch<64, false>(q, k, v, o, lse, B, H, N, scale, stream);
    return hipErrorInvalidValue;
}
