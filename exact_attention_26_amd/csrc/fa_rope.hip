// fa_rope.hip - rotary position embedding (RoPE) for gfx950, standalone and
// fused into the attention forward.
//
// RoPE ("LLM study notes", DEVOCEAN tech blog, RoPE section) reads a token's
// embedding as complex numbers and rotates them by an angle given by the
// token's absolute position, so that the inner product of a rotated query and
// key depends on their relative position only.  Here the complex numbers are
// consecutive pairs (x[2i], x[2i+1]) and the caller's fp32 tables hold the
// cosine and sine of each (position, pair) angle.
//
// fa_fwd_rope fuses the query rotation into the attention kernel's prologue
// ("LLM study notes", kernel fusion section: fewer global-memory round trips):
// a work group rotates its 128 query rows once, in registers, on load.  The
// keys are rotated once per head by rope_kernel into a workspace: a key tile
// is read by every query block of its head, so rotating it inside the
// attention kernel would repeat the same rotation N/128 times, on the VALU
// that the softmax already saturates.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_fwd_block.h"
#include "fa_fwd_persist.h"
#include "fa_kernels.h"

namespace {

using namespace fa_gfx950;

// x, y: [rows][D] bf16, row r at position r % n_pos_rows (the row index within
// its head).  One thread per 16-byte chunk (4 pairs).  y may equal x.
template <int D>
__global__ __launch_bounds__(256)
void rope_kernel(const uint16_t* x, uint16_t* y, const float* __restrict__ rope_cos,
                 const float* __restrict__ rope_sin, int64_t chunks, int n) {
    constexpr int CPR = D / 8;                 // chunks per row
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= chunks) return;
    const int64_t row = c / CPR;
    const int cc = (int)(c - row * CPR);
    const int pos = (int)(row % n);
    const int64_t t = (int64_t)pos * (D / 2) + cc * 4;
    const u32x4 v = reinterpret_cast<const u32x4*>(x)[c];
    reinterpret_cast<u32x4*>(y)[c] =
        rotate_pairs(v, *reinterpret_cast<const float4*>(rope_cos + t),
                     *reinterpret_cast<const float4*>(rope_sin + t));
}

// The dense forward with the query rotation fused (K already rotated).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * dense_fwd_waves<CAUSAL>(), 8 / dense_fwd_waves<CAUSAL>())
void fwd_rope_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                          float* __restrict__ LSE, const float* __restrict__ rope_cos,
                          const float* __restrict__ rope_sin, int N, int n_qblocks,
                          float scale_log2) {
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    const int per_head = CAUSAL ? causal_groups(n_qblocks) : n_qblocks;
    const int bh = wg / per_head;
    const int p = wg - bh * per_head;
    const size_t base = (size_t)bh * (size_t)N * D;

    constexpr int W = dense_fwd_waves<CAUSAL>();
    constexpr int BM = 32 * W;                 // query rows per block
    constexpr int TILE = FwdShape<D>::TILE;
    QRows qr;
    qr.Q = Q + base;
    qr.O = O + base;
    qr.lse = LSE != nullptr ? LSE + (size_t)bh * N : nullptr;
    qr.stride = D;
    qr.lse_stride = 1;
    qr.rows = N;
    qr.rope_cos = rope_cos;
    qr.rope_sin = rope_sin;
    qr.pos0 = 0;
    if constexpr (use_pingpong<D, CAUSAL>()) {
        __shared__ __attribute__((aligned(1024))) uint16_t kb0[TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t kb1[TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t vb0[TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t vb1[TILE];
        fwd_block_pingpong<D, true>(kb0, kb1, vb0, vb1, qr, K + base, V + base, N, p * BM,
                                    scale_log2);
    } else {
        __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * TILE];
        __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * TILE];
        DenseKV<D, W> kv;
        kv.K = K + base;
        kv.V = V + base;
        kv.len = N;
        // causal: the blocks n_qblocks-1-p and p (causal_groups)
        const int qb_first = CAUSAL ? n_qblocks - 1 - p : p;
        const int n_blocks = (CAUSAL && p < qb_first) ? 2 : 1;
        for (int i = 0; i < n_blocks; ++i) {
            if (i > 0) __syncthreads();        // the first block's last tile is read
            fwd_block<D, CAUSAL, DenseKV<D, W>, false, true>(
                smem0, smem1, qr, kv, (i == 0 ? qb_first : p) * BM, 0, scale_log2);
        }
    }
}

// The d = 128 forward with the query rotation fused, as the persistent stream
// (fa_fwd_persist.h): each block's query rows are rotated in registers when
// the block starts.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1)
void fwd_rope_persist_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                             const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                             float* __restrict__ LSE, const float* __restrict__ rope_cos,
                             const float* __restrict__ rope_sin, int N, int n_qblocks,
                             int total_units, float scale_log2) {
    constexpr int TILE = FwdShape<D>::TILE;
    __shared__ __attribute__((aligned(1024))) uint16_t kb0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t kb1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vb0[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t vb1[TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t ost[8 * kOStageBytes / 2];
    fwd_pingpong_persistent<D, CAUSAL, true>(kb0, kb1, vb0, vb1, Q, K, V, O, LSE, N, n_qblocks,
                                             total_units, scale_log2, ost, rope_cos, rope_sin);
}

template <int D>
hipError_t launch_rope(const void* x, void* y, const float* c, const float* s, int64_t rows,
                       int n, hipStream_t stream) {
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    uint16_t* yp = static_cast<uint16_t*>(y);
    int64_t chunks = rows * (D / 8);
    void* args[] = {&xp, &yp, (void*)&c, (void*)&s, &chunks, &n};
    return hipLaunchKernel(reinterpret_cast<const void*>(&rope_kernel<D>),
                           dim3((unsigned)((chunks + 255) / 256)), dim3(256), args, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_fwd_persist(const void* q, const void* k, const void* v, void* o, float* lse,
                              const float* c, const float* s, int B, int H, int N, float scale,
                              hipStream_t stream) {
    const int n_qblocks = (N + kPersistBM - 1) / kPersistBM;
    const int total = B * H * units_per_head<CAUSAL>(n_qblocks);
    const int grid = total < fa_cu_count() ? total : fa_cu_count();
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k);
    const uint16_t* vp = static_cast<const uint16_t*>(v);
    uint16_t* op = static_cast<uint16_t*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, &op, &lse, (void*)&c, (void*)&s, &N, (void*)&n_qblocks,
                    (void*)&total, &scale_log2};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_rope_persist_kernel<D, CAUSAL>),
                           dim3(grid), dim3(512), args, 0, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      const float* c, const float* s, int B, int H, int N, float scale,
                      hipStream_t stream) {
    constexpr int W = dense_fwd_waves<CAUSAL>();
    const int n_qblocks = (N + 32 * W - 1) / (32 * W);
    const int per_head = CAUSAL ? causal_groups(n_qblocks) : n_qblocks;
    const unsigned nwg = (unsigned)B * (unsigned)H * (unsigned)per_head;
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k);
    const uint16_t* vp = static_cast<const uint16_t*>(v);
    uint16_t* op = static_cast<uint16_t*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, &op, &lse, (void*)&c, (void*)&s, &N, (void*)&n_qblocks,
                    &scale_log2};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_rope_bf16_kernel<D, CAUSAL>),
                           dim3(nwg), dim3(64 * W), args, 0, stream);
}

}  // namespace

hipError_t fa_launch_rope(const void* x, void* out, const float* rope_cos, const float* rope_sin,
                          int B, int H, int N, int d, hipStream_t stream) {
    const int64_t rows = (int64_t)B * H * N;
    if (d == 128) return launch_rope<128>(x, out, rope_cos, rope_sin, rows, N, stream);
    if (d == 64) return launch_rope<64>(x, out, rope_cos, rope_sin, rows, N, stream);
    return hipErrorInvalidValue;
}

hipError_t fa_launch_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                              const float* rope_cos, const float* rope_sin, int B, int H, int N,
                              int d, int causal, float scale, void* workspace,
                              hipStream_t stream) {
    hipError_t e = fa_launch_rope(k, workspace, rope_cos, rope_sin, B, H, N, d, stream);
    if (e != hipSuccess) return e;
    if (d == 128) {
        // the persistent stream as in the plain forward (no ragged tile; short
        // sequences stay on the per-block grid)
        if (N % kFwdBN == 0 && N >= kPersistMinTiles * kFwdBN)
            return causal ? launch_fwd_persist<128, true>(q, workspace, v, o, lse, rope_cos,
                                                          rope_sin, B, H, N, scale, stream)
                          : launch_fwd_persist<128, false>(q, workspace, v, o, lse, rope_cos,
                                                           rope_sin, B, H, N, scale, stream);
        return causal ? launch_fwd<128, true>(q, workspace, v, o, lse, rope_cos, rope_sin, B, H,
                                              N, scale, stream)
                      : launch_fwd<128, false>(q, workspace, v, o, lse, rope_cos, rope_sin, B, H,
                                               N, scale, stream);
    }
    if (d == 64)
        return causal ? launch_fwd<64, true>(q, workspace, v, o, lse, rope_cos, rope_sin, B, H,
                                             N, scale, stream)
                      : launch_fwd<64, false>(q, workspace, v, o, lse, rope_cos, rope_sin, B, H,
                                              N, scale, stream);
    return hipErrorInvalidValue;
}
