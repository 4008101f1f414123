// fa_decode.hip - paged-KV decode attention for gfx950 (MI355X).
//
// One query token per sequence attends to the KV cache of that sequence.  The
// cache is a pool of fixed-size pages of 16 tokens; a block table maps each
// logical page of a sequence to a physical page, so the tokens of a sequence
// are logically contiguous but physically scattered, and sequences that share
// a prompt list the same physical pages ("LLM study notes", DEVOCEAN tech
// blog, section "Paged attention").  The softmax over the cached tokens is
// computed with the running-maximum rescaling of "Flash Attention" (velog
// @myungum, section 2, pseudocode), so no score vector is ever stored.
//
// Work split (sequence-axis parallelism, "FlashAttention-2 GPU work
// partitioning", iPLEX blog, section 3, change 2, applied to the keys because
// decode has a single query row): one work group per (sequence, head, chunk of
// 32 pages).  Its 4 waves take every 4th page of the chunk; each wave keeps
// its own (m, l, o) in registers and prefetches its next page while it
// computes the current one.  The waves merge through LDS and the work group
// writes one partial (m, l, o) to the workspace; a second kernel merges the
// chunks of each (sequence, head) with the same rescaling rule and normalises.
//
// The path is bound by HBM bandwidth (one multiply-add per byte of K and V):
// a page of one head is 16 rows x d contiguous bf16, read with 16-byte loads,
// one row spread over d/8 lanes; dot products finish with a reduction across
// those lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int PAGE = 16;          // tokens per page
constexpr int SPLIT_PAGES = 32;   // pages per work group (must match fa_validate.h)
constexpr int NWAVES = 4;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void unpack8(const u32x4& w, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

template <int D>
struct PageRegs {
    static constexpr int LPT = D / 8;          // lanes per token row (16 bytes each)
    static constexpr int TPL = 64 / LPT;       // token rows per wave-wide load
    static constexpr int NLD = PAGE / TPL;     // loads per lane per page
    u32x4 k[NLD];
    u32x4 v[NLD];
};

template <int D>
__global__ __launch_bounds__(NWAVES * 64)
void decode_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                           const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
                           const int32_t* __restrict__ lens, float* __restrict__ ws,
                           int H, int max_blocks, long long num_blocks, float scale_log2,
                           int max_splits) {
    using PR = PageRegs<D>;
    constexpr int LPT = PR::LPT, TPL = PR::TPL, NLD = PR::NLD;

    const int split = blockIdx.x;
    const int h = blockIdx.y;
    const int s = blockIdx.z;
    int L = lens[s];
    L = max(0, min(L, max_blocks * PAGE));
    const int n_pages = (L + PAGE - 1) / PAGE;
    const int p_begin = split * SPLIT_PAGES;
    if (p_begin >= n_pages) return;            // this chunk is past the sequence end
    const int p_end = min(n_pages, p_begin + SPLIT_PAGES);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int chunk = lane % LPT;              // which 8 of the d values
    const int tok = lane / LPT;                // row within a wave-wide load

    float qf[8];
    {
        const u32x4 w = *reinterpret_cast<const u32x4*>(q + ((size_t)s * H + h) * D + chunk * 8);
        unpack8(w, qf);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[e] *= scale_log2;
    }

    const int32_t* trow = table + (size_t)s * max_blocks;
    const size_t head_off = (size_t)h * PAGE * D + (size_t)chunk * 8;
    const size_t page_stride = (size_t)H * PAGE * D;

    auto load_page = [&](int p, PR& r, int& valid) {
        const int blk = trow[p];
        const bool ok = (blk >= 0) && ((long long)blk < num_blocks);
        valid = ok ? min(PAGE, L - p * PAGE) : 0;
        const uint16_t* kp = kc + (ok ? (size_t)blk : 0) * page_stride + head_off;
        const uint16_t* vp = vc + (ok ? (size_t)blk : 0) * page_stride + head_off;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int t = i * TPL + tok;
            u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
            if (t < valid) {
                kx = *reinterpret_cast<const u32x4*>(kp + (size_t)t * D);
                vx = *reinterpret_cast<const u32x4*>(vp + (size_t)t * D);
            }
            r.k[i] = kx;
            r.v[i] = vx;
        }
    };

    float m = kNegInf, l = 0.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;

    int p = p_begin + wave;
    PR cur;
    int cur_valid = 0;
    if (p < p_end) load_page(p, cur, cur_valid);
    for (; p < p_end; p += NWAVES) {
        PR nxt;
        int nxt_valid = 0;
        if (p + NWAVES < p_end) load_page(p + NWAVES, nxt, nxt_valid);
        if (cur_valid > 0) {
            float sc[NLD];
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                float kf[8];
                unpack8(cur.k[i], kf);
                float acc = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(qf[e], kf[e], acc);
#pragma unroll
                for (int off = 1; off < LPT; off <<= 1) acc += __shfl_xor(acc, off);
                sc[i] = (i * TPL + tok < cur_valid) ? acc : kNegInf;
            }
            float mt = sc[0];
#pragma unroll
            for (int i = 1; i < NLD; ++i) mt = fmaxf(mt, sc[i]);
#pragma unroll
            for (int off = LPT; off < 64; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
            const float m_new = fmaxf(m, mt);  // finite: token 0 of a page is always valid
            const float alpha = fast_exp2(m - m_new);
            l *= alpha;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
            for (int i = 0; i < NLD; ++i) {
                const float pi = fast_exp2(sc[i] - m_new);
                l += pi;
                float vf[8];
                unpack8(cur.v[i], vf);
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = fmaf(pi, vf[e], o[e]);
            }
            m = m_new;
        }
        cur = nxt;
        cur_valid = nxt_valid;
    }

    // merge the token groups of the wave (lanes with the same chunk)
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
        l += __shfl_xor(l, off);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += __shfl_xor(o[e], off);
    }

    __shared__ float sm[NWAVES], sl[NWAVES];
    __shared__ float so[NWAVES][D];
    if (lane < LPT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) so[wave][chunk * 8 + e] = o[e];
    }
    if (lane == 0) {
        sm[wave] = m;
        sl[wave] = l;
    }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < D) {
        float mm = sm[0];
#pragma unroll
        for (int w = 1; w < NWAVES; ++w) mm = fmaxf(mm, sm[w]);
        float lt = 0.f, ot = 0.f;
#pragma unroll
        for (int w = 0; w < NWAVES; ++w) {
            const float f = (sm[w] == kNegInf) ? 0.f : fast_exp2(sm[w] - mm);
            lt += f * sl[w];
            ot += f * so[w][t];
        }
        float* dst = ws + (((size_t)s * H + h) * max_splits + split) * (D + 2);
        dst[2 + t] = ot;
        if (t == 0) {
            dst[0] = mm;
            dst[1] = lt;
        }
    }
}

template <int D>
__global__ __launch_bounds__(D)
void decode_combine_kernel(const float* __restrict__ ws, const int32_t* __restrict__ lens,
                           uint16_t* __restrict__ o, float* __restrict__ lse, int H,
                           int max_blocks, int max_splits) {
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int t = threadIdx.x;
    int L = lens[s];
    L = max(0, min(L, max_blocks * PAGE));
    const int n_pages = (L + PAGE - 1) / PAGE;
    const int n_splits = (n_pages + SPLIT_PAGES - 1) / SPLIT_PAGES;
    const float* src = ws + ((size_t)s * H + h) * max_splits * (D + 2);
    float mm = kNegInf;
    for (int c = 0; c < n_splits; ++c) mm = fmaxf(mm, src[(size_t)c * (D + 2)]);
    float lt = 0.f, ot = 0.f;
    for (int c = 0; c < n_splits; ++c) {
        const float* part = src + (size_t)c * (D + 2);
        const float mc = part[0];
        const float f = (mc == kNegInf) ? 0.f : fast_exp2(mc - mm);
        lt += f * part[1];
        ot += f * part[2 + t];
    }
    const float out = (lt > 0.f) ? ot / lt : 0.f;
    const __bf16 b = (__bf16)out;
    o[((size_t)s * H + h) * D + t] = __builtin_bit_cast(uint16_t, b);
    if (lse != nullptr && t == 0)
        lse[(size_t)s * H + h] = (lt > 0.f) ? (mm + __log2f(lt)) * kLn2 : kNegInf;
}

template <int D>
hipError_t launch(const void* q, const void* k_cache, const void* v_cache, const int32_t* table,
                  const int32_t* lens, void* o, float* lse, int S, int H, int max_blocks,
                  int64_t num_blocks, float scale, float* ws, hipStream_t stream) {
    const int max_splits = (max_blocks + SPLIT_PAGES - 1) / SPLIT_PAGES;
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k_cache);
    const uint16_t* vp = static_cast<const uint16_t*>(v_cache);
    uint16_t* op = static_cast<uint16_t*>(o);
    long long nb = num_blocks;
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* a1[] = {&qp, &kp, &vp, &table, &lens, &ws, &H, &max_blocks, &nb, &scale_log2,
                  (void*)&max_splits};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_partial_kernel<D>),
                                   dim3(max_splits, H, S), dim3(NWAVES * 64), a1, 0, stream);
    if (e != hipSuccess) return e;
    void* a2[] = {&ws, &lens, &op, &lse, &H, &max_blocks, (void*)&max_splits};
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_combine_kernel<D>),
                           dim3(H, S), dim3(D), a2, 0, stream);
}

}  // namespace

hipError_t fa_launch_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  void* o, float* lse, int S, int H, int d,
                                  int max_blocks, int64_t num_blocks, float scale,
                                  float* workspace, hipStream_t stream) {
    if (d == 128)
        return launch<128>(q, k_cache, v_cache, block_table, seq_lens, o, lse, S, H, max_blocks,
                           num_blocks, scale, workspace, stream);
    if (d == 64)
        return launch<64>(q, k_cache, v_cache, block_table, seq_lens, o, lse, S, H, max_blocks,
                          num_blocks, scale, workspace, stream);
    return hipErrorInvalidValue;
}
