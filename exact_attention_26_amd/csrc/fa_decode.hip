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
// 32 pages).  Its 4 waves take every 4th page of the chunk, two pages in
// flight ahead of the one being computed; every group of d/8 lanes that holds
// one token row keeps its own (m, l, o) in registers.  The row groups and then
// the waves merge, and the work group writes one partial (m, l, o) to the
// workspace; a second kernel merges the chunks of each (sequence, head) with
// the same rescaling rule and normalises.
//
// The path is bound by HBM bandwidth (one multiply-add per byte of K and V):
// a page of one head is 16 rows x d contiguous bf16, read with 16-byte
// non-temporal buffer loads, one row spread over d/8 lanes; dot products
// finish with a DPP reduction across those lanes.  Grid order: the heads of a
// sequence side by side (a physical page holds all heads, H x 4 KiB at
// d = 128, so work groups that run together read neighbouring slices of the
// same pages: 12 % faster than one head's chunks side by side), and every
// sequence's first chunk before any second chunk (sequences that share
// prompt pages read them at about the same time, when the second read can
// still hit in L2: a further 3 %).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_kernels.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int PAGE = 16;          // tokens per page
// Pages per work group: 64 when the grid has enough work groups without
// splitting finer, else 32 (the workspace is sized for 32, the larger count
// of splits; fa_validate.h).  At the 64-sequence bench workload 64-page
// chunks ran 1.5 % faster than 32 (fewer work groups, fewer partials to
// merge); a short batch keeps 32 so that its few sequences still spread over
// the CUs.
constexpr int SPLIT_PAGES_MIN = 32;
constexpr int SPLIT_PAGES_MAX = 64;
constexpr int kMinWorkGroupsForMax = 4096;
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

constexpr int DEPTH = 2;          // pages in flight per wave ahead of the one computed
constexpr int kLoadNT = 2;        // buffer-load cache policy: non-temporal

// Sum over the LPT lanes that hold one token row (a DPP row of 16 lanes, or
// half of one).  Each step adds the value of a partner lane: swaps inside
// quads, then the half-row mirror (pairs quad 0 with 1, 2 with 3) and the row
// mirror (quad 0 with 3, 1 with 2).  Every lane adds the same pairs, so all
// lanes of the group end with bit-identical sums.
template <int LPT>
__device__ __forceinline__ float row_group_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // quad [1,0,3,2]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // quad [2,3,0,1]
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
    if constexpr (LPT == 16)
        x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
    static_assert(LPT == 8 || LPT == 16, "d = 64 or 128");
    return x;
}

template <int D, int SPLIT_PAGES>
__global__ __launch_bounds__(NWAVES * 64)
void decode_partial_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
                           const uint16_t* __restrict__ vc, const int32_t* __restrict__ table,
                           const int32_t* __restrict__ lens, float* __restrict__ ws,
                           int H, int max_blocks, long long num_blocks, float scale_log2,
                           int max_splits) {
    using PR = PageRegs<D>;
    constexpr int LPT = PR::LPT, TPL = PR::TPL, NLD = PR::NLD;

    const int s = blockIdx.x / H;              // heads of a sequence side by side,
    const int h = blockIdx.x - s * H;          // every sequence's chunk 0, then chunk 1, ...
    const int split = blockIdx.y;
    int L = lens[s];
    L = max(0, min(L, max_blocks * PAGE));
    const int n_pages = (L + PAGE - 1) / PAGE;
    const int p_begin = split * SPLIT_PAGES;
    if (p_begin >= n_pages) return;            // this chunk is past the sequence end
    const int p_end = min(n_pages, p_begin + SPLIT_PAGES);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int chunk = lane % LPT;              // which 8 of the d values
    const int tok = lane / LPT;                // row group: rows tok, tok + TPL, ...

    float qf[8];
    {
        const u32x4 w = *reinterpret_cast<const u32x4*>(q + ((size_t)s * H + h) * D + chunk * 8);
        unpack8(w, qf);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[e] *= scale_log2;
    }

    // The wave's pages are p0 + NWAVES i, i < n_my.  Their table entries are
    // fetched once (lane i holds entry i) and read back wave-uniformly.
    const int p0 = p_begin + wave;
    const int n_my = (p_end - p0 + NWAVES - 1) / NWAVES;   // 0..SPLIT_PAGES / NWAVES
    const int32_t* trow = table + (size_t)s * max_blocks;
    const int my_entry = (lane < n_my) ? trow[p0 + NWAVES * lane] : -1;
    const size_t head_off = (size_t)h * PAGE * D;
    const size_t page_stride = (size_t)H * PAGE * D;
    // byte offset of this lane's 16 bytes in row group `tok`, load 0
    const int lane_off = (tok * D + chunk * 8) * 2;

    // Page i of the wave as two buffer resources over exactly its valid rows:
    // rows past seq_len, pages the table does not resolve and the steps past
    // the wave's last page (i >= n_my) read as zeros and touch no memory, so
    // every step issues the same loads.
    auto load_page = [&](int i, PR& r, int& valid) {
        const int blk = __builtin_amdgcn_readlane(my_entry, min(i, SPLIT_PAGES / NWAVES - 1));
        const bool ok = (i < n_my) && (blk >= 0) && ((long long)blk < num_blocks);
        valid = ok ? min(PAGE, L - (p0 + NWAVES * i) * PAGE) : 0;
        const size_t base = ok ? (size_t)blk * page_stride + head_off : 0;
        const int bytes = valid * D * 2;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void*)(kc + base), (short)0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void*)(vc + base), (short)0, bytes, 0x00020000);
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            r.k[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off + j * TPL * D * 2, 0, kLoadNT);
            r.v[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off + j * TPL * D * 2, 0, kLoadNT);
        }
    };

    // per row group: running max m (log2 units, scaled), sum l, output o
    float m = kNegInf, l = 0.f;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;

    auto compute_page = [&](const PR& r, int valid) {
        if (valid <= 0) return;                // wave-uniform
        float sc[NLD];
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            float kf[8];
            unpack8(r.k[i], kf);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(qf[e], kf[e], acc);
            acc = row_group_sum<LPT>(acc);
            sc[i] = (i * TPL + tok < valid) ? acc : kNegInf;
        }
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < NLD; ++i) mt = fmaxf(mt, sc[i]);
        const float m_new = fmaxf(m, mt);
        const float mu = (m_new == kNegInf) ? 0.f : m_new;   // all hidden so far: p = 0
        const float alpha = fast_exp2(m - mu);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const float pi = fast_exp2(sc[i] - mu);
            l += pi;
            float vf[8];
            unpack8(r.v[i], vf);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = fmaf(pi, vf[e], o[e]);
        }
        m = m_new;
    };

    // DEPTH pages in flight ahead of the one computed: a ring of DEPTH + 1
    // register buffers, the loop unrolled over the ring
    if (n_my > 0) {
        PR buf[DEPTH + 1];
        int val[DEPTH + 1];
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) load_page(j, buf[j], val[j]);
        for (int base = 0; base < n_my; base += DEPTH + 1) {
#pragma unroll
            for (int j = 0; j <= DEPTH; ++j) {
                const int jn = (j + DEPTH) % (DEPTH + 1);
                load_page(base + j + DEPTH, buf[jn], val[jn]);
                compute_page(buf[j], val[j]);
            }
        }
    }

    // merge the row groups of the wave (lanes with the same chunk)
    float mw = m;
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) mw = fmaxf(mw, __shfl_xor(mw, off));
    {
        const float f = (m == kNegInf) ? 0.f : fast_exp2(m - mw);
        l *= f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= f;
    }
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
        sm[wave] = mw;
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

template <int D, int SPLIT_PAGES>
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

template <int D, int SPLIT_PAGES>
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
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&decode_partial_kernel<D, SPLIT_PAGES>),
                                   dim3(S * H, max_splits), dim3(NWAVES * 64), a1, 0, stream);
    if (e != hipSuccess) return e;
    void* a2[] = {&ws, &lens, &op, &lse, &H, &max_blocks, (void*)&max_splits};
    return hipLaunchKernel(reinterpret_cast<const void*>(&decode_combine_kernel<D, SPLIT_PAGES>),
                           dim3(H, S), dim3(D), a2, 0, stream);
}

}  // namespace

// Partials of the allocation-free entry point: one array per GPU, held until
// the process ends.  In host code `scratch` is a stand-in, not a device
// address; the kernels get the address hipGetSymbolAddress returns for the
// launching device (scratch_on).
static __device__ __align__(256) float scratch[FA_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the scratch array on the device of `stream`, looked up
// once per device with that device current.
hipError_t scratch_on(hipStream_t stream, float** out) {
    hipDevice_t dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            int cur = 0;
            e = hipGetDevice(&cur);
            if (e != hipSuccess) return e;
            if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            const hipError_t back = (cur != dev) ? hipSetDevice(cur) : hipSuccess;
            if (e != hipSuccess) return e;
            if (back != hipSuccess) return back;
            if (p == nullptr) return hipErrorInvalidSymbol;
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = static_cast<float*>(p);
    return hipSuccess;
}

}  // namespace

hipError_t fa_launch_paged_decode_scratch(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          void* o, float* lse, int S, int H, int d,
                                          int max_blocks, int64_t num_blocks, float scale,
                                          hipStream_t stream) {
    float* ws = nullptr;
    const hipError_t e = scratch_on(stream, &ws);
    if (e != hipSuccess) return e;
    return fa_launch_paged_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse, S, H, d,
                                  max_blocks, num_blocks, scale, ws, stream);
}

hipError_t fa_launch_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  void* o, float* lse, int S, int H, int d,
                                  int max_blocks, int64_t num_blocks, float scale,
                                  float* workspace, hipStream_t stream) {
    const long long wg_max = (long long)S * H *
                             ((max_blocks + SPLIT_PAGES_MAX - 1) / SPLIT_PAGES_MAX);
    const bool big = wg_max >= kMinWorkGroupsForMax;
    if (d == 128)
        return big ? launch<128, SPLIT_PAGES_MAX>(q, k_cache, v_cache, block_table, seq_lens, o,
                                                  lse, S, H, max_blocks, num_blocks, scale,
                                                  workspace, stream)
                   : launch<128, SPLIT_PAGES_MIN>(q, k_cache, v_cache, block_table, seq_lens, o,
                                                  lse, S, H, max_blocks, num_blocks, scale,
                                                  workspace, stream);
    if (d == 64)
        return big ? launch<64, SPLIT_PAGES_MAX>(q, k_cache, v_cache, block_table, seq_lens, o,
                                                 lse, S, H, max_blocks, num_blocks, scale,
                                                 workspace, stream)
                   : launch<64, SPLIT_PAGES_MIN>(q, k_cache, v_cache, block_table, seq_lens, o,
                                                 lse, S, H, max_blocks, num_blocks, scale,
                                                 workspace, stream);
    return hipErrorInvalidValue;
}
