// fa_fwd_bf16.hip - bf16 attention forward for gfx950 (MI355X, CDNA4), the hot path.
//
// Computes, per (batch, head), O = softmax(scale * Q K^T) V (optionally causal)
// and the natural-log log-sum-exp of every row, exactly as defined for scaled
// dot-product attention ("LLM study notes", DEVOCEAN tech blog, self-attention
// section), with the tiled online softmax of "Flash Attention" (velog
// @myungum, section 2 and its pseudocode): key/value tiles are staged through
// on-chip memory, a running row maximum and row sum rescale the output
// accumulator, and the score matrix never reaches HBM.  Work is split over
// batch, heads and blocks of query rows and every work group owns its rows of
// O ("FlashAttention-2 GPU work partitioning", iPLEX blog, section 3).
//
// gfx950 design
//  * Work group = 4 waves; each wave owns QS x 32 query rows, and every K/V
//    fragment read from LDS feeds QS matrix instructions.  QS = 1 is what runs:
//    all of a wave's state then fits in 256 VGPRs and two work groups share a
//    CU, so one wave's softmax overlaps the other's MFMAs (QS = 2 halves the
//    LDS reads per flop but needs one wave per SIMD, measured slower).
//  * K and V tiles (64 keys) go HBM -> LDS with global_load_lds_dwordx4 (no
//    register staging), double-buffered: the next tile is in flight while the
//    current one is computed, with one barrier per tile.  Rows are stored with
//    their 16-byte chunks XOR-swizzled by the row index (see swz), which makes
//    both the K reads and the transposed V reads free of LDS bank conflicts.
//  * Scores are computed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16,
//    Q held in registers as the B operand).  In that accumulator layout a lane
//    holds one query and 16 keys, so row max / row sum are in-lane plus one
//    exchange with lane ^ 32 (v_permlane32_swap).
//  * O^T += V^T P^T: the probabilities, converted to bf16, are already the B
//    operand; V^T operands are read straight from the row-major V tile with
//    the gfx950 LDS transpose load (ds_read_b64_tr_b16).  O^T's accumulator
//    again holds one query per lane, so rescaling and 1/l are in-lane.
//  * The exponent is 2^(c*s - c*m) with c = |scale| log2(e) folded into one
//    FMA; the accumulator is rescaled only when a row maximum grows by more
//    than 2^8 (a wave-uniform branch), and normalised once at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_kernels.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BN = 64;           // keys per tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = NWAVES * 64;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;   // log2 units


__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max / sum of x over lanes l and l ^ 32 (result in every lane)
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc *= alpha (the rare rescale path of the online softmax)
__device__ __forceinline__ void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] *= alpha;
}

// Physical 16-byte chunk of logical chunk c in LDS row r.  LDS has 64 banks
// of 4 bytes, i.e. 256-byte lines of 16 chunk slots.  The permutation makes
//  * the K fragment read (16 lanes per cycle, 16 consecutive rows, one chunk)
//  * the V transpose read (32 lanes per cycle, 4 consecutive rows x 4
//    adjacent chunks)
// touch 16 different chunk slots of a line, i.e. all 64 banks once.
// d = 128: one row per line, chunk c in 0..15, XOR with a bit-rotation of r.
// d = 64: two rows per line (slot = 8*(r&1) + chunk), chunk c in 0..7.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// One K tile and one V tile, HBM -> LDS stage (K at stage_base, V after it).
// Buffer resources span the head's rows (bytes = N*D*2); rows past the end are
// out of range and land as zeros.  gofs: this lane's byte offset within the
// tile for each of its LPW 1 KiB loads; tbase: the tile's byte offset.
template <int LPW, int TILE>
__device__ __forceinline__ void load_kv_tile(const uint16_t* Kh, const uint16_t* Vh, int bytes,
                                             int tbase, const int* gofs,
                                             uint16_t* stage_base, int wave) {
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int region = wave * LPW + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(stage_base + region * 512), 16,
                                                 gofs[i], tbase, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)(stage_base + TILE + region * 512),
                                                 16, gofs[i], tbase, 0, 0);
    }
}

template <int D, int QS, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, QS == 1 ? 2 : 1)
void fwd_bf16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                     const uint16_t* __restrict__ V, uint16_t* __restrict__ O,
                     float* __restrict__ LSE, int N, int n_qblocks, float scale_log2) {
    constexpr int BM = NWAVES * 32 * QS;       // query rows per work group
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int TILE = BN * D;               // elements per K or V tile
    constexpr int RPK = 1024 / (D * 2);        // rows per 1 KiB (one wave-wide load)
    constexpr int LPW = TILE * 2 / 1024 / NWAVES;   // wave-wide loads per wave per tensor
    constexpr int NKC = D / 16;                // S^T MFMAs along d
    constexpr int ND = D / 32;                 // 32-row blocks of O^T

    // two stages, each a K tile followed by a V tile.  The stages are separate
    // arrays: the compiler then knows that reads of one stage do not alias the
    // asynchronous HBM -> LDS loads into the other, and does not make them wait
    // for those loads (with one array, every transposed read would wait for
    // the next tile's loads to land).
    __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * TILE];
    __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * TILE];

    // work group -> (batch*head, query block); XCD-aware remap (work groups are
    // dealt round-robin to 8 XCDs: give each XCD a contiguous range so the query
    // blocks of a head share one L2)
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    const int bh = wg / n_qblocks;
    int qb = wg - bh * n_qblocks;
    if (CAUSAL) qb = n_qblocks - 1 - qb;       // longest rows first
    const int q0 = qb * BM;
    const size_t base = (size_t)bh * (size_t)N * D;
    const uint16_t* __restrict__ Qh = Q + base;
    const uint16_t* __restrict__ Kh = K + base;
    const uint16_t* __restrict__ Vh = V + base;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wq0 = q0 + wave * 32 * QS;       // first query row of this wave

    // Scores are kept raw: p = 2^(c*s - c*m).  c = 0 (scale 0) is replaced by
    // 2^-100: every finite c*s then rounds to 0 in the exponent, so all visible
    // keys get p = 1 exactly as with c = 0, while hidden keys (s = -inf) still
    // get p = 0 without a separate test.
    const float c = fmaxf(fabsf(scale_log2), 7.888609052210118e-31f);
    const uint32_t qflip = (scale_log2 < 0.f) ? 0x80008000u : 0u;   // fold a negative scale into Q
    const float tau_raw = (c > 0.f) ? kRescaleThreshold / c : __builtin_inff();

    // ---- Q fragments (B operand of S^T = K Q^T), kept in registers ----
    bf16x8 qop[QS][NKC];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        const int qrow = wq0 + 32 * qs + l32;
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < N) x = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + kc * 16 + g * 8);
            x ^= qflip;
            qop[qs][kc] = __builtin_bit_cast(bf16x8, x);
        }
    }

    f32x16 oacc[QS][ND];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[qs][db][r] = 0.f;
    float m_run[QS], l_run[QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) { m_run[qs] = kNegInf; l_run[qs] = 0.f; }

    const int n_kt_all = (N + BN - 1) / BN;
    const int n_kt = CAUSAL ? min(n_kt_all, (q0 + BM + BN - 1) / BN) : n_kt_all;
    const int n_full = CAUSAL ? min(N / BN, q0 / BN) : N / BN;   // tiles needing no mask

    // ---- HBM -> LDS, one tile: each wave issues LPW 1 KiB loads per tensor;
    //      lane l of a load writes LDS bytes 16l..16l+15 of its 1 KiB region,
    //      i.e. (row, physical chunk) = (region*RPK + l/CPR, l%CPR), and fetches
    //      the logical chunk that belongs there.  The loads go through buffer
    //      resources spanning this head's N rows: rows past N are out of range
    //      and land as zeros (those keys are masked, their V rows get p = 0).
    int gofs[LPW];                             // byte offset within the tile
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int row = (wave * LPW + i) * RPK + lane / CPR;
        gofs[i] = (row * D + swz<D>(row, lane % CPR) * 8) * 2;
    }
    auto load_tile = [&](int kt, uint16_t* stage_base) __device__ __attribute__((always_inline)) {
        load_kv_tile<LPW, TILE>(Kh, Vh, N * D * 2, kt * BN * D * 2, &gofs[0], stage_base, wave);
    };

    // ---- per-lane LDS offsets (elements) of the MFMA operand reads; the
    //      row offsets 32kb (+16cc, +8) do not change the swizzle, so they and
    //      the stage offset are immediates.
    int kofs[NKC];                             // K fragment, key row l32, chunk 2kc+g
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) kofs[kc] = l32 * D + swz<D>(l32, 2 * kc + g) * 8;
    const int h = lane >> 4;
    const int li = lane & 15;
    int vofs[2][ND];                           // V transpose read, key row 4g+li/4 (+8)
#pragma unroll
    for (int hl = 0; hl < 2; ++hl)
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            const int row = 4 * (h >> 1) + (li >> 2) + 8 * hl;
            const int col = db * 32 + 16 * (h & 1) + 4 * (li & 3);
            vofs[hl][db] = row * D + swz<D>(row, col >> 3) * 8 + (col & 7);
        }

    // ---- one key tile: wait for its loads, sync (all loads landed, everyone
    //      is done with the other buffer), start the next tile's loads into the
    //      other buffer, then scores, online softmax and PV on this one.
    auto tile_step = [&](int kt, uint16_t* cur, uint16_t* nxt, auto mask_tag) __device__
        __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const uint16_t* ks = cur;
        const uint16_t* vs = cur + TILE;
        __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0): this wave's loads have landed
        __syncthreads();
        if (kt + 1 < n_kt) load_tile(kt + 1, nxt);
        const int k0 = kt * BN;
        if (MASK && CAUSAL && k0 > wq0 + 32 * QS - 1) return;   // tile above all of this wave's rows

        // ---- S^T = K Q^T for 2 blocks of 32 keys; each K fragment feeds QS MFMAs
        f32x16 sacc[QS][2];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[qs][kb][r] = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const bf16x8 a = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(ks + kb * 32 * D + kofs[kc]));
#pragma unroll
                for (int qs = 0; qs < QS; ++qs)
                    sacc[qs][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[qs][kc],
                                                                           sacc[qs][kb], 0, 0, 0);
            }
        }
        {
            // schedule: keep four K fragment reads (DS read, 0x100) in flight
            // ahead of the score MFMAs (0x008)
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int i = 0; i < 2 * NKC * QS - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }

        // ---- online softmax per query sub-block; lane holds query
        //      wq0 + 32qs + l32 and keys k0 + 32kb + 8(r/4) + 4g + r%4
        bf16x8 pop[QS][2][2];
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) {
            const int qrow = wq0 + 32 * qs + l32;
            if constexpr (MASK) {              // ragged end of N or causal diagonal:
                // hide key k0 + 4g + off(kb, r) when it exceeds this row's last key
                const int lim = (CAUSAL ? min(N - 1, qrow) : N - 1) - (k0 + 4 * g);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * 32 + 8 * (r >> 2) + (r & 3) > lim) sacc[qs][kb][r] = kNegInf;
            }
            float mt = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[qs][kb][r]);
            mt = pair_max(mt);
            if (__any(mt > m_run[qs] + tau_raw)) {
                const float m_new = fmaxf(m_run[qs], mt);
                const float alpha = (m_run[qs] == kNegInf) ? 0.f : fast_exp2((m_run[qs] - m_new) * c);
                l_run[qs] *= alpha;
#pragma unroll
                for (int db = 0; db < ND; ++db) scale_acc(oacc[qs][db], alpha);
                m_run[qs] = m_new;
            }
            const float mc = (m_run[qs] == kNegInf) ? 0.f : m_run[qs] * c;
            float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(sacc[qs][kb][r], c, -mc));
                    if (r & 1) ps1 += p; else ps0 += p;
                    pop[qs][kb][r >> 3][r & 7] = (__bf16)p;
                }
            l_run[qs] += ps0 + ps1;            // row sum from the fp32 probabilities
        }

        // ---- O^T += V^T P^T; each V^T fragment feeds QS MFMAs.  Fragment for
        //      d rows db*32 .. +32 and keys 32kb + 16cc + {4g..4g+3, 8+4g..8+4g+3}:
        //      two transpose loads, lane (16-lane group h, index li) addressing
        //      key row 32kb + 16cc + 4g + li/4 (+8), columns db*32 + 16(h&1) + 4(li&3).
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const uint16_t* vb = vs + (kb * 32 + cc * 16) * D;
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + vofs[0][db]));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb + vofs[1][db]));
                    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo);
                    const u32x2 hi2 = __builtin_bit_cast(u32x2, hi);
                    const u32x4 w = {lo2[0], lo2[1], hi2[0], hi2[1]};
                    const bf16x8 a = __builtin_bit_cast(bf16x8, w);
#pragma unroll
                    for (int qs = 0; qs < QS; ++qs)
                        oacc[qs][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            a, pop[qs][kb][cc], oacc[qs][db], 0, 0, 0);
                }
            }
    };

    // ---- tile loops: unmasked tiles unrolled by two (each body's LDS stage is
    //      an immediate), then the few masked tiles (ragged end, causal diagonal)
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    uint16_t* const stage0 = smem0;
    uint16_t* const stage1 = smem1;
    // tile kt lives in stage kt & 1; every call names its stages statically
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

    // ---- epilogue: O = O_acc / l (bf16, round to nearest even), LSE = ln l + m
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
        const int qrow = wq0 + 32 * qs + l32;
        const float l_tot = pair_sum(l_run[qs]);
        if (qrow < N) {
            const float inv = 1.0f / l_tot;
            uint16_t* orow = O + base + (size_t)qrow * D;
#pragma unroll
            for (int db = 0; db < ND; ++db)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[qs][db][4 * i + j] * inv);
                    *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * i + 4 * g) = w;
                }
            if (LSE != nullptr && g == 0) {
                const float mc = (m_run[qs] == kNegInf) ? 0.f : m_run[qs] * c;
                LSE[(size_t)bh * N + qrow] = (mc + __log2f(l_tot)) * kLn2;
            }
        }
    }
}

template <int D, int QS, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int N, float scale, hipStream_t stream) {
    constexpr int BM = NWAVES * 32 * QS;
    const int n_qblocks = (N + BM - 1) / BM;
    const unsigned nwg = (unsigned)B * (unsigned)H * (unsigned)n_qblocks;
    const uint16_t* qp = static_cast<const uint16_t*>(q);
    const uint16_t* kp = static_cast<const uint16_t*>(k);
    const uint16_t* vp = static_cast<const uint16_t*>(v);
    uint16_t* op = static_cast<uint16_t*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qblocks, &scale_log2};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_bf16_kernel<D, QS, CAUSAL>),
                           dim3(nwg), dim3(NTHREADS), args, 0, stream);
}

}  // namespace



hipError_t fa_launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int d, int causal, float scale,
                              hipStream_t stream) {
    if (d == 128)
        return causal ? launch<128, 1, true>(q, k, v, o, lse, B, H, N, scale, stream)
                      : launch<128, 1, false>(q, k, v, o, lse, B, H, N, scale, stream);
    if (d == 64)
        return causal ? launch<64, 1, true>(q, k, v, o, lse, B, H, N, scale, stream)
                      : launch<64, 1, false>(q, k, v, o, lse, B, H, N, scale, stream);
    return hipErrorInvalidValue;
}
