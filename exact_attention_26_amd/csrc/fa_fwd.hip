// fa_fwd.hip - exact attention forward pass for gfx950 (MI355X, CDNA4).
//
// What it computes: for each (batch, head), O = softmax(scale * Q K^T) V with an
// optional causal mask, plus the natural-log log-sum-exp of every row
// ("LLM study notes", DEVOCEAN tech blog, self-attention section; "Flash
// Attention", velog @myungum, sections 1-2).
//
// How (the method of "Flash Attention", velog @myungum, section 2 and its
// pseudocode, in the work split of "FlashAttention-2 GPU work partitioning",
// iPLEX blog, section 3):
//   * one work group owns BM = 128 query rows of one (batch, head) and writes
//     exactly those rows of O; work groups never exchange anything;
//   * the key/value sequence is streamed in tiles of BN = 64 rows through LDS;
//     the next tile's global loads are in flight while the current tile is
//     computed;
//   * per tile the scores are formed by MFMA, a running row maximum m and row
//     sum l are kept in registers and the output accumulator is rescaled by
//     exp(m_old - m_new) whenever the maximum grows, so the N x N score matrix
//     never leaves the chip;
//   * O is normalised by l once, after the last tile (the FlashAttention-2
//     reduction of non-matmul work, same iPLEX page, section 3, change 1);
//     tiles completely above the causal diagonal are skipped and the mask is
//     evaluated only on tiles that straddle it or the ragged end of N.
//
// gfx950 mapping.  Each of the 4 waves owns 32 query rows.  The score tile is
// computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: in the
// accumulator layout of that instruction a lane holds one query column and 16
// key rows, so the row max / row sum of the softmax are in-lane reductions plus
// a single exchange with the partner lane (lane ^ 32).  The same registers,
// converted to bf16, are already the B operand of the next contraction
// O^T += V^T P^T, whose accumulator again holds one query per lane - the
// per-row rescale factor and the final 1/l are in-lane too.  V is written to
// LDS transposed so its A-operand reads are contiguous.
//
// The fp32 instantiation (used for the fp32 smoke configuration) runs the same
// code with v_mfma_f32_32x32x2_f32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_kernels.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128;        // query rows per work group (4 waves x 32)
constexpr int BN = 64;         // keys per tile
constexpr int NTHREADS = 256;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

template <typename T> struct Elem;

template <> struct Elem<__bf16> {
    using op_t = bf16x8;                 // one lane's MFMA operand
    static constexpr int E = 8;          // k-elements per lane per MFMA
    static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Elem<float> {
    using op_t = float;
    static constexpr int E = 1;
    static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// Element e (0..7) of a 16-byte vector holding 8 bf16 values, as raw bits.
__device__ __forceinline__ uint32_t bf16_bits(const u32x4& v, int e) {
    return (v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
}

// Largest growth of the running maximum (in log2 units) absorbed without
// rescaling: the accumulator is rescaled only when a row's maximum grows by
// more than this, so probabilities stay below 2^8 and the usual case (maximum
// unchanged or barely changed) costs no rescale at all.  The result is the
// same: O, l and m always refer to one common reference maximum.
constexpr float kRescaleThreshold = 8.0f;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(NTHREADS, 2)
void fwd_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                T* __restrict__ O, float* __restrict__ LSE, int N, int n_qblocks,
                float scale_log2) {
    using EL = Elem<T>;
    using op_t = typename EL::op_t;
    constexpr int E = EL::E;
    constexpr int KC = 2 * E;                  // contraction length of one MFMA
    constexpr int NKC = D / KC;                // MFMAs along d per 32x32 score block
    constexpr int VEC = 16 / sizeof(T);        // elements per 16-byte vector
    constexpr int CPR = D / VEC;               // 16-byte vectors per row
    constexpr int NV = BN * CPR / NTHREADS;    // consecutive rows per thread per tile
    constexpr int KS = D + VEC;                // K row stride in LDS (16-byte pad)
    constexpr int VS = BN + 4;                 // V^T row stride in LDS
    constexpr int ND = D / 32;                 // 32-row blocks of O^T
    constexpr int NCH = 32 / KC;               // PV MFMAs per 32-key block
    static_assert(NV * NTHREADS == BN * CPR, "tile does not split evenly over threads");
    static_assert(sizeof(T) == 4 ? (NV % 4 == 0) : (NV == 2 || NV == 4),
                  "transposed V store width");

    __shared__ __attribute__((aligned(16))) T Ks[BN * KS];
    __shared__ __attribute__((aligned(16))) T Vt[D * VS];

    // Work group -> (batch*head, query block).  The hardware deals work groups
    // round-robin to the 8 XCDs; remap so each XCD gets a contiguous range of
    // logical ids, i.e. all query blocks of a head share one L2 and its K/V.
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    if ((nwg & 7) == 0) wg = (wg & 7) * (nwg >> 3) + (wg >> 3);
    const int bh = wg / n_qblocks;
    int qb = wg - bh * n_qblocks;
    if (CAUSAL) qb = n_qblocks - 1 - qb;       // longest rows first
    const int q0 = qb * BM;
    const size_t base = (size_t)bh * (size_t)N * D;
    const T* __restrict__ Qh = Q + base;
    const T* __restrict__ Kh = K + base;
    const T* __restrict__ Vh = V + base;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int wq0 = q0 + wave * 32;            // first query row of this wave
    const int qrow = wq0 + l32;                // this lane's query row

    // Scores are kept raw (q.k) and scaled inside the exponent:
    // p = 2^(c*s - c*m) with c = |scale| * log2(e).  A negative scale is folded
    // into Q by flipping its sign bits, which is exact.
    const float c = fabsf(scale_log2);
    const bool neg = scale_log2 < 0.f;
    const float tau_raw = (c > 0.f) ? kRescaleThreshold / c : __builtin_inff();

    // Q fragment of this lane: B operand of S^T = K Q^T, kept in registers.
    op_t qop[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
        if constexpr (E == 8) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (qrow < N) x = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + kc * KC + g * E);
            if (neg) x ^= 0x80008000u;
            qop[kc] = __builtin_bit_cast(bf16x8, x);
        } else {
            const float x = (qrow < N) ? Qh[(size_t)qrow * D + kc * KC + g] : 0.f;
            qop[kc] = neg ? -x : x;
        }
    }

    f32x16 oacc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
    float m_run = kNegInf;                     // running max of raw scores
    float l_run = 0.f;                         // this lane's share of the row sum

    const int n_kt_all = (N + BN - 1) / BN;
    const int n_kt = CAUSAL ? min(n_kt_all, (q0 + BM + BN - 1) / BN) : n_kt_all;
    // tiles before n_full need no mask for any row of this work group
    const int n_full = CAUSAL ? min(N / BN, q0 / BN) : N / BN;

    // global -> register staging of one K/V tile.  K: thread owns NV
    // consecutive rows of one 16-byte column chunk, consecutive threads take
    // consecutive chunks (so a K row is stored as one contiguous LDS run).
    // V: same ownership, but consecutive threads take consecutive groups of
    // rows of one chunk, so the transposed store of a group of lanes fills one
    // contiguous run of a V^T row (no LDS bank conflicts).
    constexpr int RG = BN / NV;                // row groups per tile
    const int kchunk = tid % CPR;
    const int krow0 = (tid / CPR) * NV;
    const int vchunk = tid / RG;
    const int vrow0 = (tid % RG) * NV;
    u32x4 kreg[NV], vreg[NV];
    auto gload = [&](int kt) {
        const int base_row = kt * BN;
        const T* kp = Kh + (size_t)(base_row + krow0) * D + kchunk * VEC;
        const T* vp = Vh + (size_t)(base_row + vrow0) * D + vchunk * VEC;
        if (base_row + BN <= N) {
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                kreg[r] = *reinterpret_cast<const u32x4*>(kp + r * D);
                vreg[r] = *reinterpret_cast<const u32x4*>(vp + r * D);
            }
        } else {
#pragma unroll
            for (int r = 0; r < NV; ++r) {
                u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
                if (base_row + krow0 + r < N) kx = *reinterpret_cast<const u32x4*>(kp + r * D);
                if (base_row + vrow0 + r < N) vx = *reinterpret_cast<const u32x4*>(vp + r * D);
                kreg[r] = kx;
                vreg[r] = vx;
            }
        }
    };

    auto stage = [&]() {
#pragma unroll
        for (int r = 0; r < NV; ++r)
            *reinterpret_cast<u32x4*>(&Ks[(krow0 + r) * KS + kchunk * VEC]) = kreg[r];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            T* dst = &Vt[(vchunk * VEC + e) * VS + vrow0];
            if constexpr (sizeof(T) == 2) {
                // pack element e of consecutive rows: low halves (even e) or
                // high halves (odd e) of word e/2, two rows per 32-bit word
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                const int wd = e >> 1;
                if constexpr (NV == 4) {
                    u32x2 w = {__builtin_amdgcn_perm(vreg[1][wd], vreg[0][wd], sel),
                               __builtin_amdgcn_perm(vreg[3][wd], vreg[2][wd], sel)};
                    *reinterpret_cast<u32x2*>(dst) = w;
                } else {
                    *reinterpret_cast<uint32_t*>(dst) =
                        __builtin_amdgcn_perm(vreg[1][wd], vreg[0][wd], sel);
                }
            } else {
#pragma unroll
                for (int h4 = 0; h4 < NV / 4; ++h4) {
                    u32x4 w = {vreg[4 * h4][e], vreg[4 * h4 + 1][e], vreg[4 * h4 + 2][e],
                               vreg[4 * h4 + 3][e]};
                    *reinterpret_cast<u32x4*>(dst + 4 * h4) = w;
                }
            }
        }
    };

    // One key tile from LDS: scores, online softmax, PV.  MASK selects the
    // variant that hides keys >= N and (causal) keys > query.
    auto compute = [&](auto mask_tag, int k0) {
        constexpr bool MASK = decltype(mask_tag)::value;
        // ---- scores, transposed: sacc[kb] = K[k0+32kb .. +32] Q^T ----
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const T* src = &Ks[(kb * 32 + l32) * KS + kc * KC + g * E];
                op_t a;
                if constexpr (E == 8) a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src));
                else a = *src;
                sacc[kb] = EL::mma(a, qop[kc], sacc[kb]);
            }
        }
        // lane holds query qrow and keys k0 + 32kb + 8(r/4) + 4g + r%4, r = 0..15;
        // hidden keys become -inf and are mapped to p = 0 below
        float mt = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                if constexpr (MASK) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (key >= N || (CAUSAL && key > qrow)) sacc[kb][r] = kNegInf;
                }
                mt = fmaxf(mt, sacc[kb][r]);
            }
        mt = fmaxf(mt, xor32(mt));
        // rescale only when some row's maximum grew past the threshold
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
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(fmaf(sacc[kb][r], c, -mc));
                if constexpr (MASK) p = (sacc[kb][r] == kNegInf) ? 0.f : p;
                sacc[kb][r] = p;
                if (r & 1) ps1 += p; else ps0 += p;
            }
        l_run += ps0 + ps1;                    // row sum from the fp32 probabilities

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int cc = 0; cc < NCH; ++cc) {
                op_t b;
                if constexpr (E == 8) {
#pragma unroll
                    for (int s2 = 0; s2 < 8; ++s2) b[s2] = (__bf16)sacc[kb][8 * cc + s2];
                } else {
                    b = sacc[kb][cc];
                }
#pragma unroll
                for (int db = 0; db < ND; ++db) {
                    const T* vrow = &Vt[(db * 32 + l32) * VS + kb * 32];
                    op_t a;
                    if constexpr (E == 8) {
                        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 16 * cc + 4 * g);
                        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 * cc + 8 + 4 * g);
                        const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
                        a = __builtin_bit_cast(bf16x8, w);
                    } else {
                        a = vrow[8 * (cc >> 2) + 4 * g + (cc & 3)];
                    }
                    oacc[db] = EL::mma(a, b, oacc[db]);
                }
            }
        }
    };

    // Two loops, one per tile variant, so each has a single compute body
    // (one body per loop keeps the accumulators in place across iterations).
    gload(0);
    int kt = 0;
    for (; kt < n_full; ++kt) {
        __syncthreads();                       // every wave is done with the previous tile
        stage();
        __syncthreads();
        if (kt + 1 < n_kt) gload(kt + 1);      // next tile in flight during compute
        compute(std::integral_constant<bool, false>{}, kt * BN);
    }
    for (; kt < n_kt; ++kt) {
        __syncthreads();
        stage();
        __syncthreads();
        if (kt + 1 < n_kt) gload(kt + 1);
        const int k0 = kt * BN;
        if (CAUSAL && k0 > wq0 + 31) continue;   // tile entirely above this wave's diagonal
        compute(std::integral_constant<bool, true>{}, k0);
    }

    // ---- epilogue: O = O_acc / l, LSE = ln(l) + m ----
    const float l_tot = l_run + xor32(l_run);
    if (qrow < N) {
        const float inv = 1.0f / l_tot;
        T* orow = O + base + (size_t)qrow * D;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d0 = db * 32 + 8 * i + 4 * g;
                if constexpr (sizeof(T) == 2) {
                    bf16x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = (__bf16)(oacc[db][4 * i + j] * inv);
                    *reinterpret_cast<bf16x4*>(orow + d0) = w;
                } else {
                    f32x4 w;
#pragma unroll
                    for (int j = 0; j < 4; ++j) w[j] = oacc[db][4 * i + j] * inv;
                    *reinterpret_cast<f32x4*>(orow + d0) = w;
                }
            }
        if (LSE != nullptr && g == 0) {
            const float mc = (m_run == kNegInf) ? 0.f : m_run * c;
            LSE[(size_t)bh * N + qrow] = (mc + __log2f(l_tot)) * kLn2;
        }
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, float scale, hipStream_t stream) {
    const int n_qblocks = (N + BM - 1) / BM;
    const unsigned nwg = (unsigned)B * (unsigned)H * (unsigned)n_qblocks;
    const T* qp = static_cast<const T*>(q);
    const T* kp = static_cast<const T*>(k);
    const T* vp = static_cast<const T*>(v);
    T* op = static_cast<T*>(o);
    float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    void* args[] = {&qp, &kp, &vp, &op, &lse, &N, (void*)&n_qblocks, &scale_log2};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fwd_kernel<T, D, CAUSAL>),
                           dim3(nwg), dim3(NTHREADS), args, 0, stream);
}

template <typename T, int D>
hipError_t launch_causal(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int N, int causal, float scale, hipStream_t stream) {
    return causal ? launch<T, D, true>(q, k, v, o, lse, B, H, N, scale, stream)
                  : launch<T, D, false>(q, k, v, o, lse, B, H, N, scale, stream);
}

}  // namespace

hipError_t fa_launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int N, int d, int causal, float scale, int dtype,
                         hipStream_t stream) {
    if (dtype == 0) {
        return fa_launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, causal, scale, stream);
    } else {
        if (d == 128) return launch_causal<float, 128>(q, k, v, o, lse, B, H, N, causal, scale, stream);
        if (d == 64) return launch_causal<float, 64>(q, k, v, o, lse, B, H, N, causal, scale, stream);
    }
    return hipErrorInvalidValue;
}
