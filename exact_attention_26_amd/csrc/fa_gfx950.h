// fa_gfx950.h - device building blocks shared by the gfx950 attention kernels.
//
// Vector types, lane exchanges, the LDS chunk swizzle and the buffer -> LDS
// tile loader used by the forward and backward kernels.  Each piece was
// checked on the hardware (lane layouts with in-bounds probes, bank conflicts
// with counters); the facts are restated next to the code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa_gfx950 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int TILE_ROWS = 64;               // rows of a K/V (or Q/dO) tile in LDS
constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// v_permlane32_swap(x, x) returns (x[l % 32], x[32 + l % 32]) in every lane l,
// so one instruction gives a lane and its partner lane ^ 32.
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

// Physical 16-byte chunk of logical chunk c in LDS row r.  gfx950's LDS has 64
// banks of 4 bytes (256-byte lines of 16 chunk slots).  The permutation makes
//  * a row-major fragment read (16 lanes per cycle: 16 consecutive rows, one
//    chunk) and
//  * a transposed fragment read (32 lanes per cycle: 4 consecutive rows x 4
//    adjacent chunks)
// touch 16 different chunk slots, i.e. every bank once.
// d = 128: one row per line, chunk c in 0..15.
// d = 64: two rows per line (slot = 8*(r&1) + chunk), chunk c in 0..7.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset, within a tile, of the 16 bytes lane `lane` of wave-wide load
// `region` writes: buffer_load ... lds puts lane l's 16 bytes at LDS byte
// M0 + 16 l, so a 1 KiB load fills (rows region*RPK .. +RPK) x (all chunk
// slots); the lane fetches the logical chunk stored in its slot.
template <int D>
__device__ __forceinline__ int tile_load_offset(int region, int lane) {
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int RPK = 1024 / (D * 2);      // rows per 1 KiB
    const int row = region * RPK + lane / CPR;
    return (row * D + swz<D>(row, lane % CPR) * 8) * 2;
}

// Cache policy of a buffer load: non-temporal (data read once per launch).
constexpr int kLoadNT = 2;

// Rows [tbase/(2D), +TILE_ROWS) of a [rows][D] bf16 matrix X (rows*D*2 = bytes)
// into LDS `dst`, swizzled: this wave issues NLOAD 1 KiB loads, regions
// first_region .. first_region+NLOAD-1, with gofs[i] = tile_load_offset of its
// region.  The buffer resource spans X, so rows past its end arrive as zeros.
// AUX: cache policy of the loads (0, or kLoadNT).
template <int NLOAD, int AUX = 0>
__device__ __forceinline__ void load_tile_lds(const uint16_t* X, int bytes, int tbase,
                                              const int* gofs, uint16_t* dst, int first_region) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)X, (short)0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < NLOAD; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + (first_region + i) * 512), 16,
                                                 gofs[i], tbase, 0, AUX);
}

// One 1 KiB block of x (bytes [offset, offset + 1024) of a buffer of `bytes`
// bytes) into LDS `dst`, one wave, 16 bytes per lane; bytes past the end of
// the buffer arrive as zeros.
__device__ __forceinline__ void load_kib_lds(const void* x, int bytes, int offset, uint16_t* dst,
                                             int lane) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, bytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)dst, 16, lane * 16, offset, 0, 0);
}

// Row-major MFMA operand read: 8 consecutive bf16 of row `row` starting at
// logical chunk `chunk` of a swizzled [TILE_ROWS][D] tile.
template <int D>
__device__ __forceinline__ int frag_offset(int row, int chunk) {
    return row * D + swz<D>(row, chunk) * 8;
}

// Transposed MFMA operand read (ds_read_b64_tr_b16): within each 16-lane group,
// lane i receives element i%4 of the 8 bytes addressed by lane 4j + i/4, for
// j = 0..3.  For an A operand whose rows are tile columns d = col0 + 0..31 and
// whose k index runs over tile rows, lane (group h = lane/16, index li) points
// at tile row 4(h/2) + li/4 (+8 for the second half of the 8 k-slots) and
// column col0 + 16(h%2) + 4(li%4); the result is then lane (row l%32, k-group
// l/32) holding tile rows {4g..4g+3} (+8) of its column.
template <int D>
__device__ __forceinline__ int trfrag_offset(int lane, int half, int col0) {
    const int h = lane >> 4;
    const int li = lane & 15;
    const int row = 4 * (h >> 1) + (li >> 2) + 8 * half;
    const int col = col0 + 16 * (h & 1) + 4 * (li & 3);
    return row * D + swz<D>(row, col >> 3) * 8 + (col & 7);
}

// Two transposed reads (k-slots 0-3 and 4-7) combined into one bf16x8 operand.
__device__ __forceinline__ bf16x8 tr_operand(const uint16_t* lo, const uint16_t* hi) {
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lo);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)hi);
    const u32x2 a2 = __builtin_bit_cast(u32x2, a);
    const u32x2 b2 = __builtin_bit_cast(u32x2, b);
    const u32x4 w = {a2[0], a2[1], b2[0], b2[1]};
    return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Operand of one lane's own row: the 8 bf16 at columns chunk*8 .. +8 of row
// `row` of a [rows][D] matrix in global memory; zeros past `rows`; sign bits
// flipped by `flip`.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const uint16_t* X, int row, int rows, int chunk,
                                              uint32_t flip) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < rows) x = *reinterpret_cast<const u32x4*>(X + (size_t)row * D + chunk * 8);
    x ^= flip;
    return __builtin_bit_cast(bf16x8, x);
}

// Four bf16 (the packed u32x2 of a bf16x4) from four floats, round to nearest even.
__device__ __forceinline__ bf16x4 to_bf16x4(float a, float b, float c, float d) {
    bf16x4 w;
    w[0] = (__bf16)a;
    w[1] = (__bf16)b;
    w[2] = (__bf16)c;
    w[3] = (__bf16)d;
    return w;
}

// One output row (O, or dQ / dK / dV) from a lane's transposed MFMA
// accumulators (oacc[db][4j + i] holds column db*32 + 8j + 4g + i of the
// lane's row), times inv, as bf16 with 16-byte stores: lanes l and l + 32
// hold the two halves of each 16-column group of row l and swap pieces with
// v_permlane32_swap, so that each then holds 8 consecutive columns (half as
// many store instructions as 8-byte stores of the pieces as they are,
// measured 2-4 % faster in the forwards).  Every lane must run it
// (the swap reads the partner lane); `store` false skips only the stores.
template <int ND>
__device__ __forceinline__ void store_o_row(uint16_t* orow, const f32x16 (&oacc)[ND], float inv,
                                            int g, bool store) {
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
            u32x2 a = __builtin_bit_cast(
                u32x2, to_bf16x4(oacc[db][8 * pr] * inv, oacc[db][8 * pr + 1] * inv,
                                 oacc[db][8 * pr + 2] * inv, oacc[db][8 * pr + 3] * inv));
            u32x2 b = __builtin_bit_cast(
                u32x2, to_bf16x4(oacc[db][8 * pr + 4] * inv, oacc[db][8 * pr + 5] * inv,
                                 oacc[db][8 * pr + 6] * inv, oacc[db][8 * pr + 7] * inv));
            // lane l keeps a (columns 16pr .. +3 of its group) and takes the
            // partner's a (+4 .. +7); lane l + 32 takes the partner's b
            // (+8 .. +11) and keeps its own b (+12 .. +15)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const auto r = __builtin_amdgcn_permlane32_swap(a[h], b[h], false, false);
                a[h] = r[0];
                b[h] = r[1];
            }
            const u32x4 w = {a[0], a[1], b[0], b[1]};
            if (store) *reinterpret_cast<u32x4*>(orow + db * 32 + 16 * pr + 8 * g) = w;
        }
}

// Rotate the four complex numbers (x[2i] + j x[2i+1], i = 0..3) held as 8
// bf16 in x by the angles whose cosines / sines are c, s: fp32 arithmetic,
// results rounded to nearest even bf16.
__device__ __forceinline__ u32x4 rotate_pairs(u32x4 x, float4 c, float4 s) {
    const float cs[4] = {c.x, c.y, c.z, c.w};
    const float sn[4] = {s.x, s.y, s.z, s.w};
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float re = __uint_as_float(x[w] << 16);          // element 2w
        const float im = __uint_as_float(x[w] & 0xFFFF0000u);  // element 2w + 1
        const float nre = fmaf(re, cs[w], -im * sn[w]);
        const float nim = fmaf(re, sn[w], im * cs[w]);
        const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)nre);
        const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)nim);
        out[w] = lo | (hi << 16);
    }
    return out;
}

}  // namespace fa_gfx950
