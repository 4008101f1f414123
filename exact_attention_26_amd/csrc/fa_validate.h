// fa_validate.h - host-side argument checks of the C ABI (include/fa.h).
//
// Pure C++17, no HIP: the same checks are compiled into libfa.so and into a
// host-only unit test built with g++.  Every check here runs before anything is
// enqueued, so a call rejected here has launched nothing.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>

#include "fa.h"

namespace fa_host {

// Forward pass: query rows per work group.
constexpr int kFwdBlockM = 128;
// Paged decode: pages of one sequence handled by one work group.
constexpr int kDecodeSplitPages = 32;
// Paged decode: the one page size the kernels are built for.
constexpr int kDecodePageSize = 16;

inline bool fwd_head_dim_supported(int d) { return d == 64 || d == 128; }
inline bool decode_head_dim_supported(int d) { return d == 64 || d == 128; }

inline fa_status check_fwd(const void* q, const void* k, const void* v, const void* o,
                           int B, int H, int N, int d, int causal, float scale, int dtype) {
    if (!q || !k || !v || !o) return FA_ERR_INVALID;
    if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID;
    if (!std::isfinite(scale)) return FA_ERR_INVALID;
    const double elems = double(B) * double(H) * double(N) * double(d);
    if (elems >= 4611686018427387904.0) return FA_ERR_INVALID;           // 2^62
    // one head's K or V is addressed with 32-bit byte offsets
    if ((double(N) + 64.0) * double(d) * 2.0 >= 2147483648.0) return FA_ERR_INVALID;
    // one work group per (b, h, block of query rows): the 1-D grid must fit
    const double groups = double(B) * double(H) * std::ceil(double(N) / kFwdBlockM);
    if (groups > 2147483647.0) return FA_ERR_INVALID;
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
    if (!fwd_head_dim_supported(d)) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// Backward: rows per block of the row statistics; each block keeps 64 floats
// (256 bytes, one LDS DMA load): lse*log2(e) of its 32 rows, then their dO.O.
// The statistics kernel's grid has one work group per 64 rows.
constexpr int kBwdStatsRows = 32;
constexpr int kBwdStatsBlockBytes = 256;
constexpr int kBwdPrepRows = 64;

inline bool bwd_head_dim_supported(int d) { return d == 64 || d == 128; }

// Backward workspace bytes for these sizes (0 = invalid sizes).
inline size_t bwd_workspace_bytes(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
    const double blocks = double(B) * H * std::ceil(double(N) / kBwdStatsRows);
    if (blocks * kBwdStatsBlockBytes > 1.0e15) return 0;
    return size_t(B) * size_t(H) * size_t((N + kBwdStatsRows - 1) / kBwdStatsRows) *
           size_t(kBwdStatsBlockBytes);
}

inline fa_status check_bwd(const void* q, const void* k, const void* v, const void* o,
                           const void* lse, const void* dout, const void* dq, const void* dk,
                           const void* dv, int B, int H, int N, int d, int causal, float scale,
                           int dtype, const void* ws, size_t ws_bytes) {
    if (!lse || !dout || !dq || !dk || !dv) return FA_ERR_INVALID;
    // the forward's checks cover q, k, v, o, the sizes, the scale and the
    // 32-bit offsets; its grid bound (one group per 128 rows) covers the
    // backward's 128-row groups, and the statistics grid has 2x that many
    const fa_status st = check_fwd(q, k, v, o, B, H, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    if (double(B) * H * std::ceil(double(N) / kBwdPrepRows) > 2147483647.0) return FA_ERR_INVALID;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!bwd_head_dim_supported(d)) return FA_ERR_UNSUPPORTED;
    const size_t need = bwd_workspace_bytes(B, H, N, d);
    if (need == 0 || !ws || ws_bytes < need) return FA_ERR_INVALID;
    return FA_OK;
}

inline int decode_max_splits(int max_blocks_per_seq) {
    return (max_blocks_per_seq + kDecodeSplitPages - 1) / kDecodeSplitPages;
}

// Workspace: per (sequence, head, split) one partial result of d + 2 floats
// (running max, running sum, unnormalised output row).  0 = invalid sizes.
inline size_t decode_workspace_bytes(int S, int H, int d, int page_size, int max_blocks) {
    if (S < 1 || H < 1 || d < 1 || page_size < 1 || max_blocks < 1) return 0;
    const double bytes = double(S) * H * decode_max_splits(max_blocks) * (double(d) + 2.0) * 4.0;
    if (bytes > 1.0e15) return 0;
    return size_t(S) * size_t(H) * size_t(decode_max_splits(max_blocks)) * (size_t(d) + 2) * 4;
}

inline fa_status check_decode(const void* q, const void* kc, const void* vc, const void* table,
                              const void* lens, const void* o, int S, int H, int d,
                              int page_size, int max_blocks, int64_t num_blocks, float scale,
                              int dtype, const void* ws, size_t ws_bytes) {
    if (!q || !kc || !vc || !table || !lens || !o) return FA_ERR_INVALID;
    if (S < 1 || H < 1 || d < 1 || page_size < 1 || max_blocks < 1 || num_blocks < 1)
        return FA_ERR_INVALID;
    if (!std::isfinite(scale)) return FA_ERR_INVALID;
    if (S > 65535 || H > 65535) return FA_ERR_INVALID;
    // grid: x = (sequence, head) pairs, y = chunks of 32 pages
    if (double(S) * H > 2147483647.0) return FA_ERR_INVALID;
    if (decode_max_splits(max_blocks) > 65535) return FA_ERR_INVALID;
    const double pool = double(num_blocks) * H * page_size * d;
    if (pool >= 4611686018427387904.0) return FA_ERR_INVALID;
    if (double(S) * max_blocks >= 2147483647.0) return FA_ERR_INVALID;   // int32 table index
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!decode_head_dim_supported(d)) return FA_ERR_UNSUPPORTED;
    if (page_size != kDecodePageSize) return FA_ERR_UNSUPPORTED;
    const size_t need = decode_workspace_bytes(S, H, d, page_size, max_blocks);
    if (need == 0 || !ws || ws_bytes < need) return FA_ERR_INVALID;
    return FA_OK;
}

// The allocation-free decode: the same checks, then the workspace must fit
// the library's scratch array (FA_NOALLOC_SCRATCH_BYTES).
inline fa_status check_decode_noalloc(const void* q, const void* kc, const void* vc,
                                      const void* table, const void* lens, const void* o, int S,
                                      int H, int d, int page_size, int max_blocks,
                                      int64_t num_blocks, float scale, int dtype) {
    static const char placeholder = 0;   // stands for the scratch array in the shared checks
    const fa_status st = check_decode(q, kc, vc, table, lens, o, S, H, d, page_size, max_blocks,
                                      num_blocks, scale, dtype, &placeholder, SIZE_MAX);
    if (st != FA_OK) return st;
    if (decode_workspace_bytes(S, H, d, page_size, max_blocks) > FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_TOO_LARGE;
    return FA_OK;
}

inline fa_status check_prefill(const void* q, const void* kc, const void* vc, const void* table,
                               const void* lens, const void* cu, const void* o, int S, int H,
                               int d, int page_size, int max_blocks, int64_t num_blocks,
                               int total_q, int max_q_len, int causal, float scale, int dtype) {
    if (!q || !kc || !vc || !table || !lens || !cu || !o) return FA_ERR_INVALID;
    if (S < 1 || H < 1 || d < 1 || page_size < 1 || max_blocks < 1 || num_blocks < 1 ||
        total_q < 1 || max_q_len < 1)
        return FA_ERR_INVALID;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID;
    if (!std::isfinite(scale)) return FA_ERR_INVALID;
    const double pool = double(num_blocks) * H * page_size * d;
    if (pool >= 4611686018427387904.0) return FA_ERR_INVALID;            // 2^62 elements
    if (double(total_q) * H * d >= 4611686018427387904.0) return FA_ERR_INVALID;
    if (double(S) * max_blocks >= 2147483647.0) return FA_ERR_INVALID;   // int32 table index
    if (double(max_blocks) * page_size >= 2147483647.0) return FA_ERR_INVALID;
    // one work group per (sequence, head, block of kFwdBlockM new rows), the
    // (sequence, head) count padded to a multiple of 8 (the XCD dealing)
    const double units = std::ceil(double(S) * H / 8.0) * 8.0;
    const double groups = units * std::ceil(double(max_q_len) / kFwdBlockM);
    if (groups > 2147483647.0) return FA_ERR_INVALID;
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (!fwd_head_dim_supported(d)) return FA_ERR_UNSUPPORTED;
    if (page_size != kDecodePageSize) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// Draft-tree verification: at most this many nodes per tree.
constexpr int kTreeMaxNodes = 64;

inline fa_status check_tree(const void* q, const void* kc, const void* vc, const void* table,
                            const void* lens, const void* cu, const void* parents, const void* o,
                            int S, int H, int d, int page_size, int max_blocks,
                            int64_t num_blocks, int total_q, int max_q_len, float scale,
                            int dtype) {
    if (!parents) return FA_ERR_INVALID;
    const fa_status st = check_prefill(q, kc, vc, table, lens, cu, o, S, H, d, page_size,
                                       max_blocks, num_blocks, total_q, max_q_len, 0, scale,
                                       dtype);
    if (st != FA_OK) return st;
    if (max_q_len > kTreeMaxNodes) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

inline fa_status check_rope(const void* x, const void* out, const void* c, const void* s, int B,
                            int H, int N, int d, int dtype) {
    if (!x || !out || !c || !s) return FA_ERR_INVALID;
    if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID;
    const double elems = double(B) * H * N * d;
    if (elems >= 4611686018427387904.0) return FA_ERR_INVALID;
    if (elems / 8.0 / 256.0 > 2147483647.0) return FA_ERR_INVALID;      // 1-D grid
    if (dtype != FA_BF16 && dtype != FA_F32) return FA_ERR_UNSUPPORTED;
    if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    return FA_OK;
}

// Forward with RoPE: the rotated keys go to the workspace, [B][H][N][d] bf16.
inline size_t fwd_rope_workspace_bytes(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
    const double bytes = double(B) * H * N * d * 2.0;
    if (bytes > 1.0e15) return 0;
    return size_t(B) * size_t(H) * size_t(N) * size_t(d) * 2;
}

inline fa_status check_fwd_rope(const void* q, const void* k, const void* v, const void* o,
                                const void* c, const void* s, int B, int H, int N, int d,
                                int causal, float scale, int dtype, const void* ws,
                                size_t ws_bytes) {
    if (!c || !s) return FA_ERR_INVALID;
    fa_status st = check_fwd(q, k, v, o, B, H, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    st = check_rope(k, ws ? ws : k, c, s, B, H, N, d, dtype);
    if (st != FA_OK) return st;
    const size_t need = fwd_rope_workspace_bytes(B, H, N, d);
    if (need == 0 || !ws || ws_bytes < need) return FA_ERR_INVALID;
    return FA_OK;
}

inline const char* status_string(int s) {
    switch (s) {
        case FA_OK: return "FA_OK";
        case FA_ERR_INVALID: return "FA_ERR_INVALID: invalid argument";
        case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: no kernel for this configuration";
        case FA_ERR_HIP: return "FA_ERR_HIP: a HIP runtime call failed";
        case FA_ERR_TOO_LARGE:
            return "FA_ERR_TOO_LARGE: the call needs more than the 32 MiB of scratch memory "
                   "the allocation-free entry point holds";
        default: return "unknown fa_status";
    }
}

}  // namespace fa_host
