// fa_api.cpp - the C ABI of libfa.so (declared in include/fa.h).
//
// Validates on the host (fa_validate.h), then enqueues the kernels on the
// caller's stream.  Never allocates, frees or synchronises.
#include <hip/hip_runtime.h>

#include "fa.h"
#include "fa_kernels.h"
#include "fa_validate.h"

namespace {
thread_local int t_last_hip_error = 0;

fa_status hip_status(hipError_t e) {
    if (e == hipSuccess) return FA_OK;
    t_last_hip_error = static_cast<int>(e);
    return FA_ERR_HIP;
}
}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale, int dtype, void* stream) {
    const fa_status st = fa_host::check_fwd(q, k, v, o, B, H, N, d, causal, scale, dtype);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, dtype,
                                    static_cast<hipStream_t>(stream)));
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
    return fa_host::bwd_workspace_bytes(B, H, N, d);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                 int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream) {
    const fa_status st = fa_host::check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, causal,
                                            scale, dtype, workspace, workspace_bytes);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, d, causal,
                                         scale, workspace, static_cast<hipStream_t>(stream)));
}

size_t fa_paged_decode_workspace_size(int num_seqs, int H, int d, int page_size,
                                      int max_blocks_per_seq) {
    return fa_host::decode_workspace_bytes(num_seqs, H, d, page_size, max_blocks_per_seq);
}

fa_status fa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, void* o,
                          float* lse, int num_seqs, int H, int d, int page_size,
                          int max_blocks_per_seq, int64_t num_blocks, float scale, int dtype,
                          void* workspace, size_t workspace_bytes, void* stream) {
    const fa_status st = fa_host::check_decode(q, k_cache, v_cache, block_table, seq_lens, o,
                                               num_seqs, H, d, page_size, max_blocks_per_seq,
                                               num_blocks, scale, dtype, workspace,
                                               workspace_bytes);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_paged_decode(q, k_cache, v_cache, block_table, seq_lens, o, lse,
                                             num_seqs, H, d, max_blocks_per_seq, num_blocks,
                                             scale, static_cast<float*>(workspace),
                                             static_cast<hipStream_t>(stream)));
}

fa_status fa_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens, void* o,
                                  float* lse, int num_seqs, int H, int d, int page_size,
                                  int max_blocks_per_seq, int64_t num_blocks, float scale,
                                  int dtype, void* stream) {
    const fa_status st = fa_host::check_decode_noalloc(q, k_cache, v_cache, block_table,
                                                       seq_lens, o, num_seqs, H, d, page_size,
                                                       max_blocks_per_seq, num_blocks, scale,
                                                       dtype);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_paged_decode_scratch(q, k_cache, v_cache, block_table, seq_lens,
                                                     o, lse, num_seqs, H, d, max_blocks_per_seq,
                                                     num_blocks, scale,
                                                     static_cast<hipStream_t>(stream)));
}

fa_status fa_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* cu_seqlens_q, void* o, float* lse, int num_seqs, int H,
                           int d, int page_size, int max_blocks_per_seq, int64_t num_blocks,
                           int total_q, int max_q_len, int causal, float scale, int dtype,
                           void* stream) {
    const fa_status st = fa_host::check_prefill(q, k_cache, v_cache, block_table, seq_lens,
                                                cu_seqlens_q, o, num_seqs, H, d, page_size,
                                                max_blocks_per_seq, num_blocks, total_q,
                                                max_q_len, causal, scale, dtype);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_paged_prefill(q, k_cache, v_cache, block_table, seq_lens,
                                              cu_seqlens_q, o, lse, num_seqs, H, d,
                                              max_blocks_per_seq, num_blocks, total_q, max_q_len,
                                              causal, scale, static_cast<hipStream_t>(stream)));
}

fa_status fa_tree_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* cu_seqlens_q, const int32_t* tree_parents, void* o,
                         float* lse, int num_seqs, int H, int d, int page_size,
                         int max_blocks_per_seq, int64_t num_blocks, int total_q, int max_q_len,
                         float scale, int dtype, void* stream) {
    const fa_status st = fa_host::check_tree(q, k_cache, v_cache, block_table, seq_lens,
                                             cu_seqlens_q, tree_parents, o, num_seqs, H, d,
                                             page_size, max_blocks_per_seq, num_blocks, total_q,
                                             max_q_len, scale, dtype);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_tree_decode(q, k_cache, v_cache, block_table, seq_lens,
                                            cu_seqlens_q, tree_parents, o, lse, num_seqs, H, d,
                                            max_blocks_per_seq, num_blocks, total_q, scale,
                                            static_cast<hipStream_t>(stream)));
}

fa_status fa_rope(const void* x, void* out, const float* rope_cos, const float* rope_sin, int B,
                  int H, int N, int d, int dtype, void* stream) {
    const fa_status st = fa_host::check_rope(x, out, rope_cos, rope_sin, B, H, N, d, dtype);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_rope(x, out, rope_cos, rope_sin, B, H, N, d,
                                     static_cast<hipStream_t>(stream)));
}

size_t fa_fwd_rope_workspace_size(int B, int H, int N, int d) {
    return fa_host::fwd_rope_workspace_bytes(B, H, N, d);
}

fa_status fa_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                      const float* rope_cos, const float* rope_sin, int B, int H, int N, int d,
                      int causal, float scale, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
    const fa_status st = fa_host::check_fwd_rope(q, k, v, o, rope_cos, rope_sin, B, H, N, d,
                                                 causal, scale, dtype, workspace,
                                                 workspace_bytes);
    if (st != FA_OK) return st;
    return hip_status(fa_launch_fwd_rope(q, k, v, o, lse, rope_cos, rope_sin, B, H, N, d, causal,
                                         scale, workspace, static_cast<hipStream_t>(stream)));
}

const char* fa_status_string(int status) { return fa_host::status_string(status); }

int fa_last_hip_error(void) { return t_last_hip_error; }

}  // extern "C"
