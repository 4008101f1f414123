// fa_kernels.h - launchers of the gfx950 kernels, called by the C ABI (fa_api.cpp).
// Arguments have already been validated by fa_validate.h when these run.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

hipError_t fa_launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int N, int d, int causal, float scale, int dtype,
                         hipStream_t stream);

// Compute units of the current device, queried once per device (fa_fwd_bf16.hip):
// the grid of the persistent forwards
int fa_cu_count();

// bf16 fast path (fa_fwd_bf16.hip)
hipError_t fa_launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, int d, int causal, float scale,
                              hipStream_t stream);

// bf16 backward (fa_bwd.hip): row statistics, dK/dV, dQ; workspace holds the
// row statistics (fa_host::bwd_workspace_bytes)
hipError_t fa_launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              int B, int H, int N, int d, int causal, float scale, void* workspace,
                              hipStream_t stream);

// bf16 prefill of new tokens against a paged KV cache (fa_prefill.hip)
hipError_t fa_launch_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* cu_seqlens_q, void* o, float* lse, int S, int H,
                                   int d, int max_blocks, int64_t num_blocks, int total_q,
                                   int max_q_len, int causal, float scale, hipStream_t stream);

// bf16 draft-tree verification against a paged KV cache (fa_prefill.hip)
hipError_t fa_launch_tree_decode(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_table, const int32_t* seq_lens,
                                 const int32_t* cu_seqlens_q, const int32_t* parents, void* o,
                                 float* lse, int S, int H, int d, int max_blocks,
                                 int64_t num_blocks, int total_q, float scale,
                                 hipStream_t stream);

// RoPE (fa_rope.hip): standalone rotation, and the forward with fused query rotation
hipError_t fa_launch_rope(const void* x, void* out, const float* rope_cos, const float* rope_sin,
                          int B, int H, int N, int d, hipStream_t stream);
hipError_t fa_launch_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                              const float* rope_cos, const float* rope_sin, int B, int H, int N,
                              int d, int causal, float scale, void* workspace,
                              hipStream_t stream);

hipError_t fa_launch_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  void* o, float* lse, int S, int H, int d,
                                  int max_blocks, int64_t num_blocks, float scale,
                                  float* workspace, hipStream_t stream);
// The same decode with the partials in the library's static scratch array
// (fa_decode.hip); the caller has checked that they fit.
hipError_t fa_launch_paged_decode_scratch(const void* q, const void* k_cache, const void* v_cache,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          void* o, float* lse, int S, int H, int d,
                                          int max_blocks, int64_t num_blocks, float scale,
                                          hipStream_t stream);
