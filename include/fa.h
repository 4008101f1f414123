/*
 * fa.h - C ABI of libfa.so: exact scaled-dot-product attention on MI355X (gfx950).
 *
 * Six operations sit behind this interface.
 *
 *   fa_fwd           the attention forward pass computed FlashAttention-style:
 *                    Q, K, V in device memory, O (and the per-row log-sum-exp)
 *                    written back, the N x N score matrix never stored.
 *   fa_bwd           its backward pass: dQ, dK, dV from dO, recomputing the
 *                    scores from Q, K and the stored log-sum-exp.
 *   fa_paged_decode  one query token per sequence attending to a KV cache that
 *                    is stored in fixed-size pages and reached through a block
 *                    table.
 *   fa_paged_prefill the new tokens of a batch of sequences of different
 *                    lengths attending to that paged cache (prefill, chunked
 *                    prefill, continuous batching).
 *   fa_tree_decode   the nodes of a draft token tree per sequence attending to
 *                    that paged cache under a tree mask (speculative decoding).
 *   fa_rope,         rotary position embedding of queries / keys, standalone and
 *   fa_fwd_rope      fused into the forward pass.
 *
 * What is computed.  For every batch b and head h, with s_ij = scale * q_i . k_j
 * over the keys j that query i may see (all j, or j <= i when causal):
 *     o_i   = sum_j exp(s_ij) v_j / sum_j exp(s_ij)
 *     lse_i = ln sum_j exp(s_ij)                       (natural log)
 * This is the textbook scaled dot-product attention ("LLM study notes",
 * DEVOCEAN tech blog, section on the self-attention computation: dot-product
 * similarity, division by the square root of the key dimension, softmax,
 * weighting of V; "Flash Attention", velog @myungum, section 1).  The method
 * computes it exactly ("Flash Attention", velog @myungum, section 2: exact
 * attention with far fewer memory accesses), so results differ from the plain
 * definition only by floating-point rounding.
 *
 * Conventions shared by every entry point.
 *   - Pointers are DEVICE pointers (HBM) unless stated otherwise.  The caller
 *     owns every buffer; the library never allocates, frees or synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued on it and the call returns at once; results are valid after
 *     the stream has been synchronised.
 *   - Every array is row-major and densely packed.
 *   - Errors are reported by the return value only.  Anything that can be
 *     checked on the host is checked BEFORE any work is enqueued: a call that
 *     returns FA_ERR_INVALID or FA_ERR_UNSUPPORTED has launched nothing and
 *     written nothing.  FA_ERR_UNSUPPORTED means "valid request, no kernel for
 *     it here": a caller may fall back to another implementation, as the fast
 *     attention path in PyTorch does when head size, dtype, mask or hardware is
 *     not supported ("How does Flash Attention reduce memory traffic in local
 *     inference?", ZimaSpace blog, section on hardware and shape support).
 *   - FA_ERR_HIP means a HIP call (a launch) failed; fa_last_hip_error() gives
 *     the hipError_t of the last such failure on the calling thread.  Faults
 *     during execution surface at stream synchronisation, as usual in HIP.
 *   - Calls are deterministic: the same inputs give bit-identical outputs.
 *   - Outputs must not alias inputs.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID = 1,      /* malformed arguments (null pointer, size < 1, non-finite scale, ...) */
    FA_ERR_UNSUPPORTED = 2,  /* well-formed, but no kernel for this head size / dtype / page size */
    FA_ERR_HIP = 3,          /* a HIP runtime call failed; see fa_last_hip_error() */
    FA_ERR_TOO_LARGE = 4     /* fa_paged_decode_noalloc only: the call needs more scratch
                                memory than the library holds (FA_NOALLOC_SCRATCH_BYTES) */
} fa_status;

/* Device scratch memory that fa_paged_decode_noalloc holds on every GPU it runs on. */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

typedef enum {
    FA_BF16 = 0,             /* bfloat16 inputs and outputs, float32 accumulation */
    FA_F32 = 1               /* float32 inputs and outputs, float32 accumulation */
} fa_dtype;

/*
 * fa_fwd - attention forward pass, one kernel launch.
 *
 * Follows "Flash Attention" (velog @myungum), section 2 and its pseudocode:
 * Q, K, V split into row blocks staged through on-chip memory, scores computed
 * per block, a running row max m and row sum l rescale the partial output as
 * new key blocks arrive, so only O (and the row statistics) reach HBM.  Work is
 * split over batch, heads and blocks of query rows, and each work group owns
 * its rows of O ("FlashAttention-2 GPU work partitioning", iPLEX blog,
 * section 3, changes 2 and 3).  The optional causal mask lets query i see keys
 * j <= i only (same page, section 4).
 *
 *   q, k, v   [B][H][N][d] elements of `dtype`           (read)
 *   o         [B][H][N][d] elements of `dtype`           (written; must not alias q, k, v)
 *   lse       [B][H][N] float32, natural-log log-sum-exp of the scaled scores
 *             of each row (written), or NULL to skip it
 *   B, H, N   batch, heads, sequence length; each >= 1 (any N, not only
 *             multiples of the tile size)
 *   d         head dimension: 64 or 128 (else FA_ERR_UNSUPPORTED)
 *   causal    0 = every query sees every key; 1 = query i sees keys 0..i
 *   scale     multiplies q.k before the softmax; must be finite
 *             (1/sqrt(d) is the textbook choice)
 *   dtype     FA_BF16 or FA_F32 (a fa_dtype value)
 *   stream    hipStream_t, or NULL
 *
 * Returns FA_OK, FA_ERR_INVALID (null q/k/v/o, B/H/N < 1, causal not 0/1,
 * non-finite scale, N*d*2 bytes of one head beyond 2^31, or more than 2^31-1
 * work groups), FA_ERR_UNSUPPORTED (d not 64/128, unknown dtype), or FA_ERR_HIP.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, int causal, float scale,
                 int dtype, void* stream);

/*
 * fa_bwd_workspace_size - bytes of device workspace fa_bwd needs for these
 * sizes (0 if the sizes are invalid).  Host-only, no HIP call.  It is
 * B * H * ceil(N / 32) * 256 bytes: per 32 rows, their log-sum-exp and dO . O.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * fa_bwd - attention backward pass: dQ, dK, dV from dO.
 *
 * The pages present the method as built for training, with a backward pass
 * that keeps only the forward's output and row statistics and recomputes the
 * attention scores block by block instead of storing the N x N matrix
 * ("PagedAttention vs FlashAttention: key differences", training section;
 * "LLM study notes", DEVOCEAN tech blog, FlashAttention core principles:
 * recomputation; the row statistics are the lse output of fa_fwd).  With
 * P = softmax(scale * Q K^T) (the same mask as the forward) it computes the
 * plain gradient of O = P V:
 *     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - rowsum(dO o O)),
 *     dQ = scale * dS K,  dK = scale * dS^T Q.
 * No N x N matrix is stored and no atomics are used (deterministic).
 *
 *   q, k, v     [B][H][N][d] bf16, the forward's inputs          (read)
 *   o           [B][H][N][d] bf16, the forward's output          (read)
 *   lse         [B][H][N] float32, the forward's natural-log lse (read)
 *   dout        [B][H][N][d] bf16, gradient of the loss w.r.t. o (read)
 *   dq, dk, dv  [B][H][N][d] bf16 gradients                      (written;
 *               must not alias any input or each other)
 *   B, H, N, d, causal, scale   as in fa_fwd (and equal to the forward's)
 *   dtype       FA_BF16 (FA_F32 -> FA_ERR_UNSUPPORTED)
 *   workspace   device scratch of at least fa_bwd_workspace_size(B, H, N, d)
 *               bytes, owned by the caller; contents on entry do not matter;
 *               it must not be shared with a call still running on another
 *               stream.
 *   stream      hipStream_t, or NULL
 *
 * o and lse are taken as given: with another o or lse the result is the
 * gradient formula above evaluated with them, not the true gradient.
 *
 * Returns FA_OK, FA_ERR_INVALID (any null pointer, the size checks of fa_fwd,
 * workspace NULL or too small), FA_ERR_UNSUPPORTED (d not 64/128, dtype not
 * FA_BF16), or FA_ERR_HIP.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, int causal, float scale,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_paged_decode_workspace_size - bytes of device workspace fa_paged_decode
 * needs for these sizes (0 if the sizes are invalid).  Host-only, no HIP call.
 */
size_t fa_paged_decode_workspace_size(int num_seqs, int H, int d, int page_size,
                                      int max_blocks_per_seq);

/*
 * fa_paged_decode - one query token per sequence against a paged KV cache.
 *
 * The KV cache is stored in fixed-size blocks ("pages") of `page_size` tokens;
 * a per-sequence block table maps the logically contiguous token positions of a
 * sequence onto physically scattered pages, and sequences may share pages
 * (a common prompt prefix) simply by listing the same physical ids ("LLM study
 * notes", DEVOCEAN tech blog, section "Paged attention": block table, at most
 * block-size minus one wasted slots per sequence, prompt sharing).  The query
 * attends to all seq_lens[s] cached tokens of its sequence (no mask).  The
 * keys of one sequence are split into chunks worked on by separate work
 * groups; a second small kernel merges the chunk results with the
 * online-softmax rescaling rule ("Flash Attention", velog @myungum,
 * pseudocode).
 *
 *   q            [S][H][d] elements of `dtype`              (read)
 *   k_cache      [num_blocks][H][page_size][d] of `dtype`    (read)
 *   v_cache      [num_blocks][H][page_size][d] of `dtype`    (read)
 *   block_table  [S][max_blocks_per_seq] int32, physical page ids (read)
 *   seq_lens     [S] int32, tokens cached per sequence       (read)
 *   o            [S][H][d] elements of `dtype`              (written)
 *   lse          [S][H] float32 natural-log log-sum-exp, or NULL
 *   num_seqs (S), H >= 1 (each at most 65535, S * H at most 2^31 - 1);
 *   d: 64 or 128 (else FA_ERR_UNSUPPORTED);  page_size: 16 (else FA_ERR_UNSUPPORTED);
 *   max_blocks_per_seq >= 1 and at most 65535 * 32 (one work group per 32 pages and head);
 *   num_blocks >= 1;  scale finite;  dtype: FA_BF16 (FA_F32 -> UNSUPPORTED)
 *   workspace    device scratch of at least
 *                fa_paged_decode_workspace_size(S, H, d, page_size, max_blocks_per_seq)
 *                bytes, owned by the caller; contents on entry do not matter;
 *                it must not be shared with a call still running on another
 *                stream.
 *
 * Device-resident inputs are not inspected on the host (that would need a
 * synchronisation).  Their out-of-range values have defined results instead:
 *   seq_lens[s] <= 0        -> o[s] = 0 and lse[s] = -inf (empty softmax)
 *   seq_lens[s] > max_blocks_per_seq * page_size -> clamped to that many tokens
 *   a block_table entry outside [0, num_blocks) -> that page is skipped
 *   table entries past page ceil(seq_lens[s]/page_size)-1, and cache slots
 *   past seq_lens[s] in the last page, are never read.
 *
 * Returns FA_OK, FA_ERR_INVALID (null required pointer, sizes < 1 or past the
 * limits above, non-finite scale, workspace NULL or too small),
 * FA_ERR_UNSUPPORTED, or FA_ERR_HIP.
 */
fa_status fa_paged_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens,
                          void* o, float* lse,
                          int num_seqs, int H, int d, int page_size,
                          int max_blocks_per_seq, int64_t num_blocks, float scale,
                          int dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * fa_paged_decode_noalloc - fa_paged_decode for callers that cannot allocate.
 *
 * For callers that cannot call hipMalloc around an attention call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results as fa_paged_decode, minus the workspace:
 * the per-split partial results live in a scratch array of
 * FA_NOALLOC_SCRATCH_BYTES (32 MiB) that the library keeps in device memory,
 * one copy per GPU, held from the first call on that GPU until the process
 * ends.  The call allocates nothing (no hipMalloc / hipFree); its first call
 * on a GPU looks up that GPU's copy once (hipGetSymbolAddress).
 *
 *   requirement  fa_paged_decode_workspace_size(num_seqs, H, d, page_size,
 *                max_blocks_per_seq) <= FA_NOALLOC_SCRATCH_BYTES, i.e.
 *                num_seqs * H * ceil(max_blocks_per_seq / 32) * (d + 2) * 4
 *                bytes: e.g. 64 sequences x 32 heads of d = 128 with up to
 *                16384-token tables need 17 MB.  Larger requests return
 *                FA_ERR_TOO_LARGE and launch nothing.
 *   sharing      every call on one GPU uses that GPU's single array, which
 *                keeps the last call's contents (each call writes every entry
 *                it reads, so nothing needs clearing).  Calls that overlap in
 *                time on one GPU (several streams or threads) race on it and
 *                give wrong results: issue them on one stream, or serialise.
 *   stream       the array of the stream's device is used.
 *
 * Returns FA_OK, FA_ERR_INVALID / FA_ERR_UNSUPPORTED as fa_paged_decode (less
 * the workspace checks), FA_ERR_TOO_LARGE, or FA_ERR_HIP.
 */
fa_status fa_paged_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  void* o, float* lse,
                                  int num_seqs, int H, int d, int page_size,
                                  int max_blocks_per_seq, int64_t num_blocks, float scale,
                                  int dtype, void* stream);

/*
 * fa_paged_prefill - new query tokens of several sequences against a paged KV cache.
 *
 * Continuous batching mixes sequences of different lengths in one call
 * ("LLM study notes", DEVOCEAN tech blog, batching section), and the paged
 * cache and FlashAttention-style compute are used together ("PagedAttention
 * vs FlashAttention: key differences"): K/V are read through the block table
 * ("LLM study notes", section "Paged attention") in tiles of 64 keys, with
 * the online softmax of fa_fwd.  Sequence s has seq_lens[s] cached tokens,
 * INCLUDING its new ones, which are the last n_s = cu_seqlens_q[s+1] -
 * cu_seqlens_q[s] of them (their K/V must already be in the cache).  New
 * query i of sequence s stands at position seq_lens[s] - n_s + i; causal = 1
 * lets it see positions 0 .. seq_lens[s] - n_s + i (the current and earlier
 * tokens, "FlashAttention-2 GPU work partitioning", iPLEX blog, section 4),
 * causal = 0 lets it see all seq_lens[s] tokens.
 *
 *   q            [total_q][H][d] bf16, sequence s at rows cu_seqlens_q[s] ..  (read)
 *   k_cache      [num_blocks][H][page_size][d] bf16                          (read)
 *   v_cache      [num_blocks][H][page_size][d] bf16                          (read)
 *   block_table  [S][max_blocks_per_seq] int32 physical page ids             (read)
 *   seq_lens     [S] int32 cached tokens per sequence, new ones included     (read)
 *   cu_seqlens_q [S+1] int32, cu_seqlens_q[0] = 0, non-decreasing,
 *                cu_seqlens_q[S] = total_q                                   (read)
 *   o            [total_q][H][d] bf16                                        (written)
 *   lse          [total_q][H] float32 natural-log log-sum-exp, or NULL       (written)
 *   num_seqs (S), H >= 1;  d: 64 or 128;  page_size: 16;  max_blocks_per_seq >= 1;
 *   num_blocks >= 1;  total_q >= 1;  max_q_len >= 1 and >= every n_s (rows of
 *   a sequence past max_q_len are not written);  causal 0 or 1;  scale finite;
 *   dtype FA_BF16 (FA_F32 -> FA_ERR_UNSUPPORTED).  No workspace.
 *
 * Device-resident inputs are not inspected on the host; their out-of-range
 * values have defined results:
 *   a query that sees no token (seq_lens[s] <= 0, or causal with
 *   n_s > seq_lens[s] for its first n_s - seq_lens[s] queries)  -> o = 0, lse = -inf
 *   seq_lens[s] > max_blocks_per_seq * page_size -> clamped to that many tokens
 *   a block_table entry outside [0, num_blocks) -> that page's tokens are not seen
 *   rows cu_seqlens_q[s] .. that fall outside [0, total_q) -> not written
 *   table entries past page ceil(seq_lens[s]/page_size)-1 and cache slots past
 *   seq_lens[s] in the last page are never read.
 *
 * Returns FA_OK, FA_ERR_INVALID (null required pointer, sizes < 1, causal not
 * 0/1, non-finite scale, more than 2^31-1 work groups), FA_ERR_UNSUPPORTED
 * (d, page_size or dtype), or FA_ERR_HIP.
 */
fa_status fa_paged_prefill(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* cu_seqlens_q, void* o, float* lse,
                           int num_seqs, int H, int d, int page_size, int max_blocks_per_seq,
                           int64_t num_blocks, int total_q, int max_q_len, int causal,
                           float scale, int dtype, void* stream);

/*
 * fa_tree_decode - verify a draft token tree per sequence in one pass.
 *
 * Speculative decoding ("LLM study notes", DEVOCEAN tech blog, speculative
 * decoding section): a draft model proposes candidate tokens organised as a
 * tree, each node one token, and the target model computes every node in a
 * single forward pass with tree attention.  Here sequence s has seq_lens[s]
 * cached tokens whose last n_s = cu_seqlens_q[s+1] - cu_seqlens_q[s] are the
 * tree's nodes in node order (their K/V already in the cache); node i sees
 * the seq_lens[s] - n_s committed tokens and the nodes on its own path from
 * the root -- itself, its parent, its parent's parent, ... -- and no other
 * node (no siblings, no descendants).  K/V are read through the block table
 * ("LLM study notes", section "Paged attention") with the tiled online
 * softmax of fa_fwd.
 *
 *   q, k_cache, v_cache, block_table, seq_lens, cu_seqlens_q, o, lse,
 *   num_seqs, H, d, page_size, max_blocks_per_seq, num_blocks, total_q, scale,
 *   dtype, stream    as in fa_paged_prefill
 *   tree_parents     [total_q] int32, packed like q: the index (0-based among
 *                    the sequence's nodes) of node i's parent, which must be
 *                    smaller than i, or -1 when node i hangs directly off the
 *                    committed tokens                                    (read)
 *   max_q_len        >= every n_s and at most 64 (else FA_ERR_UNSUPPORTED):
 *                    one work group per (sequence, head) holds the whole tree
 *
 * Device-resident inputs: a parent index outside [0, i) is taken as -1;
 * nodes past the 64th of a sequence are not written; the rest as in
 * fa_paged_prefill (a node that sees no token gets o = 0, lse = -inf).
 *
 * Returns FA_OK, FA_ERR_INVALID (as fa_paged_prefill, or tree_parents NULL),
 * FA_ERR_UNSUPPORTED (d, page_size, dtype, or max_q_len > 64), or FA_ERR_HIP.
 */
fa_status fa_tree_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* cu_seqlens_q, const int32_t* tree_parents,
                         void* o, float* lse, int num_seqs, int H, int d, int page_size,
                         int max_blocks_per_seq, int64_t num_blocks, int total_q, int max_q_len,
                         float scale, int dtype, void* stream);

/*
 * fa_rope - rotary position embedding (RoPE) of a [B][H][N][d] tensor.
 *
 * "LLM study notes" (DEVOCEAN tech blog), RoPE section: a token's embedding is
 * read as complex numbers and rotated in the complex plane by an angle given
 * by its absolute position, so that the inner product of a rotated query and
 * a rotated key depends only on their relative position.  Here the complex
 * numbers are consecutive pairs z_i = x[2i] + j x[2i+1], and row n of every
 * (b, h) -- position n -- becomes z_i * (cos[n][i] + j sin[n][i]), computed in
 * fp32 and rounded to nearest-even bf16.  The tables carry any frequency
 * schedule (the usual one turns pair i by n * 10000^(-2i/d) radians).
 *
 *   x          [B][H][N][d] bf16                                   (read)
 *   out        [B][H][N][d] bf16; may be x itself (in place)      (written)
 *   rope_cos,  [N][d/2] float32 cosine / sine of each (position,   (read)
 *   rope_sin   pair) angle
 *   d          64 or 128;  dtype FA_BF16
 *
 * Returns FA_OK, FA_ERR_INVALID (null pointer, sizes < 1), FA_ERR_UNSUPPORTED
 * (d, dtype), or FA_ERR_HIP.
 */
fa_status fa_rope(const void* x, void* out, const float* rope_cos, const float* rope_sin,
                  int B, int H, int N, int d, int dtype, void* stream);

/*
 * fa_fwd_rope_workspace_size - bytes of workspace fa_fwd_rope needs:
 * B * H * N * d * 2 (the rotated keys).  0 if the sizes are invalid.
 */
size_t fa_fwd_rope_workspace_size(int B, int H, int N, int d);

/*
 * fa_fwd_rope - fa_fwd on RoPE-rotated queries and keys, the query rotation
 * fused into the attention kernel.
 *
 * Kernel fusion ("LLM study notes", kernel fusion section) saves the global
 * memory round trip of an intermediate.  Each work group rotates its query
 * rows once, in registers, as it loads them (the rotated queries never reach
 * HBM).  The keys are rotated once per head into the workspace (fa_rope's
 * kernel) before the attention kernel runs: every query block of a head
 * reads every key tile, so rotating keys inside the attention kernel would
 * repeat each rotation N/128 times.  The result equals fa_fwd on
 * fa_rope(q) and fa_rope(k).
 *
 *   q, k       [B][H][N][d] bf16, NOT rotated; row n is at position n   (read)
 *   v, o, lse, B, H, N, d, causal, scale, stream   as in fa_fwd (bf16 only)
 *   rope_cos, rope_sin   as in fa_rope ([N][d/2] float32)                  (read)
 *   workspace  device scratch of at least fa_fwd_rope_workspace_size(B, H, N, d)
 *              bytes, owned by the caller; contents on entry do not matter;
 *              not shared with a call running on another stream.
 *
 * Returns FA_OK, FA_ERR_INVALID (fa_fwd's checks, null tables, workspace NULL
 * or too small), FA_ERR_UNSUPPORTED (d, dtype), or FA_ERR_HIP.
 */
fa_status fa_fwd_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                      const float* rope_cos, const float* rope_sin,
                      int B, int H, int N, int d, int causal, float scale, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_string(int status);

/* hipError_t of the last FA_ERR_HIP returned on the calling thread (0 if none). */
int fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
