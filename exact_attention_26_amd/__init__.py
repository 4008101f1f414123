"""MI355X-native exact attention: FlashAttention-style forward and backward, paged-KV
decode, paged prefill, draft-tree verification and RoPE (standalone and fused).

The compute path is hand-written HIP for gfx950 behind a C ABI (``libfa.so``,
declared in ``include/fa.h``).  This package is the thin Python binding over
that library: it marshals torch tensors (device memory and the current HIP
stream) into the C calls and raises if a call reports an error.  Nothing here
computes attention; if the shared library is missing the calls raise.
"""
from ._binding import (  # noqa: F401
    FA_BF16, FA_ERR_TOO_LARGE, FA_F32, FA_NOALLOC_SCRATCH_BYTES, FaError, attention,
    attention_backward, fa_bwd, fa_bwd_workspace_size, fa_fwd, fa_paged_decode,
    fa_paged_decode_noalloc, fa_paged_decode_workspace_size, fa_paged_prefill, fa_status_string,
    fa_last_hip_error, fa_tree_decode, library_path, load_library, paged_decode, paged_prefill,
    tree_decode, fa_rope, fa_fwd_rope, fa_fwd_rope_workspace_size, rope, attention_rope,
)
