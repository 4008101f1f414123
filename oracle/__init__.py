"""CPU oracle -- test infrastructure only (tests/, smoke(), bench.py's cpu_baseline).

Plain float64 attention written from the definition; shares no code with the
HIP path and imports nothing from it.
"""
from .attention import (  # noqa: F401
    attention_backward_fp64, attention_bruteforce, attention_fp64, paged_decode_fp64,
    paged_gather_fp64, paged_prefill_fp64, tree_ancestors, tree_decode_fp64, rope_fp64,
    attention_rope_fp64,
)
