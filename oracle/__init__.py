"""fp64 CPU oracle for absorbed MLA decode — test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the HIP library.  oracle.fp8_cache holds the fp8
latent-cache format (quantisation, dequantisation, row layout).
"""
from . import fp8_cache  # noqa: F401
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import (absorb_query, absorbed_decode, append_rows, cache_bytes,  # noqa: F401
                         cache_elements_per_token_layer, causal_attention, expanded_prefill, combine_splits, decode_layer,
                         default_scale, expanded_decode, gather_rows, head_block,
                         latent_attention, linear, logsumexp, output_projection,
                         page_slot, paged_decode, rope, softmax, up_project_values)
