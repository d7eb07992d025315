"""fp64 CPU oracle for paged latent attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library itself.
"""

from .mla_oracle import (  # noqa: F401
    absorb_query,
    append_kv,
    append_kv_fp8,
    attention,
    attention_fp8,
    attention_loops,
    dequantize_cache,
    fp8_e4m3_decode,
    fp8_e4m3_encode,
    fp8_quantize_rows,
    gather_row_keys,
    head_matmul,
    kv_lengths,
    merge_state,
    up_project,
    validate,
    visible_keys,
    widen,
)
