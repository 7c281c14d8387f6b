"""fp64 CPU oracle for differential attention -- test infrastructure only.

Imported by the tests, the smoke check and the benchmark's CPU-baseline leg;
never by the library itself.
"""
from .diffattn_oracle import (  # noqa: F401
    gda_combine,
    gda_decode,
    gda_forward,
    gda_heads,
    gda_sequence,
    gqa_kv_head,
    lambda_init,
    out_projection,
    sigmoid,
    softmax_rows,
    v1_attention,
    v1_backward,
    v1_decode,
    v1_forward,
    v1_head,
    v1_head_backward,
    v1_norm,
    v1_norm_backward,
    v2_backward,
    v2_attention_param_counts,
    v2_backward_key_rows,
    v2_backward_query_rows,
    v2_combine,
    v2_decode,
    v2_forward,
    v2_forward_stats,
    v2_heads,
    v2_lambda_logits,
    v2_sequence,
    v2_sequence_backward,
    v2_varlen_forward,
)
