"""CPU oracle for the CLO decode step (test infrastructure; see clo_oracle)."""
from .clo_oracle import (  # noqa: F401
    as_f64,
    attend,
    decode_layer,
    decode_steps_unit,
    dequantize_row,
    decode_unit,
    group_cosine,
    pack_int4,
    plan_persistent,
    quant_max,
    quantize_row,
    quantized_rows,
    reuse_decision,
    select_blocks,
    select_topk,
    token_scores,
)
