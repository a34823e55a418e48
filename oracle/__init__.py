"""CPU oracle for the CLO decode step (test infrastructure; see clo_oracle)."""
from .clo_oracle import (  # noqa: F401
    as_f64,
    attend,
    decode_layer,
    decode_steps_unit,
    decode_unit,
    group_cosine,
    plan_persistent,
    reuse_decision,
    select_topk,
    token_scores,
)
