"""Plain CPU oracle for calibration-free top-k channel selection in routed MoE experts.

TEST INFRASTRUCTURE ONLY. The test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers; the library and its Python binding never
import, call or link anything in this package, and this package imports nothing
from the library.

See ``oracle.moe_oracle`` for the computation and the passages it follows.
"""
from .moe_oracle import (  # noqa: F401
    ORACLE_CONSTANTS,
    SCORE_KINDS,
    OracleLayer,
    bf16_bits_to_f64,
    compensation,
    expert_swiglu_selected,
    f64_to_bf16_bits,
    preacts_from_dots,
    prepare_expert,
    quantize_token,
    residual_rmsnorm,
    route,
    router_logits,
    score_channels,
    score_from_preacts,
    select_threshold,
    select_topk,
    silu_pinned,
    sketch_preacts,
    ternary_sketch_row,
)
