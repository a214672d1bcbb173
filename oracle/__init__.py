"""CPU oracle for the LatentMoE MXFP4 (w4a16) routed-expert layer.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, float64 statement
of what the layer computes. It is imported by the test suite, by the smoke
check in __graft_entry__.py and by the bench's CPU-baseline leg, and by
nothing else: the product path (the HIP library and its Python binding)
never imports, links or calls it, and it shares no code with that path. Inputs come from the seeded
generators in the separate `workloads` package.
"""
from .lmoe_oracle import (  # noqa: F401
    E2M1_MAGNITUDES,
    e2m1_table,
    e8m0_scale,
    dequant_mxfp4,
    bf16_from_f64,
    f64_from_bf16,
    f32_round,
    router_logits,
    topk_select,
    softmax_selected,
    permute_routes,
    glu_ffn,
    combine,
    forward,
    forward_tokens,
    ACT_FORMATS,
    ACT_EMAX,
    e4m3_table,
    round_to_format,
    format_values,
    mx_quantize,
    mx_dequant,
    act_values,
    RMS_EPS,
    shared_gate_up_rows,
    moe_input,
    rms_norm,
    moe_tail,
    block_forward,
)
