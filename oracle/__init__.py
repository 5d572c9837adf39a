"""CPU oracle for the MoE-layer hot path (test infrastructure, not product code).

A plain, slow, float64 NumPy implementation of what the layer computes: router,
top-k selection and weights, the stable expert-major schedule, MXFP8
quantisation, the per-expert SwiGLU FFN, the weighted combine, and the backward
pass with transposed-operand requantisation.  It is written from the published
description of Cursor's Mixture-of-Kittens MoE megakernel (a DeepSeek-V3-style
MoE layer computed in MXFP8, deterministic, with a reusable expert schedule:
knowledge card "Mixture-of-Kittens——面向NVL72的开源MoE训练megakernel",
section 方法/产品要点) and from the OCP Microscaling (MX) v1.0 format definition
for MXFP8.  Where the pages leave a step open, the reading taken is stated in
the docstring of the function that takes it.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``mixture_experts_layer_schedule_amd``) and never imports it.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
something other than itself (hand values of the MX format, a library float8
codec, exact sums, brute force on tiny inputs, closed forms and invariants,
central finite differences of the unquantised layer).
"""
from .mxfp8 import (  # noqa: F401
    BLOCK,
    E4M3_MAX,
    dequantize,
    e4m3_decode,
    e4m3_encode,
    quantize,
    quantize_range,
    requantize,
    scale_exponent,
)
from .layer import (  # noqa: F401
    LayerForward,
    LayerBackward,
    build_schedule,
    combine,
    expert_backward,
    expert_forward,
    layer_backward,
    layer_forward,
    oracle_experts,
    router_backward,
    router_logits,
    routing_weights,
    select_topk,
    swiglu,
    swiglu_backward,
    token_quantize,
    token_requant,
)
