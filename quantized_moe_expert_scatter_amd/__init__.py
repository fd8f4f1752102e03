"""MI355X (gfx950) prefill routed-expert product: q8_1 quantize-scatter,
Q2_0/NL4 expert products on int8 MFMA with a per-32-value fp32 epilogue, and a
fused swiglu + q8_1 pass, behind the C ABI in include/moe_prefill.h.

The HIP library is loaded on first use; if it has not been built, that use
raises ImportError.
"""
from ._lib import (MOE_W_NL4, MOE_W_Q2_0, MoeError, Plan, Weights, expert_down, expert_gate_up,
                   moe_debug_block_dots, moe_plan_device_bytes, moe_prefill_plan, moe_q8_1_bytes,
                   moe_weight_bytes, quantize_scatter, swiglu_q8)

__all__ = ["MOE_W_Q2_0", "MOE_W_NL4", "MoeError", "Plan", "Weights", "moe_prefill_plan",
           "quantize_scatter", "expert_gate_up", "swiglu_q8", "expert_down",
           "moe_debug_block_dots", "moe_q8_1_bytes", "moe_weight_bytes", "moe_plan_device_bytes"]
