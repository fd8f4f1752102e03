"""MI355X (gfx950) prefill routed-expert product: q8_1 quantize-scatter,
Q2_0/NL4 expert products on fp16 matrix cores (v_mfma_f32_32x32x16_f16: the
int8 values and the scaled 2-bit weights are exact in fp16, so each 32-value
block's dot comes out exact) with a per-32-value fp32 epilogue, a fused
swiglu + q8_1 pass and the routing-weighted combine, behind the C ABI in
include/moe_prefill.h.

The HIP library is loaded on first use; if it has not been built, that use
raises ImportError.
"""
from ._lib import (MOE_W_GU_INTERLEAVED, MOE_W_NL4, MOE_W_Q2_0, MOE_W_TILED, MoeError, Plan,
                   Weights, expert_down, expert_gate_up, expert_gate_up_swiglu_q8, moe_combine,
                   moe_debug_block_dots, moe_plan_device_bytes, moe_prefill_plan,
                   moe_prefill_plan_device, moe_q8_1_bytes, moe_weight_bytes, moe_weights_pack,
                   quantize_scatter, swiglu_q8)

__all__ = ["MOE_W_Q2_0", "MOE_W_NL4", "MOE_W_TILED", "MOE_W_GU_INTERLEAVED", "MoeError", "Plan",
           "Weights", "moe_weights_pack", "moe_prefill_plan", "moe_prefill_plan_device",
           "quantize_scatter", "expert_gate_up", "swiglu_q8", "expert_gate_up_swiglu_q8",
           "expert_down", "moe_combine", "moe_debug_block_dots", "moe_q8_1_bytes",
           "moe_weight_bytes", "moe_plan_device_bytes"]
