"""INT4 group-128 top-k MoE SwiGLU FFN forward for AMD Instinct MI355X (gfx950).

The computation lives in the HIP library libq4moe.so (C ABI in include/q4moe.h);
this package is its thin Python binding.  Importing the package loads the library
and raises ImportError if it has not been built.
"""
from ._lib import (  # noqa: F401
    Q4_BF16, Q4_F16, Q4_F32, Q4_W4A8, Q4_W4A16, Q4_W8A8, Q4_REPACK_GATE_UP, Q4_REPACK_PLAIN, Q4_NOALLOC_SCRATCH_BYTES,
    LoRALayer, MoELayer, Q4Error, act_quant_int8, expert_bits_apex, expert_bits_by_hotness, expert_groups_by_hotness, int4_linear_forward, int4_w4a8_group_acc,
    moe_int4_ffn_debug, moe_int4_ffn_forward, moe_int4_ffn_forward_noalloc, moe_int4_ffn_plan, moe_lora_ffn_forward, moe_permute, moe_route_topk, q4_device_bytes, q4_device_bytes_grouped, q4_repack_device, q4_repack_device_grouped,
    int2_w2a8_group_acc, int8_w8a8_group_acc, q2_device_bytes, q2_repack_device, quantize_int2_g128, q8_device_bytes, q8_repack_device, quantize_int4_g128, quantize_int4_grouped, quantize_int8_g128, version,
)
