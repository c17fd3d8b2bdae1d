"""CPU oracle (fp64, NumPy) for the routed-MoE expert path.

TEST INFRASTRUCTURE: imported only by tests/, the package smoke check and
the benchmark's CPU-baseline leg.  The product path never imports it.
"""

from .moe_oracle import (  # noqa: F401
    OFFSET, CODE_BYTES, CODE_BITS, SCALE_BYTES, MXFP4, e2m1_value, e8m0_value, block_bytes, unpack_codes,
    dequant_blocks, split_record,
    dequant_expert, router_logits, select_topk, routing_weights, silu, expert_ffn,
    permute, route, moe_layer, moe_stack,
)
