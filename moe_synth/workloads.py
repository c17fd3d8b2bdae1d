"""The five workload shapes of the routed-MoE expert path.

Shapes follow the model geometry the Strata pages describe: hidden 2560,
512 routed experts per layer, top-10, 48 layers (lcz.me/topic/2153,
section 三 "Strata 的源码绑死了什么"; blog.5616760.com/0039.html, section 五
"MoE 的本质"), the 1+3-token MTP verify window (devotd.net "Strata memory
tiers", section "用草拟 token 提高生成速度的 MTP"), the 8192-token prefill
chunk (same page, section "读取提示与写出回答时"; blog.5616760.com/0039.html
section 七) and the DeepSeek-V4-Flash layer with 256 routed experts plus one
shared expert (lcz.me/topic/2153, section 一).  Expert widths, block formats
and value distributions are the workload definitions the pages leave open.

Only storage parameters live here (bits per code, bytes per block); the
dequantisation offsets belong to the arithmetic and are defined separately
by each implementation.
"""

from dataclasses import dataclass
from typing import Dict

# fmt -> (bits per code, code bytes per 32-weight block); 5 is MXFP4 (4-bit
# E2M1 elements with one E8M0 scale byte per block of 32, OCP Microscaling
# Formats v1.0), the others the Q2/Q3/Q4 blocks with an fp16 scale
FORMATS: Dict[int, tuple] = {2: (2, 8), 3: (3, 12), 4: (4, 16), 5: (4, 16)}
MXFP4 = 5
BLOCK = 32          # weights per quantised block
# bytes of the per-block scale stored after the codes: fp16, or E8M0 for MXFP4
SCALE_BYTES: Dict[int, int] = {2: 2, 3: 2, 4: 2, 5: 1}


def canonical_block_bytes(fmt: int) -> int:
    """Bytes of one canonical block: codes followed by the scale."""
    return FORMATS[fmt][1] + SCALE_BYTES[fmt]


@dataclass(frozen=True)
class Workload:
    name: str
    hidden: int          # H
    inter: int           # I, expert intermediate width
    n_experts: int       # E routed experts per layer
    top_k: int           # k
    fmt: int             # 2 / 3 / 4 bit codes
    tokens: int          # T per call
    biased: bool         # log-Zipf router bias present
    n_shared: int = 0    # always-on shared experts (0 or 1)
    n_layers: int = 1    # layers in the stack
    steps: int = 1       # decode steps in the stream (stack workload)
    zipf_s: float = 1.1
    d_sigma: float = 0.02  # expert scales d = |N(0, d_sigma^2)|

    def expert_bytes(self) -> int:
        blk = canonical_block_bytes(self.fmt)
        return 3 * self.inter * (self.hidden // BLOCK) * blk

    def router_bytes(self) -> int:
        return 4 * self.n_experts * self.hidden


WORKLOADS: Dict[str, Workload] = {
    # single layer, one token, Q2, unbiased router
    "decode_t1_q2": Workload("decode_t1_q2", 2560, 512, 512, 10, 2, 1, False),
    # same layer, 1+3-token MTP verify batch, Zipf-skewed router
    "mtp_verify_t4_q2": Workload("mtp_verify_t4_q2", 2560, 512, 512, 10, 2, 4, True),
    # same layer, 6-token verify of a prompt-lookup draft (1 + 5 tokens)
    "lookup_verify_t6_q2": Workload("lookup_verify_t6_q2", 2560, 512, 512, 10, 2, 6, True),
    # 48-layer Q3 stack, single-token decode stream of 256 steps
    # (scales a quarter of the single-layer ones: with d ~ |N(0, 0.02^2)| each
    # layer's output grows as the square of its input and the residual stream
    # overflows fp32 by about layer 8; at 0.005 each layer moves h by ~2%)
    "stack48_q3_decode": Workload("stack48_q3_decode", 2560, 512, 512, 10, 3, 1, True,
                                  n_layers=48, steps=256, d_sigma=0.005),
    # skinny batches between the one-pass decode and the 8K chunk (batched
    # slots, longer verify windows), same layer and Zipf-skewed router
    "skinny_t16_q2": Workload("skinny_t16_q2", 2560, 512, 512, 10, 2, 16, True),
    "skinny_t32_q2": Workload("skinny_t32_q2", 2560, 512, 512, 10, 2, 32, True),
    "skinny_t64_q2": Workload("skinny_t64_q2", 2560, 512, 512, 10, 2, 64, True),
    # 8192-token prefill chunk through one Q2 layer, Zipf-skewed router
    "prefill_t8192_q2": Workload("prefill_t8192_q2", 2560, 512, 512, 10, 2, 8192, True),
    # the opt-in 32768-token prefill chunk through the same layer
    "prefill_t32768_q2": Workload("prefill_t32768_q2", 2560, 512, 512, 10, 2, 32768, True),
    # DeepSeek-V4-Flash-shaped layer, Q4, 256 routed + 1 shared, top-6
    "deepseek_q4_t1": Workload("deepseek_q4_t1", 4096, 2048, 256, 6, 4, 1, True, n_shared=1),
    "deepseek_q4_t2048": Workload("deepseek_q4_t2048", 4096, 2048, 256, 6, 4, 2048, True,
                                  n_shared=1),
    # the same layer with MXFP4 experts (the format of the pages' DeepSeek
    # suites): E2M1 codes, E8M0 block scales 2^(floor(log2 |N(0, 0.02^2)|) - 2)
    "deepseek_mxfp4_t1": Workload("deepseek_mxfp4_t1", 4096, 2048, 256, 6, 5, 1, True, n_shared=1),
    "deepseek_mxfp4_t2048": Workload("deepseek_mxfp4_t2048", 4096, 2048, 256, 6, 5, 2048, True,
                                     n_shared=1),
}
