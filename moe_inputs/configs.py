"""The five workload configurations of the sparse-MoE expert-FFN layer.

Shapes come from the pages:
  * Qwen3.8-Flash-Next: 48 layers x 512 experts, about 10 active per token,
    hidden 2560, expert FF 640 (teardown page "Strata 引擎深度拆解", section 二;
    geometry literals quoted on "Strata 改源码去跑 DeepSeek V4 Flash？", section 三).
  * DeepSeek-V4-Flash: 43 layers, hidden 4096, 256 routed + 1 shared expert,
    6 active, expert FF 2048, fused expert tensors 256x2048x4096
    ("Strata 改源码去跑 DeepSeek V4 Flash？", section 二 GGUF table).
  * Decode windows of 1/4/8 tokens stand for the multi-token verify window
    (teardown page, section 二.1: the draft guesses 3-5 tokens, one forward
    verifies them).

Input recipe (synthetic; no dataset or trained weight is involved):
  activations bf16 N(0,1); router weights bf16 N(0,0.02); experts are
  quantised N(0,0.02) draws; bias per config (none, Zipf(s) over a seeded
  per-layer permutation of ranks, or N(0, sigma)).
"""
from dataclasses import dataclass, field
from typing import Tuple

Q4B32 = 1
Q2B32 = 2
Q2B64 = 3  # 2-bit codes, one fp16 scale per 64 weights: 2.25 bits per weight

BIAS_NONE = 0
BIAS_ZIPF = 1
BIAS_NORMAL = 2


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: Tuple[int, ...]      # tokens per call (decode windows or prefill chunk)
    H: int                  # hidden
    F: int                  # expert FF dim
    E: int                  # routed experts
    S: int                  # shared experts (0 or 1)
    k: int                  # top-k
    L: int                  # layers
    fmt: int                # Q4B32, Q2B32 or Q2B64
    bias_kind: int
    bias_param: float
    seeds: Tuple[int, ...] = field(default=(1,))
    description: str = ""

    @property
    def block_bytes(self) -> int:
        return 10 if self.fmt == Q2B32 else 18

    @property
    def block_weights(self) -> int:
        return 64 if self.fmt == Q2B64 else 32

    @property
    def expert_bytes(self) -> int:
        return 3 * self.H * self.F // self.block_weights * self.block_bytes

    @property
    def router_bytes(self) -> int:
        return self.E * self.H * 2


C1 = MoEConfig("C1", (4,), 256, 128, 16, 0, 2, 1, Q4B32, BIAS_NONE, 0.0, (1,),
               "tiny layer: hidden 256, 16 experts, top-2, FF 128, 4 tokens, q4b32")
C2 = MoEConfig("C2", (4,), 2560, 640, 512, 0, 10, 1, Q2B32, BIAS_ZIPF, 1.1, (1, 2, 3),
               "Qwen-shaped decode layer: hidden 2560, 512 experts, top-10, FF 640, window 4, q2b32, Zipf(1.1) bias")
C3 = MoEConfig("C3", (1, 4, 8), 2560, 640, 512, 0, 10, 48, Q2B32, BIAS_ZIPF, 1.1, (1, 2, 3),
               "Qwen-shaped 48-layer decode chain with residual, windows 1/4/8, q2b32, per-layer Zipf(1.1)")
C4 = MoEConfig("C4", (1, 4, 8), 4096, 2048, 256, 1, 6, 43, Q4B32, BIAS_NORMAL, 0.5, (1, 2, 3),
               "DeepSeek-shaped 43-layer decode chain, 256+1 experts, top-6, FF 2048, q4b32, bias N(0,0.5)")
# The Qwen-shaped layer and chain with the 2.25-bit expert format (one fp16
# scale per 64 weights): 1,382,400 bytes per expert, the size of the pages'
# 2-bit expert blob, and 48 x 512 experts in 33.97 GB.
C2_Q2B64 = MoEConfig("C2_q2b64", (4,), 2560, 640, 512, 0, 10, 1, Q2B64, BIAS_ZIPF, 1.1, (1, 2, 3),
                     "Qwen-shaped decode layer as C2 with q2b64 experts (2.25 bits per weight)")
C3_Q2B64 = MoEConfig("C3_q2b64", (1, 4, 8), 2560, 640, 512, 0, 10, 48, Q2B64, BIAS_ZIPF, 1.1, (1, 2, 3),
                     "Qwen-shaped 48-layer decode chain as C3 with q2b64 experts (2.25 bits per weight)")
# Zipf exponent for the prefill chunk: the smallest multiple of 0.1 for which the
# seed-1 routing (computed by the oracle) sends more than 500 tokens to some
# expert.  Written by tests/golden/make_golden.py; see tests/golden/c5_zipf.json.
C5_ZIPF_S = 0.3
C5 = MoEConfig("C5", (4096,), 4096, 2048, 256, 1, 6, 1, Q4B32, BIAS_ZIPF, C5_ZIPF_S, (1, 2, 3),
               "DeepSeek-shaped prefill chunk: 4096 tokens, 256+1 experts, top-6, FF 2048, q4b32, Zipf-skewed")

CONFIGS = {c.name: c for c in (C1, C2, C3, C4, C5, C2_Q2B64, C3_Q2B64)}
