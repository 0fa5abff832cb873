"""Seeded synthetic workloads for the MoE layer: presets (:mod:`.configs`) and
input generators (:mod:`.gen`).  Holds no part of the layer's arithmetic."""
from .configs import (CONFIGS, BY_NAME, MoEConfig, TINY_TOP2_FP32, MIXTRAL_PREFILL, MIXTRAL_DECODE,
                      DEEPSEEK_V3, DEEPSEEK_V3_BALANCED, SWITCH_SKEWED, GATE_TOPK_SOFTMAX, GATE_SOFTMAX_RENORM,
                      GATE_SWITCH_TOP1, ACT_SWIGLU, ACT_GELU)
from .gen import LayerInputs, make_inputs, gen_expert, round_to_bf16_bits
