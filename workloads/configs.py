"""Named MoE-layer workloads (shapes, gate rule, balancing options).

Five presets describe the layers this library is measured and checked on:

* ``tiny_top2_fp32``   the seeded six-token, eight-expert top-2 example printed on
  the Ultralytics glossary page ("Load balancing and expert capacity" section),
  fp32, GELU experts with biases, no residual.
* ``mixtral_prefill``  Mixtral-8x7B-shaped prefill: 4096 tokens, d=4096, 8 SwiGLU
  experts of width 14336, top-2, softmax over the selected logits, residual add.
* ``mixtral_decode``   the same layer at 16 tokens (weight streaming bound).
* ``deepseek_v3``      DeepSeek-V3-shaped fine-grained layer: 8192 tokens, d=7168,
  256 routed SwiGLU experts of width 2048 plus one shared expert, softmax over
  all experts, top-8 of (score + per-expert selection bias), renormalised raw
  scores as gates, then the aux-loss-free +-gamma bias step.
* ``switch_skewed``    Switch-style top-1 with capacity 1.25*N/E: 16384 tokens,
  d=2048, 64 GELU experts of width 8192, router logits offset so that about 90%
  of the argmax mass lands on expert 3; emits the auxiliary loss and the drop count.

Only shapes and options live here; :mod:`workloads.gen` draws the values.
"""
from __future__ import annotations

import dataclasses

import numpy as np
from dataclasses import dataclass

# Gate rules (what the router does with the logits z of one token).
GATE_TOPK_SOFTMAX = "topk_softmax"      # select top-k of z (+ selection bias); gate = softmax of the selected raw z
GATE_SOFTMAX_RENORM = "softmax_renorm"  # p = softmax(z); select top-k of p + bias; gate = p_S / sum(p_S)
GATE_SWITCH_TOP1 = "switch_top1"        # argmax z; gate = p[argmax] (not renormalised)

ACT_SWIGLU = "swiglu"
ACT_GELU = "gelu"


@dataclass(frozen=True)
class MoEConfig:
    name: str
    n_tokens: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    d_ff_shared: int = 0              # 0: no shared expert
    act: str = ACT_SWIGLU
    ffn_bias: bool = False            # expert Linear layers carry biases (GELU form only)
    gate_rule: str = GATE_TOPK_SOFTMAX
    capacity_factor: float = 0.0      # <= 0: unlimited capacity
    capacity_layout: str = "packed"   # "packed": experts' kept rows back to back; "padded": [E, C] rows
    capacity_priority: str = "slot"   # which slots an over-full expert keeps: "slot" (ascending t*k+j)
                                      # or "choice" (all first choices, then second choices, ...)
    dtype: str = "bf16"               # storage type of x, weights and out ("bf16" or "f32")
    residual: bool = True             # out = x + MoE(x)
    sel_bias_range: float = 0.0       # > 0: selection bias ~ U(-r, r) per expert
    logit_offset: tuple | None = None  # (expert, delta): fixed router logit offset
    gamma: float = 0.0                # > 0: emit the +-gamma bias step
    aux_loss: bool = False            # emit E * sum_e f_e * P_e
    init: str = "normal"              # "normal": W ~ N(0, 1/fan_in); "uniform": U(+-1/sqrt(fan_in))
    seed: int = 0

    def scaled(self, **kw) -> "MoEConfig":
        """The same layer kind at other sizes (tests use this for small cases)."""
        return dataclasses.replace(self, **kw)

    @property
    def n_slots(self) -> int:
        return self.n_tokens * self.top_k

    @property
    def capacity(self) -> int | None:
        """Per-expert capacity floor(cf * N / E), or None when unlimited."""
        if self.capacity_factor <= 0:
            return None
        # the factor as the C ABI carries it (fp32), then floor(cf * N / E) in double
        return int(float(np.float32(self.capacity_factor)) * self.n_tokens / self.n_experts)


TINY_TOP2_FP32 = MoEConfig(
    name="tiny_top2_fp32", n_tokens=6, d_model=32, n_experts=8, top_k=2, d_ff=128,
    act=ACT_GELU, ffn_bias=True, gate_rule=GATE_TOPK_SOFTMAX, dtype="f32",
    residual=False, init="torch_seed0", seed=1000)

MIXTRAL_PREFILL = MoEConfig(
    name="mixtral_prefill", n_tokens=4096, d_model=4096, n_experts=8, top_k=2, d_ff=14336,
    act=ACT_SWIGLU, gate_rule=GATE_TOPK_SOFTMAX, residual=True, seed=1001)

# Same weights and routing as the prefill layer (same seed), 16 tokens.
MIXTRAL_DECODE = MIXTRAL_PREFILL.scaled(name="mixtral_decode", n_tokens=16)

DEEPSEEK_V3 = MoEConfig(
    name="deepseek_v3", n_tokens=8192, d_model=7168, n_experts=256, top_k=8, d_ff=2048,
    d_ff_shared=2048, act=ACT_SWIGLU, gate_rule=GATE_SOFTMAX_RENORM, residual=True,
    sel_bias_range=0.05, gamma=1e-3, seed=1003)

# The same layer at the balancing's starting point (selection biases zero): routing by the
# scores alone, close to uniform over the experts (about 256 rows each).
DEEPSEEK_V3_BALANCED = DEEPSEEK_V3.scaled(name="deepseek_v3_balanced", sel_bias_range=0.0)

# delta = 3.7475 puts P(argmax = 3) at 0.900 for i.i.d. N(0,1) logits of 64 experts.
SWITCH_SKEWED = MoEConfig(
    name="switch_skewed", n_tokens=16384, d_model=2048, n_experts=64, top_k=1, d_ff=8192,
    act=ACT_GELU, ffn_bias=True, gate_rule=GATE_SWITCH_TOP1, capacity_factor=1.25,
    residual=True, logit_offset=(3, 3.7475), aux_loss=True, init="uniform_experts", seed=1004)

CONFIGS = [TINY_TOP2_FP32, MIXTRAL_PREFILL, MIXTRAL_DECODE, DEEPSEEK_V3, DEEPSEEK_V3_BALANCED, SWITCH_SKEWED]
BY_NAME = {c.name: c for c in CONFIGS}
