"""Seeded, synthetic inputs for the MoE-layer workloads.

This module draws numbers and nothing else: it holds none of the layer's
arithmetic.  Both the GPU path (which copies these exact bytes to the device)
and the fp64 CPU oracle (which decodes the same bytes) read its output.

Recipe (every tensor is reproducible on its own, so one expert can be
regenerated without the others):

* generator: numpy ``PCG64`` seeded with ``SeedSequence(cfg.seed,
  spawn_key=(tensor_id, expert_id))``;
* draws are float32 samples, stored as IEEE fp32 (``dtype == "f32"``) or
  rounded to bfloat16 with round-to-nearest-even and kept as the raw 16-bit
  patterns (``dtype == "bf16"``);
* ``x ~ N(0, 1)``; router ``W_r ~ N(0, 1/d)``;
* ``init == "normal"``: expert weights ``~ N(0, 1/fan_in)``;
* ``init == "uniform_experts"``: expert weights and biases ``~ U(+-1/sqrt(fan_in))``
  (the ``torch.nn.Linear`` default, as in the glossary page's expert form);
* ``init == "torch_seed0"``: the glossary page's own construction, drawn with
  torch's CPU generator after ``manual_seed(0)``: eight experts
  Linear(d, 4d) / GELU / Linear(4d, d) first, then the bias-free router
  Linear(d, E), then ``randn(N, d)`` tokens;
* selection bias ``~ U(-r, r)`` per expert (fp32; zeros when ``r == 0`` and the layer has a
  bias step); a fixed router logit offset
  ``(expert, delta)`` becomes an fp32 ``logit_bias[E]`` vector.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import MoEConfig

# tensor ids used in the spawn key
T_X, T_ROUTER, T_W1, T_W3, T_W2, T_B1, T_B2, T_SH_W1, T_SH_W3, T_SH_W2, T_SEL_BIAS = range(11)


def round_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 samples -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _rng(cfg: MoEConfig, tensor_id: int, expert_id: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(cfg.seed, spawn_key=(tensor_id, expert_id))))


def _store(cfg: MoEConfig, a32: np.ndarray) -> np.ndarray:
    return a32.astype(np.float32) if cfg.dtype == "f32" else round_to_bf16_bits(a32)


def _normal(cfg, tid, eid, shape, std):
    z = _rng(cfg, tid, eid).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    return _store(cfg, z.reshape(shape))


def _uniform(cfg, tid, eid, shape, bound):
    u = _rng(cfg, tid, eid).random(int(np.prod(shape)), dtype=np.float32)
    u = (u * np.float32(2.0) - np.float32(1.0)) * np.float32(bound)
    return _store(cfg, u.reshape(shape))


@dataclass
class LayerInputs:
    """Host copies of one layer's inputs.  bf16 tensors are uint16 bit patterns."""
    cfg: MoEConfig
    x: np.ndarray                     # [N, d]
    w_router: np.ndarray              # [E, d]
    logit_bias: np.ndarray | None     # [E] fp32 or None
    sel_bias: np.ndarray | None       # [E] fp32 or None
    w1: np.ndarray | None = None      # [E, F, d]   (None until materialised)
    w3: np.ndarray | None = None      # [E, F, d]   (SwiGLU only)
    w2: np.ndarray | None = None      # [E, d, F]
    b1: np.ndarray | None = None      # [E, F]      (ffn_bias only)
    b2: np.ndarray | None = None      # [E, d]
    sh_w1: np.ndarray | None = None   # [Fs, d]
    sh_w3: np.ndarray | None = None   # [Fs, d]
    sh_w2: np.ndarray | None = None   # [d, Fs]

    def expert(self, e: int) -> dict:
        """One expert's tensors; drawn on demand when not materialised."""
        if self.w1 is not None:
            out = {"w1": self.w1[e], "w2": self.w2[e]}
            if self.w3 is not None:
                out["w3"] = self.w3[e]
            if self.b1 is not None:
                out["b1"] = self.b1[e]
                out["b2"] = self.b2[e]
            return out
        return gen_expert(self.cfg, e)


def gen_expert(cfg: MoEConfig, e: int) -> dict:
    """Draw expert ``e``'s weights (and biases) for ``cfg``."""
    d, F = cfg.d_model, cfg.d_ff
    if cfg.init == "torch_seed0":
        raise ValueError("torch_seed0 experts are materialised by make_inputs")
    out = {}
    if cfg.init == "uniform_experts":
        out["w1"] = _uniform(cfg, T_W1, e, (F, d), 1.0 / math.sqrt(d))
        out["w2"] = _uniform(cfg, T_W2, e, (d, F), 1.0 / math.sqrt(F))
        if cfg.act == "swiglu":
            out["w3"] = _uniform(cfg, T_W3, e, (F, d), 1.0 / math.sqrt(d))
        if cfg.ffn_bias:
            out["b1"] = _uniform(cfg, T_B1, e, (F,), 1.0 / math.sqrt(d))
            out["b2"] = _uniform(cfg, T_B2, e, (d,), 1.0 / math.sqrt(F))
    else:
        out["w1"] = _normal(cfg, T_W1, e, (F, d), 1.0 / math.sqrt(d))
        out["w2"] = _normal(cfg, T_W2, e, (d, F), 1.0 / math.sqrt(F))
        if cfg.act == "swiglu":
            out["w3"] = _normal(cfg, T_W3, e, (F, d), 1.0 / math.sqrt(d))
        if cfg.ffn_bias:
            out["b1"] = _normal(cfg, T_B1, e, (F,), 1.0 / math.sqrt(d))
            out["b2"] = _normal(cfg, T_B2, e, (d,), 1.0 / math.sqrt(F))
    return out


def _torch_seed0_inputs(cfg: MoEConfig) -> LayerInputs:
    """The glossary page's construction, drawn with torch's CPU generator."""
    import torch  # CPU only; used here as a random-number source

    d, E, F, N = cfg.d_model, cfg.n_experts, cfg.d_ff, cfg.n_tokens
    with torch.random.fork_rng(devices=[]):
        torch.manual_seed(0)
        experts = [torch.nn.Sequential(torch.nn.Linear(d, F), torch.nn.GELU(), torch.nn.Linear(F, d))
                   for _ in range(E)]
        router = torch.nn.Linear(d, E, bias=False)
        x = torch.randn(N, d)
    w1 = np.stack([m[0].weight.detach().numpy() for m in experts]).astype(np.float32)
    b1 = np.stack([m[0].bias.detach().numpy() for m in experts]).astype(np.float32)
    w2 = np.stack([m[2].weight.detach().numpy() for m in experts]).astype(np.float32)
    b2 = np.stack([m[2].bias.detach().numpy() for m in experts]).astype(np.float32)
    return LayerInputs(cfg=cfg, x=x.numpy().astype(np.float32).copy(),
                       w_router=router.weight.detach().numpy().astype(np.float32).copy(),
                       logit_bias=None, sel_bias=None, w1=w1, w2=w2, b1=b1, b2=b2)


def make_inputs(cfg: MoEConfig, materialize_experts: bool = True,
                threads: int | None = None) -> LayerInputs:
    """Draw every input of ``cfg``.  With ``materialize_experts=False`` the
    expert weights are left to :meth:`LayerInputs.expert` (drawn per expert)."""
    if cfg.init == "torch_seed0":
        if cfg.dtype != "f32":
            raise ValueError("torch_seed0 construction is fp32")
        return _torch_seed0_inputs(cfg)
    N, d, E, F, Fs = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.d_ff, cfg.d_ff_shared
    x = _normal(cfg, T_X, 0, (N, d), 1.0)
    w_router = _normal(cfg, T_ROUTER, 0, (E, d), 1.0 / math.sqrt(d))
    logit_bias = None
    if cfg.logit_offset is not None:
        logit_bias = np.zeros(E, np.float32)
        logit_bias[cfg.logit_offset[0]] = np.float32(cfg.logit_offset[1])
    sel_bias = None
    if cfg.sel_bias_range > 0:
        u = _rng(cfg, T_SEL_BIAS, 0).random(E, dtype=np.float32)
        sel_bias = ((u * np.float32(2.0) - np.float32(1.0)) * np.float32(cfg.sel_bias_range)).astype(np.float32)
    elif cfg.gamma > 0:
        sel_bias = np.zeros(E, np.float32)   # a bias step with no starting bias: the balancing's first step
    inp = LayerInputs(cfg=cfg, x=x, w_router=w_router, logit_bias=logit_bias, sel_bias=sel_bias)
    if Fs > 0:
        inp.sh_w1 = _normal(cfg, T_SH_W1, 0, (Fs, d), 1.0 / math.sqrt(d))
        inp.sh_w3 = _normal(cfg, T_SH_W3, 0, (Fs, d), 1.0 / math.sqrt(d))
        inp.sh_w2 = _normal(cfg, T_SH_W2, 0, (d, Fs), 1.0 / math.sqrt(Fs))
    if materialize_experts:
        st = np.float32 if cfg.dtype == "f32" else np.uint16
        inp.w1 = np.empty((E, F, d), st)
        inp.w2 = np.empty((E, d, F), st)
        if cfg.act == "swiglu":
            inp.w3 = np.empty((E, F, d), st)
        if cfg.ffn_bias:
            inp.b1 = np.empty((E, F), st)
            inp.b2 = np.empty((E, d), st)

        def fill(e):
            t = gen_expert(cfg, e)
            for k, v in t.items():
                getattr(inp, k)[e] = v

        n = threads or min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(max_workers=max(1, n)) as ex:
            list(ex.map(fill, range(E)))
    return inp
