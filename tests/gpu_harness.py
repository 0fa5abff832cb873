"""Helpers for the GPU parity tests: cases, running the HIP path, comparing
with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

from workloads import (TINY_TOP2_FP32, MIXTRAL_PREFILL, MIXTRAL_DECODE, DEEPSEEK_V3, DEEPSEEK_V3_BALANCED,
                       SWITCH_SKEWED,
                       make_inputs)

# Tolerances of the parity bar: max|gpu - ref| / max|ref|.
TOL = {"bf16": 2e-2, "f32": 1e-5}

# Reduced sizes the oracle finishes in seconds; each still spans several GEMM
# tiles per expert (or many small ragged segments) and a ragged tail.
SMALL = {
    "tiny_top2_fp32": TINY_TOP2_FP32,
    "mixtral_prefill_small": MIXTRAL_PREFILL.scaled(name="mixtral_prefill_small", n_tokens=1000, d_model=256,
                                                    d_ff=384),
    "mixtral_decode_small": MIXTRAL_DECODE.scaled(name="mixtral_decode_small", d_model=256, d_ff=384),
    "deepseek_v3_small": DEEPSEEK_V3.scaled(name="deepseek_v3_small", n_tokens=1024, d_model=512, d_ff=128,
                                            d_ff_shared=192),
    "switch_skewed_small": SWITCH_SKEWED.scaled(name="switch_skewed_small", n_tokens=2048, d_model=256,
                                                d_ff=512),
}

FULL = {c.name: c for c in (MIXTRAL_PREFILL, MIXTRAL_DECODE, DEEPSEEK_V3, DEEPSEEK_V3_BALANCED, SWITCH_SKEWED)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max() if ref.size else 0.0
    if den == 0:
        return float(np.abs(got - ref).max()) if ref.size else 0.0
    return float(np.abs(got - ref).max() / den)


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def run_layer(cfg, inp=None, device="cuda", runs=1):
    """Upload inputs, run moe_forward `runs` times; return (inputs, host outputs of the last run, layer)."""
    import torch
    from mixture_experts_layer_histogram_amd import MoELayer, upload_inputs

    if inp is None:
        inp = make_inputs(cfg)
    dev = upload_inputs(inp, device)
    layer = MoELayer(cfg, dev, device)
    outs = None
    for _ in range(runs):
        outs = layer.forward()
    torch.cuda.synchronize()
    return inp, {k: host(v) for k, v in outs.items()}, layer
