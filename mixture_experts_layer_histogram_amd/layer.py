"""Device-side convenience around the C ABI: a config from any object with the
layer's attributes, host->device upload of layer inputs, and a layer object
that owns its workspace and calls ``moe_forward``."""
from __future__ import annotations

import numpy as np

from . import _lib


def config_from(c, n_tokens: int | None = None) -> _lib.MoeConfig:
    """Build the C config from an object carrying n_tokens, d_model, n_experts,
    top_k, d_ff, d_ff_shared, act, ffn_bias, gate_rule, capacity_factor, dtype,
    residual."""
    return _lib.make_config(c.n_tokens if n_tokens is None else n_tokens, c.d_model, c.n_experts, c.top_k,
                            c.d_ff, c.d_ff_shared, c.act, c.ffn_bias, c.gate_rule, c.capacity_factor,
                            c.dtype, c.residual, getattr(c, "capacity_layout", "packed"),
                            getattr(c, "capacity_priority", "slot"))


def to_device(a, device, dtype: str):
    """Host array -> device tensor.  bf16 arrays are uint16 bit patterns."""
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device, non_blocking=False)


def upload_inputs(inp, device) -> dict:
    """Copy a layer's host inputs (x, router, experts, biases, shared expert) to `device`."""
    dt = inp.cfg.dtype
    names = ["x", "w_router", "w1", "w3", "w2", "b1", "b2", "sh_w1", "sh_w3", "sh_w2"]
    out = {n: to_device(getattr(inp, n), device, dt) for n in names}
    out["logit_bias"] = to_device(inp.logit_bias, device, "f32")
    out["sel_bias"] = to_device(inp.sel_bias, device, "f32")
    return out


def _storage_dtype(dt):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


class MoELayer:
    """Holds device weights and a workspace; `forward` enqueues the whole layer."""

    def __init__(self, cfg_obj, dev: dict, device="cuda"):
        import torch
        self.cfg_obj = cfg_obj
        self.cfg = config_from(cfg_obj)
        self.dev = dev
        self.device = device
        self.ws = torch.empty(_lib.workspace_size(self.cfg), dtype=torch.uint8, device=device)
        N, E, k, d = cfg_obj.n_tokens, cfg_obj.n_experts, cfg_obj.top_k, cfg_obj.d_model
        i32, f32 = torch.int32, torch.float32
        self.out = {
            "out": torch.empty((N, d), dtype=_storage_dtype(cfg_obj.dtype), device=device),
            "logits": torch.empty((N, E), dtype=f32, device=device),
            "topk_idx": torch.empty((N, k), dtype=i32, device=device),
            "gates": torch.empty((N, k), dtype=f32, device=device),
            "counts": torch.empty(E, dtype=i32, device=device),
            "offsets": torch.empty(E + 1, dtype=i32, device=device),
            "perm": torch.empty(max(_lib.expert_rows(self.cfg), 1), dtype=i32, device=device),
            "slot_pos": torch.empty(N * k, dtype=i32, device=device),
            "drop_count": torch.empty(1, dtype=torch.int64, device=device),
            "probsum": torch.empty(E, dtype=f32, device=device),
            "aux": torch.empty(1, dtype=f32, device=device),
            "signs": torch.empty(E, dtype=torch.int8, device=device),
            "sel_bias_next": torch.empty(E, dtype=f32, device=device),
        }

    def forward(self, x=None, sel_bias="default", bias_gamma=None, outputs=None):
        x = self.dev["x"] if x is None else x
        sb = self.dev.get("sel_bias") if isinstance(sel_bias, str) else sel_bias
        gamma = self.cfg_obj.gamma if bias_gamma is None else bias_gamma
        outs = dict(self.out) if outputs is None else outputs
        if sb is None or gamma <= 0:
            outs = {k: v for k, v in outs.items() if k != "sel_bias_next"}
            gamma = 0.0
        if not self.cfg_obj.aux_loss and outputs is None:
            outs = {k: v for k, v in outs.items() if k != "aux"}
        _lib.forward(self.cfg, self.dev, x, outs["out"], residual=None, sel_bias=sb, outputs=outs,
                     bias_gamma=gamma, ws=self.ws)
        return outs
