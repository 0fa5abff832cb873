"""Single-GPU sparse Mixture-of-Experts FFN layer for AMD MI355X (gfx950).

Every step of the layer runs in hand-written HIP kernels of ``libmoe_hip.so``
behind the C ABI in ``include/moe.h``; this package only marshals arguments.
"""
from . import _lib
from ._lib import (MoeConfig, MoeError, make_config, workspace_size, route, permute, permute_noalloc, expert_ffn,
                   expert_up, expert_up_gather, expert_up_save, expert_down_combine, quantize_fp8, expert_up_fp8,
                   expert_down_fp8, backward, backward_workspace_size, expert_down, shared_ffn, combine,
                   bias_update, aux_loss, forward, status_str, lib, expert_rows, capacity, probe_hbm_read,
                   probe_mfma_bf16, probe_mfma_flop_per_iter)
from .layer import MoELayer, config_from, upload_inputs, to_device

__all__ = ["MoeConfig", "MoeError", "make_config", "workspace_size", "route", "permute", "permute_noalloc",
           "expert_ffn", "expert_up", "expert_up_gather", "expert_up_save", "expert_down_combine", "expert_down",
           "quantize_fp8", "expert_up_fp8", "expert_down_fp8", "backward", "backward_workspace_size", "shared_ffn",
           "combine", "bias_update", "aux_loss", "forward", "status_str", "lib", "expert_rows", "capacity",
           "probe_hbm_read", "probe_mfma_bf16", "probe_mfma_flop_per_iter",
           "MoELayer", "config_from", "upload_inputs", "to_device"]
