"""moe_permute_noalloc (the dispatch on the library's static per-GPU scratch)
against moe_permute (the same kernels on a caller's workspace): bit-identical
counts, offsets, permutation, slot positions, drop count and gathered rows, on
two calls in a row, the second with a smaller batch (the scratch keeps the
first call's contents, which must not leak into the second)."""
import numpy as np
import pytest

from gpu_harness import SMALL, host, say
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _dispatch_both(cfg):
    import torch
    import mixture_experts_layer_histogram_amd as M
    inp = make_inputs(cfg)
    dev = M.upload_inputs(inp, "cuda")
    c = M.config_from(cfg)
    N, E, k, d = cfg.n_tokens, cfg.n_experts, cfg.top_k, cfg.d_model
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device="cuda")
    z = torch.empty((N, E), dtype=torch.float32, device="cuda")
    idx = torch.empty((N, k), dtype=torch.int32, device="cuda")
    g = torch.empty((N, k), dtype=torch.float32, device="cuda")
    M.route(c, dev["x"], dev["w_router"], idx, g, logit_bias=dev["logit_bias"], sel_bias=dev["sel_bias"], logits=z,
            ws=ws)
    R = max(M.expert_rows(c), 1)
    outs = []
    for noalloc in (False, True):
        o = {"counts": torch.full((E,), -7, dtype=torch.int32, device="cuda"),
             "offsets": torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
             "perm": torch.full((R,), -7, dtype=torch.int32, device="cuda"),
             "slot_pos": torch.full((N * k,), -7, dtype=torch.int32, device="cuda"),
             "drop": torch.full((1,), -7, dtype=torch.int64, device="cuda"),
             "x_perm": torch.zeros((R, d), dtype=torch.bfloat16, device="cuda")}
        args = (c, idx, dev["x"], o["counts"], o["offsets"], o["perm"], o["slot_pos"])
        if noalloc:
            M.permute_noalloc(*args, x_perm=o["x_perm"], drop_count=o["drop"])
        else:
            M.permute(*args, x_perm=o["x_perm"], drop_count=o["drop"], ws=ws)
        torch.cuda.synchronize()
        outs.append({n: host(t) for n, t in o.items()})
    return outs


def test_noalloc_dispatch_matches_workspace_dispatch():
    big = SMALL["deepseek_v3_small"].scaled(name="noalloc_big", n_tokens=4096, n_experts=64, top_k=8,
                                            capacity_factor=1.5)
    small = SMALL["switch_skewed_small"].scaled(name="noalloc_small", n_tokens=300)
    for cfg in (big, small):
        say(f"noalloc dispatch: {cfg.name} N={cfg.n_tokens} E={cfg.n_experts} k={cfg.top_k}")
        ref, got = _dispatch_both(cfg)
        kept = int(ref["offsets"][-1])
        assert kept > 0 and int(ref["drop"][0]) > 0
        for n in ("counts", "offsets", "slot_pos", "drop"):
            assert np.array_equal(got[n], ref[n]), (cfg.name, n)
        assert np.array_equal(got["perm"][:kept], ref["perm"][:kept]), cfg.name
        assert np.array_equal(got["x_perm"][:kept], ref["x_perm"][:kept]), cfg.name
