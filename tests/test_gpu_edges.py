"""GPU edge cases: empty and one-token batches, a single expert, k = E, k
above the top-k lane group, a capacity that drops every slot, exact logit
ties, odd expert counts, K-split tails, the GEMM router's short tail."""
import numpy as np
import pytest

import oracle
from gpu_harness import SMALL, TOL, host, rel_err, run_layer, say
from workloads import MIXTRAL_PREFILL, DEEPSEEK_V3, SWITCH_SKEWED, TINY_TOP2_FP32

pytestmark = pytest.mark.gpu

BASE = SMALL["mixtral_prefill_small"]

EDGE = {
    "one_token": BASE.scaled(name="one_token", n_tokens=1),
    "single_expert": BASE.scaled(name="single_expert", n_tokens=333, n_experts=1, top_k=1),
    "k_equals_e": BASE.scaled(name="k_equals_e", n_tokens=200, n_experts=4, top_k=4),
    "odd_experts": BASE.scaled(name="odd_experts", n_tokens=517, n_experts=100, top_k=3, d_model=128, d_ff=192),
    "all_dropped": SWITCH_SKEWED.scaled(name="all_dropped", n_tokens=300, d_model=128, d_ff=128,
                                        capacity_factor=0.01),
    "topk_bias_rule_a": BASE.scaled(name="topk_bias_rule_a", n_tokens=400, sel_bias_range=0.3),
    "f32_swiglu_shared": DEEPSEEK_V3.scaled(name="f32_swiglu_shared", n_tokens=77, d_model=48, d_ff=40,
                                            d_ff_shared=24, n_experts=16, top_k=4, dtype="f32"),
    "f32_switch_capacity": SWITCH_SKEWED.scaled(name="f32_switch_capacity", n_tokens=129, d_model=36, d_ff=20,
                                                n_experts=8, dtype="f32", init="normal"),
    "decode_e256": DEEPSEEK_V3.scaled(name="decode_e256", n_tokens=3, d_model=256, d_ff=64, d_ff_shared=64),
    # large segments: the 256-row GEMM tiles with the GELU + bias epilogues and a ragged tail
    "gelu_big_segments": SWITCH_SKEWED.scaled(name="gelu_big_segments", n_tokens=2100, n_experts=8, d_model=320,
                                              d_ff=576, capacity_factor=0.0, logit_offset=None, aux_loss=True),
    "swiglu_big_segments": BASE.scaled(name="swiglu_big_segments", n_tokens=1500, n_experts=4, d_model=192,
                                       d_ff=320),
    # more tiles than one round of workgroups with a partial last round: the K-split tail path
    # k larger than the top-k lane group (8 lanes per token for E <= 64)
    "k16_e32": BASE.scaled(name="k16_e32", n_tokens=300, n_experts=32, top_k=16),
    # E = 64 router on the grouped GEMM with a logit bias and a short tail (64-row tiles)
    "router_gemm_tail": SWITCH_SKEWED.scaled(name="router_gemm_tail", n_tokens=600, d_model=256, d_ff=256),
    # capacity-buffer layout ([E, C] rows, padding rows read as zero) and choice-major priority
    "padded_capacity": BASE.scaled(name="padded_capacity", n_tokens=600, capacity_factor=1.25,
                                   capacity_layout="padded"),
    "choice_priority": BASE.scaled(name="choice_priority", n_tokens=600, capacity_factor=1.25,
                                   capacity_priority="choice"),
    "padded_choice_f32": DEEPSEEK_V3.scaled(name="padded_choice_f32", n_tokens=77, d_model=48, d_ff=40,
                                            d_ff_shared=24, n_experts=16, top_k=4, dtype="f32",
                                            capacity_factor=1.5, capacity_layout="padded",
                                            capacity_priority="choice"),
    "padded_gelu_bias": SWITCH_SKEWED.scaled(name="padded_gelu_bias", n_tokens=700, d_model=192, d_ff=320,
                                             capacity_layout="padded"),
    "split_k_up": BASE.scaled(name="split_k_up", n_tokens=2048, n_experts=4, d_model=256, d_ff=2240),
    "split_k_down_gelu": SWITCH_SKEWED.scaled(name="split_k_down_gelu", n_tokens=2048, n_experts=4, d_model=8448,
                                              d_ff=256, capacity_factor=0.0, logit_offset=None),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_parity(name):
    cfg = EDGE[name]
    say(f"edge {name}: N={cfg.n_tokens} E={cfg.n_experts} k={cfg.top_k} dtype={cfg.dtype}")
    inp, o, _ = run_layer(cfg)
    r = oracle.oracle_route(cfg, o["logits"], inp.sel_bias)
    assert np.array_equal(o["topk_idx"], r.topk_idx)
    assert np.array_equal(o["counts"], r.disp.counts)
    assert np.array_equal(o["offsets"], r.disp.offsets)
    assert np.array_equal(o["slot_pos"], r.disp.slot_pos)
    assert int(o["drop_count"][0]) == r.disp.drop_count
    _, ref = oracle.oracle_layer(cfg, inp, logits_override=o["logits"])
    assert rel_err(o["out"], ref) <= TOL[cfg.dtype], rel_err(o["out"], ref)
    if cfg.capacity_layout == "padded":      # padding rows carry -1 in perm
        assert np.array_equal(o["perm"], r.disp.perm)
    else:
        kept = int(r.disp.offsets[-1])
        assert np.array_equal(o["perm"][:kept], r.disp.perm)
    if name == "all_dropped":
        assert r.disp.drop_count == cfg.n_tokens
        assert np.array_equal(o["out"], host_x(inp))      # residual passes through unchanged


def host_x(inp):
    return oracle.to_f64(inp.x, inp.cfg.dtype)


def test_empty_batch():
    import torch
    cfg = BASE.scaled(name="empty", n_tokens=0, aux_loss=True)
    inp, o, _ = run_layer(cfg)
    assert o["out"].shape == (0, cfg.d_model)
    assert np.all(o["counts"] == 0) and np.all(o["offsets"] == 0)
    assert int(o["drop_count"][0]) == 0
    assert float(o["aux"][0]) == 0.0


@pytest.mark.parametrize("rule", ["topk_softmax", "softmax_renorm", "switch_top1"])
def test_exact_ties_go_to_lower_index(rule):
    """Router logits with many exact ties (passed through logits_in): the chosen
    experts match the oracle's stable ranking bit for bit."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    for E, k in ((8, 2), (64, 1), (256, 8), (100, 3)):
        if rule == "switch_top1":
            k = 1
        N = 300
        cfg = DEEPSEEK_V3.scaled(name="ties", n_tokens=N, n_experts=E, top_k=k, gate_rule=rule, d_model=64,
                                 d_ff=64, d_ff_shared=0, sel_bias_range=0.0, gamma=0.0)
        rng = np.random.default_rng(E * 7 + k)
        z = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(N, E)).astype(np.float32)
        sb = rng.choice(np.array([0.0, 0.0, 0.25], np.float32), size=E).astype(np.float32)
        if rule == "switch_top1":
            sb = None
        c = M.config_from(cfg)
        zt = torch.from_numpy(z).cuda()
        sbt = torch.from_numpy(sb).cuda() if sb is not None else None
        idx = torch.empty((N, k), dtype=torch.int32, device="cuda")
        g = torch.empty((N, k), dtype=torch.float32, device="cuda")
        zo = torch.empty_like(zt)
        M.route(c, None, None, idx, g, sel_bias=sbt, logits_in=zt, logits=zo)
        torch.cuda.synchronize()
        r = oracle.oracle_route(cfg, z, sb)
        assert np.array_equal(host(idx), r.topk_idx), (rule, E, k)
        assert rel_err(host(g), r.gates) <= 1e-6
        assert np.array_equal(host(zo), z)
