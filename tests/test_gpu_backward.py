"""GPU parity of the layer backward (moe_backward) against the fp64 oracle.

The forward runs through the step entry points (its routing decides both
sides); the oracle's backward runs on the GPU's logits.  Every gradient must
satisfy max|gpu - ref| / max|ref| <= 2e-2 (bf16 operands and intermediates,
fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
from gpu_harness import SMALL, TOL, host, rel_err, say
from workloads import make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "swiglu_rule_a": SMALL["mixtral_prefill_small"].scaled(name="bw_swiglu_rule_a", n_tokens=600),
    "rule_b_shared": SMALL["deepseek_v3_small"].scaled(name="bw_rule_b_shared", n_tokens=512),
    "gelu_bias_aux_capacity": SMALL["switch_skewed_small"].scaled(name="bw_gelu_bias_aux", n_tokens=1024),
    "padded_choice": SMALL["mixtral_prefill_small"].scaled(name="bw_padded_choice", n_tokens=500,
                                                           capacity_factor=1.25, capacity_layout="padded",
                                                           capacity_priority="choice"),
}


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_parity(name):
    import torch
    import mixture_experts_layer_histogram_amd as M
    cfg = CASES[name]
    say(f"backward {name}: N={cfg.n_tokens} d={cfg.d_model} E={cfg.n_experts} k={cfg.top_k} F={cfg.d_ff} "
        f"Fs={cfg.d_ff_shared} rule={cfg.gate_rule}")
    inp = make_inputs(cfg)
    dev = M.upload_inputs(inp, "cuda")
    c = M.config_from(cfg)
    N, E, k, d, F, Fs = cfg.n_tokens, cfg.n_experts, cfg.top_k, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    R = M._lib.expert_rows(c)
    st, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device="cuda")
    z = torch.empty((N, E), dtype=f32, device="cuda")
    idx = torch.empty((N, k), dtype=i32, device="cuda")
    g = torch.empty((N, k), dtype=f32, device="cuda")
    counts = torch.empty(E, dtype=i32, device="cuda")
    offs = torch.empty(E + 1, dtype=i32, device="cuda")
    perm = torch.empty(max(R, 1), dtype=i32, device="cuda")
    sp = torch.empty(N * k, dtype=i32, device="cuda")
    h = torch.empty((max(R, 1), F), dtype=st, device="cuda")
    y = torch.empty((max(R, 1), d), dtype=st, device="cuda")
    M.route(c, dev["x"], dev["w_router"], idx, g, logit_bias=dev["logit_bias"], sel_bias=dev["sel_bias"],
            logits=z, ws=ws)
    M.permute(c, idx, None, counts, offs, perm, sp, None, ws=ws)
    M.expert_up_gather(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h, b1=dev["b1"], ws=ws)
    M.expert_down(c, h, offs, dev["w2"], y, b2=dev["b2"], ws=ws)

    rng = np.random.default_rng(99)
    dout_np = rng.standard_normal((N, d)).astype(np.float32)
    dout = _bf16(dout_np)
    d_aux = 0.5 if cfg.aux_loss else 0.0
    grads = {"dx": torch.empty((N, d), dtype=st, device="cuda"),
             "dw_router": torch.empty((E, d), dtype=f32, device="cuda"),
             "dlogit_bias": torch.empty(E, dtype=f32, device="cuda"),
             "dw1": torch.empty((E, F, d), dtype=f32, device="cuda"),
             "dw2": torch.empty((E, d, F), dtype=f32, device="cuda"),
             "dgates": torch.empty((N, k), dtype=f32, device="cuda")}
    if cfg.act == "swiglu":
        grads["dw3"] = torch.empty((E, F, d), dtype=f32, device="cuda")
    if cfg.ffn_bias:
        grads["db1"] = torch.empty((E, F), dtype=f32, device="cuda")
        grads["db2"] = torch.empty((E, d), dtype=f32, device="cuda")
    if Fs:
        grads["dsh_w1"] = torch.empty((Fs, d), dtype=f32, device="cuda")
        grads["dsh_w3"] = torch.empty((Fs, d), dtype=f32, device="cuda")
        grads["dsh_w2"] = torch.empty((d, Fs), dtype=f32, device="cuda")
    bws = torch.empty(M.backward_workspace_size(c), dtype=torch.uint8, device="cuda")
    saved = {"logits": z, "topk_idx": idx, "gates": g, "counts": counts, "offsets": offs, "perm": perm,
             "slot_pos": sp, "y_perm": y}
    M.backward(c, dev, dev["x"], dout, saved, grads, d_aux=d_aux, ws=bws)
    torch.cuda.synchronize()

    dout_ref = host(dout)
    ref = oracle.oracle_layer_backward(cfg, inp, dout_ref, d_aux=d_aux, logits_override=host(z))
    tol = TOL["bf16"]
    checks = [("dx", "x"), ("dw_router", "w_router"), ("dlogit_bias", "logit_bias"), ("dw1", "w1"), ("dw2", "w2"),
              ("dgates", "gates")]
    checks += [("dw3", "w3")] if cfg.act == "swiglu" else []
    checks += [("db1", "b1"), ("db2", "b2")] if cfg.ffn_bias else []
    checks += [("dsh_w1", "sh_w1"), ("dsh_w3", "sh_w3"), ("dsh_w2", "sh_w2")] if Fs else []
    for gk, rk in checks:
        err = rel_err(host(grads[gk]), ref[rk])
        say(f"  {gk}: rel err {err:.3e}")
        assert err <= tol, (name, gk, err)
    # deterministic: a second call gives the same bits
    dx1 = host(grads["dx"]).copy()
    w1a = host(grads["dw1"]).copy()
    M.backward(c, dev, dev["x"], dout, saved, grads, d_aux=d_aux, ws=bws)
    torch.cuda.synchronize()
    assert np.array_equal(host(grads["dx"]), dx1) and np.array_equal(host(grads["dw1"]), w1a)
