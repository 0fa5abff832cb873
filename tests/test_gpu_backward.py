"""GPU parity of the layer backward (moe_backward) against the fp64 oracle.

The forward runs through the step entry points (its routing decides both
sides); the oracle's backward runs on the GPU's logits.  Every gradient must
satisfy max|gpu - ref| / max|ref| <= 2e-2 (bf16 operands and intermediates,
fp32 accumulation).
"""
import numpy as np
import pytest

import oracle
from gpu_harness import FULL, SMALL, TOL, host, rel_err, say
from workloads import make_inputs

pytestmark = pytest.mark.gpu

CASES = {
    "swiglu_rule_a": SMALL["mixtral_prefill_small"].scaled(name="bw_swiglu_rule_a", n_tokens=600),
    "rule_b_shared": SMALL["deepseek_v3_small"].scaled(name="bw_rule_b_shared", n_tokens=512),
    "gelu_bias_aux_capacity": SMALL["switch_skewed_small"].scaled(name="bw_gelu_bias_aux", n_tokens=1024),
    "padded_choice": SMALL["mixtral_prefill_small"].scaled(name="bw_padded_choice", n_tokens=500,
                                                           capacity_factor=1.25, capacity_layout="padded",
                                                           capacity_priority="choice"),
    # E not a multiple of 64 (padded router width), k = 3, a ragged token count
    "e100_k3": SMALL["mixtral_prefill_small"].scaled(name="bw_e100_k3", n_tokens=333, n_experts=100, top_k=3),
    "one_token": SMALL["deepseek_v3_small"].scaled(name="bw_one_token", n_tokens=1),
    # one hot expert (~1350 rows: 256x256 weight-gradient tiles over a long K), the others with a
    # handful of rows or none (128x128 tiles, zero gradients); d and F not multiples of 128
    "skewed_long_short": SMALL["switch_skewed_small"].scaled(name="bw_skewed_long_short", n_tokens=1500,
                                                             d_model=320, d_ff=448, capacity_factor=0.0),
}


def _bf16(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).astype(np.float32)).to(torch.bfloat16).cuda()


def _run_backward(cfg, inp, dout, d_aux, save_pre=False):
    """Forward through the step entry points, then moe_backward; returns the
    device gradients, the device logits and a callable that repeats the backward.
    save_pre: the up-projection is moe_expert_up_save and the backward reuses its
    pre-activations instead of recomputing them."""
    import torch
    import mixture_experts_layer_histogram_amd as M
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
    pre = None
    if save_pre:
        n_mat = 2 if cfg.act == "swiglu" else 1
        pre = torch.empty((n_mat, max(R, 1), F), dtype=st, device="cuda")
        M.expert_up_save(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h, pre, b1=dev["b1"], ws=ws)
        h_ref = torch.empty_like(h)
        M.expert_up_gather(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h_ref, b1=dev["b1"], ws=ws)
        torch.cuda.synchronize()
        kept = int(offs[-1].item())
        assert torch.equal(h[:kept], h_ref[:kept])      # saving changes nothing else
        del h_ref
    else:
        M.expert_up_gather(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h, b1=dev["b1"], ws=ws)
    M.expert_down(c, h, offs, dev["w2"], y, b2=dev["b2"], ws=ws)
    del h, ws
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
             "slot_pos": sp, "y_perm": y, "pre_act": pre}

    def again():
        M.backward(c, dev, dev["x"], dout, saved, grads, d_aux=d_aux, ws=bws)
        torch.cuda.synchronize()
    again()
    return grads, z, sp, again


SAVED = ["swiglu_rule_a", "gelu_bias_aux_capacity", "padded_choice"]


@pytest.mark.parametrize("name,save_pre", [(n, False) for n in sorted(CASES)] + [(n, True) for n in SAVED],
                         ids=[n for n in sorted(CASES)] + [n + "-saved_pre" for n in SAVED])
def test_backward_parity(name, save_pre):
    cfg = CASES[name]
    say(f"backward {name}: N={cfg.n_tokens} d={cfg.d_model} E={cfg.n_experts} k={cfg.top_k} F={cfg.d_ff} "
        f"Fs={cfg.d_ff_shared} rule={cfg.gate_rule} saved pre-activations={save_pre}")
    inp = make_inputs(cfg)
    rng = np.random.default_rng(99)
    dout = _bf16(rng.standard_normal((cfg.n_tokens, cfg.d_model)).astype(np.float32))
    d_aux = 0.5 if cfg.aux_loss else 0.0
    grads, z, _, again = _run_backward(cfg, inp, dout, d_aux, save_pre)

    ref = oracle.oracle_layer_backward(cfg, inp, host(dout), d_aux=d_aux, logits_override=host(z))
    tol = TOL["bf16"]
    checks = [("dx", "x"), ("dw_router", "w_router"), ("dlogit_bias", "logit_bias"), ("dw1", "w1"), ("dw2", "w2"),
              ("dgates", "gates")]
    checks += [("dw3", "w3")] if cfg.act == "swiglu" else []
    checks += [("db1", "b1"), ("db2", "b2")] if cfg.ffn_bias else []
    checks += [("dsh_w1", "sh_w1"), ("dsh_w3", "sh_w3"), ("dsh_w2", "sh_w2")] if cfg.d_ff_shared else []
    for gk, rk in checks:
        err = rel_err(host(grads[gk]), ref[rk])
        say(f"  {gk}: rel err {err:.3e}")
        assert err <= tol, (name, gk, err)
    # deterministic: a second call gives the same bits
    dx1 = host(grads["dx"]).copy()
    w1a = host(grads["dw1"]).copy()
    again()
    assert np.array_equal(host(grads["dx"]), dx1) and np.array_equal(host(grads["dw1"]), w1a)


def _sample_rows(cfg, slot_pos, n=12):
    N = cfg.n_tokens
    rows = set(np.linspace(0, N - 1, min(n, N)).astype(int).tolist())
    dropped = np.nonzero((slot_pos.reshape(N, cfg.top_k) < 0).any(axis=1))[0]
    rows.update(dropped[:4].tolist())                       # tokens with a dropped slot
    return np.array(sorted(rows))


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_prefill", "mixtral_decode", "switch_skewed", "deepseek_v3"])
def test_backward_full_size(name):
    """Full sizes: dx and dgates on sampled tokens, the weight gradients of
    sampled hidden units of the busiest, the least busy and the first expert
    (and of the shared expert), each computed by the oracle one by one.  The
    router gradients element by element from the oracle's logit gradients of
    every token (and dx of every token) at the Mixtral and Switch shapes; at
    every shape also through a property of each softmax-based gate rule (a
    token's logit gradient sums to zero over the experts, so the expert sums
    of dlogit_bias and of dw_router vanish)."""
    import torch
    cfg = FULL[name]
    say(f"backward full {name}: generating inputs")
    inp = make_inputs(cfg)
    N, E, d, F, Fs = cfg.n_tokens, cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    gen = torch.Generator(device="cuda").manual_seed(98)
    dout = (torch.randn((N, d), device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    d_aux = 0.5 if cfg.aux_loss else 0.0
    say(f"backward full {name}: forward + backward")
    grads, z, sp, _ = _run_backward(cfg, inp, dout, d_aux)
    dout_h, sp_h = host(dout), host(sp)
    tol = TOL["bf16"]

    rows = _sample_rows(cfg, sp_h)
    say(f"backward full {name}: oracle on {rows.size} sampled tokens")
    rb = oracle.oracle_backward_rows(cfg, inp, dout_h, rows, d_aux=d_aux, logits_override=host(z))
    rows_t = torch.from_numpy(rows).cuda()
    for gk, ref in (("dx", rb["x"]), ("dgates", rb["gates"])):
        err = rel_err(host(grads[gk].index_select(0, rows_t)), ref)
        say(f"  {gk} rows: rel err {err:.3e}")
        assert err <= tol, (name, gk, err)

    kept = rb["route"].disp.offsets[1:] - rb["route"].disp.offsets[:-1]
    busy = [int(np.argmax(kept)), int(np.argmin(np.where(kept > 0, kept, kept.max() + 1))), 0]
    cols = np.array(sorted({0, F // 3, F - 1}))
    cols_t = torch.from_numpy(cols).cuda()
    for e in dict.fromkeys(busy):
        if kept[e] == 0:
            continue
        gc = oracle.oracle_expert_grad_columns(cfg, inp, dout_h, e, cols, rb["route"])
        got = {"w1": grads["dw1"][e].index_select(0, cols_t), "w2": grads["dw2"][e].index_select(1, cols_t)}
        if cfg.act == "swiglu":
            got["w3"] = grads["dw3"][e].index_select(0, cols_t)
        if cfg.ffn_bias:
            got["b1"] = grads["db1"][e].index_select(0, cols_t)
            got["b2"] = grads["db2"][e]
        for n, t in got.items():
            err = rel_err(host(t), gc[n])
            say(f"  expert {e} ({kept[e]} rows) d{n} cols: rel err {err:.3e}")
            assert err <= tol, (name, e, n, err)
    if Fs:
        sc = np.array([0, Fs // 2, Fs - 1])
        sc_t = torch.from_numpy(sc).cuda()
        gs = oracle.oracle_shared_grad_columns(cfg, inp, dout_h, sc)
        for n, t in (("w1", grads["dsh_w1"].index_select(0, sc_t)), ("w3", grads["dsh_w3"].index_select(0, sc_t)),
                     ("w2", grads["dsh_w2"].index_select(1, sc_t))):
            err = rel_err(host(t), gs[n])
            say(f"  shared dsh_{n} cols: rel err {err:.3e}")
            assert err <= tol, (name, "sh", n, err)

    if name in ("mixtral_prefill", "mixtral_decode", "switch_skewed"):
        # router gradients element by element: the oracle's dL/dlogits of every token, then
        # dW_r = dz^T x and dlogit_bias = sum_t dz
        say(f"backward full {name}: oracle dlogits of all {N} tokens")
        ra = oracle.oracle_backward_rows(cfg, inp, dout_h, np.arange(N), d_aux=d_aux, logits_override=host(z))
        dz = ra["logits"]
        x64 = oracle.to_f64(inp.x, cfg.dtype)
        for gk, ref in (("dw_router", dz.T @ x64), ("dlogit_bias", dz.sum(axis=0))):
            err = rel_err(host(grads[gk]), ref)
            say(f"  {gk}: rel err {err:.3e} (every element)")
            assert err <= tol, (name, gk, err)
        err = rel_err(host(grads["dx"]), ra["x"])
        say(f"  dx: rel err {err:.3e} (every token)")
        assert err <= tol, (name, "dx all", err)

    # router: sum over experts of each token's dlogits is zero
    db = host(grads["dlogit_bias"])
    dwr = grads["dw_router"]
    s_db = abs(float(db.sum())) / max(float(np.abs(db).max()), 1e-30)
    s_wr = float(dwr.double().sum(0).abs().max()) / max(float(dwr.abs().max()), 1e-30)
    say(f"  router: |sum_e dlogit_bias| {s_db:.3e}, |sum_e dw_router| {s_wr:.3e} (relative)")
    assert s_db <= 1e-3 and s_wr <= tol


def test_backward_empty_batch():
    """N = 0: no launches on token buffers; every weight gradient comes back zero."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    cfg = SMALL["deepseek_v3_small"].scaled(name="bw_empty", n_tokens=0)
    inp = make_inputs(cfg)
    dev = M.upload_inputs(inp, "cuda")
    c = M.config_from(cfg)
    E, d, F, Fs = cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    nan = float("nan")
    grads = {"dw_router": torch.full((E, d), nan, device="cuda"), "dlogit_bias": torch.full((E,), nan, device="cuda"),
             "dw1": torch.full((E, F, d), nan, device="cuda"), "dw3": torch.full((E, F, d), nan, device="cuda"),
             "dw2": torch.full((E, d, F), nan, device="cuda"), "dsh_w1": torch.full((Fs, d), nan, device="cuda"),
             "dsh_w3": torch.full((Fs, d), nan, device="cuda"), "dsh_w2": torch.full((d, Fs), nan, device="cuda")}
    bws = torch.empty(max(M.backward_workspace_size(c), 1), dtype=torch.uint8, device="cuda")
    M.backward(c, dev, None, None, {}, grads, d_aux=0.0, ws=bws)
    torch.cuda.synchronize()
    for n, t in grads.items():
        assert torch.count_nonzero(t).item() == 0, n
