"""GPU parity: the HIP layer (through the C ABI) against the fp64 oracle.

Integer outputs (selected experts, counts, offsets, permutation, slot
positions / drop mask, drop count, bias signs) must be bit-exact given the
GPU's fp32 router logits; floating-point outputs must be within
max|gpu - ref| / max|ref| <= 2e-2 (bf16 storage) or 1e-5 (fp32 storage).
"""
import numpy as np
import pytest

import oracle
from gpu_harness import SMALL, TOL, host, rel_err, run_layer, say
from workloads import make_inputs

pytestmark = pytest.mark.gpu


def _check_route(cfg, inp, o):
    """Routing, dispatch, aux and bias step against the oracle run on the GPU logits."""
    tol = TOL[cfg.dtype]
    dt = cfg.dtype
    z_ref = oracle.router_logits(oracle.to_f64(inp.x, dt), oracle.to_f64(inp.w_router, dt), inp.logit_bias)
    assert rel_err(o["logits"], z_ref) <= tol, rel_err(o["logits"], z_ref)
    r = oracle.oracle_route(cfg, o["logits"], inp.sel_bias)
    say(f"{cfg.name}: min selection gap {r.min_gap:.3e}")
    assert np.array_equal(o["topk_idx"], r.topk_idx), "topk_idx differs"
    assert rel_err(o["gates"], r.gates) <= tol
    assert np.array_equal(o["counts"], r.disp.counts), (o["counts"], r.disp.counts)
    assert np.array_equal(o["offsets"], r.disp.offsets)
    kept = int(r.disp.offsets[-1])
    assert np.array_equal(o["perm"][:kept], r.disp.perm)
    assert np.array_equal(o["slot_pos"], r.disp.slot_pos)
    assert int(o["drop_count"][0]) == r.disp.drop_count
    if cfg.aux_loss:
        assert abs(float(o["aux"][0]) - r.aux) <= tol * abs(r.aux), (o["aux"], r.aux)
        assert rel_err(o["probsum"], r.probs.sum(axis=0)) <= tol
    if cfg.gamma > 0:
        assert np.array_equal(o["signs"].astype(np.int64), r.signs)
        assert rel_err(o["sel_bias_next"], r.new_bias) <= 1e-6
    return r


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_parity_small(name):
    cfg = SMALL[name]
    say(f"case {name}: N={cfg.n_tokens} d={cfg.d_model} E={cfg.n_experts} k={cfg.top_k} F={cfg.d_ff}")
    inp, o, _ = run_layer(cfg)
    _check_route(cfg, inp, o)
    _, ref = oracle.oracle_layer(cfg, inp, logits_override=o["logits"])
    err = rel_err(o["out"], ref)
    say(f"{name}: out rel err {err:.3e}")
    assert err <= TOL[cfg.dtype], err


@pytest.mark.parametrize("name", sorted(SMALL))
def test_layer_deterministic(name):
    """Two runs, and a run with the workspace at another address, give identical bits."""
    import torch
    cfg = SMALL[name]
    inp, o1, layer = run_layer(cfg, runs=2)
    layer.ws = torch.empty(layer.ws.numel() + 4096, dtype=torch.uint8, device="cuda")[4096:]
    o2 = {k: host(v) for k, v in layer.forward().items()}
    torch.cuda.synchronize()
    for k in o1:
        assert np.array_equal(o1[k], o2[k]), k


def test_steps_match_forward():
    """moe_route -> moe_permute -> moe_expert_ffn / moe_shared_ffn -> moe_combine ->
    moe_aux_loss / moe_bias_update give the bits moe_forward gives."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    for name in ("deepseek_v3_small", "switch_skewed_small", "mixtral_prefill_small"):
        cfg = SMALL[name]
        inp, o, layer = run_layer(cfg)
        dev, c, ws = layer.dev, layer.cfg, layer.ws
        N, E, k, d, F = cfg.n_tokens, cfg.n_experts, cfg.top_k, cfg.d_model, cfg.d_ff
        st = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        z = torch.empty((N, E), dtype=torch.float32, device="cuda")
        idx = torch.empty((N, k), dtype=torch.int32, device="cuda")
        g = torch.empty((N, k), dtype=torch.float32, device="cuda")
        ps = torch.empty(E, dtype=torch.float32, device="cuda")
        M.route(c, dev["x"], dev["w_router"], idx, g, logit_bias=dev["logit_bias"], sel_bias=dev["sel_bias"],
                logits=z, probsum=ps, ws=ws)
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(N * k, dtype=torch.int32, device="cuda")
        sp = torch.empty(N * k, dtype=torch.int32, device="cuda")
        drop = torch.empty(1, dtype=torch.int64, device="cuda")
        xp = torch.empty((N * k, d), dtype=st, device="cuda")
        M.permute(c, idx, dev["x"], counts, offs, perm, sp, xp, drop_count=drop, ws=ws)
        h = torch.empty((N * k, F), dtype=st, device="cuda")
        y = torch.empty((N * k, d), dtype=st, device="cuda")
        M.expert_ffn(c, xp, offs, dev["w1"], dev["w3"], dev["w2"], h, y, b1=dev["b1"], b2=dev["b2"], ws=ws)
        ysh = None
        if cfg.d_ff_shared:
            hsh = torch.empty((N, cfg.d_ff_shared), dtype=st, device="cuda")
            ysh = torch.empty((N, d), dtype=st, device="cuda")
            M.shared_ffn(c, dev["x"], dev["sh_w1"], dev["sh_w3"], dev["sh_w2"], hsh, ysh, ws=ws)
        out = torch.empty((N, d), dtype=st, device="cuda")
        M.combine(c, y, sp, g, out, residual=dev["x"] if cfg.residual else None, shared_y=ysh)
        torch.cuda.synchronize()
        kept = int(host(offs)[-1])
        # x_perm rows are exact copies of the token rows
        xp_h, x_h, perm_h = host(xp)[:kept], host(dev["x"]), host(perm)[:kept]
        assert np.array_equal(xp_h, x_h[perm_h // k])
        for key, t in (("logits", z), ("topk_idx", idx), ("gates", g), ("counts", counts), ("offsets", offs),
                       ("slot_pos", sp), ("drop_count", drop), ("out", out)):
            assert np.array_equal(host(t), o[key]), (name, key)
        assert np.array_equal(host(perm)[:kept], o["perm"][:kept])
        # the fused dispatch: indices only, then the up GEMM gathers token rows through perm
        perm2 = torch.full_like(perm, -7)
        sp2 = torch.empty_like(sp)
        counts2 = torch.empty_like(counts)
        offs2 = torch.empty_like(offs)
        M.permute(c, idx, None, counts2, offs2, perm2, sp2, None, ws=ws)
        h2 = torch.empty_like(h)
        M.expert_up_gather(c, dev["x"], perm2, offs2, dev["w1"], dev["w3"], h2, b1=dev["b1"], ws=ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(counts2), host(counts)) and np.array_equal(host(offs2), host(offs))
        assert np.array_equal(host(perm2)[:kept], perm_h) and np.array_equal(host(sp2), host(sp))
        assert np.array_equal(host(h2)[:kept], host(h)[:kept]), (name, "gathered up-projection differs")
        if cfg.aux_loss:
            aux = torch.empty(1, dtype=torch.float32, device="cuda")
            M.aux_loss(c, counts, ps, aux)
            torch.cuda.synchronize()
            assert host(aux)[0] == o["aux"][0]
        if cfg.gamma > 0:
            b = dev["sel_bias"].clone()
            signs = torch.empty(E, dtype=torch.int8, device="cuda")
            M.bias_update(c, counts, cfg.gamma, b, signs)
            torch.cuda.synchronize()
            assert np.array_equal(host(signs), o["signs"])
            assert np.array_equal(host(b), o["sel_bias_next"])


def test_expert_ffn_parity_per_segment():
    """y_perm rows against the oracle's expert FFN on the same gathered rows."""
    for name in ("mixtral_prefill_small", "switch_skewed_small", "deepseek_v3_small"):
        cfg = SMALL[name]
        inp, o, layer = run_layer(cfg)
        import torch
        import mixture_experts_layer_histogram_amd as M
        N, k, d, F = cfg.n_tokens, cfg.top_k, cfg.d_model, cfg.d_ff
        st = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        dev = layer.dev
        offs = torch.from_numpy(o["offsets"]).cuda()
        perm = o["perm"]
        kept = int(o["offsets"][-1])
        xp = dev["x"][torch.from_numpy(perm[:kept] // k).long().cuda()].contiguous()
        xpad = torch.zeros((N * k, d), dtype=st, device="cuda")
        xpad[:kept] = xp
        h = torch.empty((N * k, F), dtype=st, device="cuda")
        yp = torch.empty((N * k, d), dtype=st, device="cuda")
        M.expert_ffn(layer.cfg, xpad, offs, dev["w1"], dev["w3"], dev["w2"], h, yp, b1=dev["b1"], b2=dev["b2"],
                     ws=layer.ws)
        torch.cuda.synchronize()
        with np.errstate(invalid="raise"):                 # a NaN in the written rows fails here
            yp_h = host(yp[:kept])                         # rows past `kept` are never written
        x64 = oracle.to_f64(inp.x, cfg.dtype)
        for e in range(cfg.n_experts):
            lo, hi = int(o["offsets"][e]), int(o["offsets"][e + 1])
            if hi == lo:
                continue
            w = {n: oracle.to_f64(v, cfg.dtype) for n, v in inp.expert(e).items()}
            ref = oracle.expert_apply(cfg.act, x64[perm[lo:hi] // k], w)
            err = rel_err(yp_h[lo:hi], ref)
            assert err <= TOL[cfg.dtype], (name, e, err)


# Segment sizes that make the forward kernels attach short tails to whole 256-row tiles
# (tails of 1, 14, 31, 32, 33, 44, 84 and 127 rows on one whole tile; of 1, 38, 64, 88
# and 127 rows on two; 384 rows with a tail of exactly 128 as a whole tile; empty and
# tile-less segments); the last 80 of the 336 whole-tile units, among them the 639-row
# segment's attached rows, run as K-parts with a fix-up.  The host-model test
# test_attach_edge_sizes_select_attaching_tiles shows the kernels' tail rule picks the
# attaching kind for these sizes.
ATTACH_EDGE_ROWS = [257, 270, 287, 288, 289, 300, 340, 383, 513, 550, 576, 600, 639, 384, 0, 1, 64, 127, 128]


@pytest.mark.parametrize("act", ["swiglu", "gelu_bias"])
def test_attached_tail_segments(act):
    """Every row of y_perm against the oracle's expert FFN for segments whose short tails
    ride on whole 256-row tiles, in the up projection (SwiGLU, or GELU + bias) and the down
    projection; the gathered up projection writes the same bits as the one on pre-gathered
    rows."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    from workloads import MIXTRAL_PREFILL, SWITCH_SKEWED
    rows = ATTACH_EDGE_ROWS
    R, E = sum(rows), len(rows)
    if act == "swiglu":
        cfg = MIXTRAL_PREFILL.scaled(name="attach_swiglu", n_tokens=R, n_experts=E, top_k=1, d_ff=2048)
    else:
        cfg = SWITCH_SKEWED.scaled(name="attach_gelu", n_tokens=R, n_experts=E, top_k=1, d_model=4096, d_ff=4096,
                                   capacity_factor=0.0, logit_offset=None)
    say(f"attached tails {act}: R={R} E={E} d={cfg.d_model} F={cfg.d_ff}")
    inp = make_inputs(cfg)
    dev = M.upload_inputs(inp, "cuda")
    c = M.config_from(cfg)
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device="cuda")
    offs_h = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    perm_h = np.random.default_rng(7).permutation(R).astype(np.int32)   # the expert order's token rows
    offs = torch.from_numpy(offs_h).cuda()
    perm = torch.from_numpy(perm_h).cuda()
    xp = dev["x"][perm.long()].contiguous()
    h = torch.empty((R, cfg.d_ff), dtype=torch.bfloat16, device="cuda")
    h2 = torch.empty_like(h)
    y = torch.full((R, cfg.d_model), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.expert_ffn(c, xp, offs, dev["w1"], dev["w3"], dev["w2"], h, y, b1=dev["b1"], b2=dev["b2"], ws=ws)
    M.expert_up_gather(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h2, b1=dev["b1"], ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16)), "gathered up projection differs"
    yh = host(y)
    assert np.isfinite(yh).all(), "rows left unwritten"
    x64 = oracle.to_f64(inp.x, cfg.dtype)
    for e in range(E):
        lo, hi = int(offs_h[e]), int(offs_h[e + 1])
        if hi == lo:
            continue
        w = {n: oracle.to_f64(v, cfg.dtype) for n, v in inp.expert(e).items()}
        ref = oracle.expert_apply(cfg.act, x64[perm_h[lo:hi]], w)
        err = rel_err(yh[lo:hi], ref)
        assert err <= TOL[cfg.dtype], (act, e, rows[e], err)


def test_router_paths_agree():
    """bf16 routers with E <= 64 run the fused router kernel (GEMM, softmax, top-k in one
    launch) with or without a workspace; wider ones with E a multiple of 64 run on the
    grouped GEMM when a workspace is given, otherwise on the router kernel.  Every path
    matches the oracle's logits, and each routing is bit-exact against the oracle run on
    its own logits."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    for name in ("deepseek_v3_small", "switch_skewed_small"):
        cfg = SMALL[name]
        inp, o, layer = run_layer(cfg)
        dev, c = layer.dev, layer.cfg
        N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
        z_ref = oracle.router_logits(oracle.to_f64(inp.x, cfg.dtype), oracle.to_f64(inp.w_router, cfg.dtype),
                                     inp.logit_bias)
        zs = []
        for ws in (layer.ws, None):
            z = torch.empty((N, E), dtype=torch.float32, device="cuda")
            idx = torch.empty((N, k), dtype=torch.int32, device="cuda")
            g = torch.empty((N, k), dtype=torch.float32, device="cuda")
            M.route(c, dev["x"], dev["w_router"], idx, g, logit_bias=dev["logit_bias"], sel_bias=dev["sel_bias"],
                    logits=z, ws=ws)
            torch.cuda.synchronize()
            zh = host(z)
            assert rel_err(zh, z_ref) <= TOL[cfg.dtype], (name, ws is None)
            r = oracle.oracle_route(cfg, zh, inp.sel_bias)
            assert np.array_equal(host(idx), r.topk_idx), (name, ws is None)
            zs.append(zh)
        assert rel_err(zs[0], zs[1]) <= 1e-5, (name, rel_err(zs[0], zs[1]))
        assert np.array_equal(zs[0], o["logits"]), name   # moe_forward takes the GEMM path


@pytest.mark.parametrize("variant", ["shared_no_residual", "padded_capacity"])
def test_down_combine_matches_unfused(variant):
    """moe_expert_down_combine (top-1: the gate-weighted combine in the down
    projection's epilogue) gives the bits of moe_expert_down + moe_combine,
    including dropped tokens, padding rows and a shared expert."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    if variant == "shared_no_residual":
        cfg = SMALL["deepseek_v3_small"].scaled(name="top1_shared", top_k=1, residual=False, n_tokens=700)
    else:
        cfg = SMALL["switch_skewed_small"].scaled(name="top1_padded", capacity_layout="padded",
                                                  capacity_priority="choice")
    inp = make_inputs(cfg)
    dev = M.upload_inputs(inp, "cuda")
    c = M.config_from(cfg)
    N, E, d, F, Fs = cfg.n_tokens, cfg.n_experts, cfg.d_model, cfg.d_ff, cfg.d_ff_shared
    R = M._lib.expert_rows(c)
    st = torch.bfloat16
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device="cuda")
    idx = torch.empty((N, 1), dtype=torch.int32, device="cuda")
    g = torch.empty((N, 1), dtype=torch.float32, device="cuda")
    z = torch.empty((N, E), dtype=torch.float32, device="cuda")
    M.route(c, dev["x"], dev["w_router"], idx, g, logit_bias=dev["logit_bias"], sel_bias=dev["sel_bias"], logits=z,
            ws=ws)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offs = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(max(R, 1), dtype=torch.int32, device="cuda")
    sp = torch.empty(N, dtype=torch.int32, device="cuda")
    M.permute(c, idx, None, counts, offs, perm, sp, None, ws=ws)
    h = torch.empty((max(R, 1), F), dtype=st, device="cuda")
    M.expert_up_gather(c, dev["x"], perm, offs, dev["w1"], dev["w3"], h, b1=dev["b1"], ws=ws)
    ysh = None
    if Fs:
        hsh = torch.empty((N, Fs), dtype=st, device="cuda")
        ysh = torch.empty((N, d), dtype=st, device="cuda")
        M.shared_ffn(c, dev["x"], dev["sh_w1"], dev["sh_w3"], dev["sh_w2"], hsh, ysh, ws=ws)
    res = dev["x"] if cfg.residual else None
    y = torch.empty((max(R, 1), d), dtype=st, device="cuda")
    M.expert_down(c, h, offs, dev["w2"], y, b2=dev["b2"], ws=ws)
    ref = torch.empty((N, d), dtype=st, device="cuda")
    M.combine(c, y, sp, g, ref, residual=res, shared_y=ysh)
    out = torch.full((N, d), float("nan"), dtype=st, device="cuda")
    M.expert_down_combine(c, h, offs, perm, sp, g, dev["w2"], out, b2=dev["b2"], residual=res, shared_y=ysh, ws=ws)
    torch.cuda.synchronize()
    dropped = int((host(sp) < 0).sum())
    say(f"down_combine {variant}: N={N} E={E} dropped={dropped}")
    assert np.array_equal(host(out), host(ref))


def test_combine_streaming_matches_cached():
    """moe_combine switches to nontemporal loads and stores once the expert
    rows exceed the 256 MB last-level cache; the arithmetic is the same, so
    the first tokens of a large call must give the bits of a small call over
    the same rows (the large call's parity against the oracle is covered at
    the DeepSeek-V3 full size)."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    from workloads import DEEPSEEK_V3
    N, k, d, T = 8192, 8, 2112, 512                       # 8192 * 8 * 2112 * 2 B = 277 MB of expert rows
    big = DEEPSEEK_V3.scaled(name="combine_stream", n_tokens=N, d_model=d, d_ff=64, d_ff_shared=0)
    small = big.scaled(name="combine_cached", n_tokens=T)
    gen = torch.Generator(device="cuda").manual_seed(11)
    y = (torch.randn((N * k, d), device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    slot_pos = torch.randperm(N * k, device="cuda", generator=gen).to(torch.int32)
    slot_pos[3 * k + 1] = -1                                # a dropped slot
    gates = torch.rand((N, k), device="cuda", generator=gen)
    res = (torch.randn((N, d), device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    out = torch.empty((N, d), dtype=torch.bfloat16, device="cuda")
    M.combine(M.config_from(big), y, slot_pos, gates, out, residual=res)
    # the small call reads the same rows, renumbered 0 .. T k - 1
    sp = slot_pos[: T * k].long()
    kept = sp >= 0
    y_small = torch.zeros((T * k, d), dtype=torch.bfloat16, device="cuda")
    y_small[kept.nonzero().squeeze(1)] = y[sp[kept]]
    sp_small = torch.where(kept, torch.arange(T * k, device="cuda"), torch.full_like(sp, -1)).to(torch.int32)
    out_small = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    M.combine(M.config_from(small), y_small, sp_small, gates[:T].contiguous(), out_small,
              residual=res[:T].contiguous())
    torch.cuda.synchronize()
    say(f"combine streaming: {N * k * d * 2 / 2**20:.0f} MiB of expert rows against {T * k * d * 2 / 2**20:.0f} MiB")
    assert torch.equal(out[:T], out_small)


@pytest.mark.parametrize("d,T", [(4096, 16), (4096, 100), (2048, 3), (7168, 8)])
def test_combine_small_batch_split_matches(d, T):
    """A batch of fewer than 1024 tokens spreads each token's row over up to 8
    wavefronts (contiguous column ranges, the same per-element arithmetic): its
    output must be bit-identical to one wavefront per token, which a batch of
    1024 or more tokens uses, over the same expert rows and shared-expert rows."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    from workloads import MIXTRAL_PREFILL
    N, k = 1100, 2
    big = MIXTRAL_PREFILL.scaled(name="combine_big", n_tokens=N, d_model=d, d_ff=64)
    small = big.scaled(name="combine_small", n_tokens=T)
    gen = torch.Generator(device="cuda").manual_seed(12)
    y = (torch.randn((N * k, d), device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    slot_pos = torch.randperm(N * k, device="cuda", generator=gen).to(torch.int32)
    slot_pos[1] = -1                                        # a dropped slot
    gates = torch.rand((N, k), device="cuda", generator=gen)
    res = (torch.randn((N, d), device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    sh = (torch.randn((N, d), device="cuda", generator=gen) * 0.1).to(torch.bfloat16)
    out = torch.empty((N, d), dtype=torch.bfloat16, device="cuda")
    M.combine(M.config_from(big), y, slot_pos, gates, out, residual=res, shared_y=sh)
    out_small = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    M.combine(M.config_from(small), y, slot_pos[: T * k].contiguous(), gates[:T].contiguous(), out_small,
              residual=res[:T].contiguous(), shared_y=sh[:T].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out[:T], out_small)


@pytest.mark.parametrize("priority", ["slot", "choice"])
def test_small_dispatch_matches_three_pass(priority):
    """At most 1024 slots, packed, no row copy: the single-workgroup dispatch
    kernel.  Its counts, offsets, permutation, slot positions and drop count
    must equal the three-kernel path's (taken when x_perm is requested) and the
    oracle's dispatch of the same routing, with capacity drops."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    from workloads import SWITCH_SKEWED
    cfg = SWITCH_SKEWED.scaled(name="small_dispatch", n_tokens=500, n_experts=64, top_k=2, d_model=128, d_ff=128,
                               gate_rule="topk_softmax", capacity_factor=1.5, capacity_priority=priority)
    c = M.config_from(cfg)
    N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
    gen = torch.Generator(device="cuda").manual_seed(13)
    # skewed routing: expert 3 in most tokens' first choice, second choices spread
    idx = torch.randint(0, E, (N, k), device="cuda", generator=gen, dtype=torch.int32)
    idx[: 2 * N // 3, 0] = 3
    idx[:, 1] = torch.where(idx[:, 1] == idx[:, 0], (idx[:, 1] + 1) % E, idx[:, 1])
    x = torch.zeros((N, cfg.d_model), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device="cuda")
    outs = []
    for xp in (None, torch.empty((N * k, cfg.d_model), dtype=torch.bfloat16, device="cuda")):
        o = [torch.full((E,), -7, dtype=torch.int32, device="cuda"), torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
             torch.full((N * k,), -7, dtype=torch.int32, device="cuda"), torch.full((N * k,), -7, dtype=torch.int32, device="cuda"),
             torch.full((1,), -7, dtype=torch.int64, device="cuda")]
        M.permute(c, idx, x, o[0], o[1], o[2], o[3], xp, drop_count=o[4], ws=ws)
        torch.cuda.synchronize()
        outs.append([host(t) for t in o])
    kept = int(outs[0][1][-1])
    ref = oracle.dispatch(host(idx).astype(np.int64), E, cfg.capacity, "packed", priority)
    assert ref.drop_count > 0
    (cf, of, pf, sf, df), (ct, ot, pt, st, dt) = outs               # fused, three-pass
    assert np.array_equal(cf, ct) and np.array_equal(of, ot) and np.array_equal(sf, st) and np.array_equal(df, dt)
    assert np.array_equal(pf[:kept], pt[:kept])
    assert np.array_equal(outs[0][0], ref.counts) and np.array_equal(outs[0][1], ref.offsets)
    assert np.array_equal(outs[0][2][:kept], ref.perm) and np.array_equal(outs[0][3], ref.slot_pos)
    assert int(outs[0][4][0]) == ref.drop_count


@pytest.mark.parametrize("n_tokens,d_model", [(1100, 512), (66000, 512)])
def test_wide_router_split_logits(n_tokens, d_model):
    """E = 256 on the logits GEMM: the top-k kernel completes the logits from the
    GEMM's K-part partials.  1100 tokens: four 256-row tiles and two 64-row
    tiles, all split along K; 66000 tokens: more 256-row tiles than workgroups,
    so the first ones are final in the GEMM's own epilogue and only the
    remainder is split.  Logits against the oracle's and the router kernel's
    (no workspace), routing and probability sums oracle-exact on the GPU's
    logits."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    from workloads import DEEPSEEK_V3
    cfg = DEEPSEEK_V3.scaled(name=f"wide_router_{n_tokens}", n_tokens=n_tokens, d_model=d_model, d_ff=64,
                             d_ff_shared=0)
    say(f"wide router: N={n_tokens} d={d_model} E={cfg.n_experts}")
    inp = make_inputs(cfg)
    c = M.config_from(cfg)
    N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
    x = M.to_device(inp.x, "cuda", cfg.dtype)
    wr = M.to_device(inp.w_router, "cuda", cfg.dtype)
    sb = M.to_device(inp.sel_bias, "cuda", "f32")
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device="cuda")
    z_ref = oracle.router_logits(oracle.to_f64(inp.x, cfg.dtype), oracle.to_f64(inp.w_router, cfg.dtype),
                                 inp.logit_bias)
    zs = []
    for w in (ws, None):
        z = torch.empty((N, E), dtype=torch.float32, device="cuda")
        idx = torch.empty((N, k), dtype=torch.int32, device="cuda")
        g = torch.empty((N, k), dtype=torch.float32, device="cuda")
        ps = torch.empty(E, dtype=torch.float32, device="cuda")
        M.route(c, x, wr, idx, g, sel_bias=sb, logits=z, probsum=ps if w is not None else None, ws=w)
        torch.cuda.synchronize()
        zh = host(z)
        assert rel_err(zh, z_ref) <= TOL[cfg.dtype], (w is None, rel_err(zh, z_ref))
        r = oracle.oracle_route(cfg, zh, inp.sel_bias)
        assert np.array_equal(host(idx), r.topk_idx), w is None
        assert rel_err(host(g), r.gates) <= TOL[cfg.dtype]
        if w is not None:
            assert rel_err(host(ps), r.probs.sum(axis=0)) <= 1e-5
        zs.append(zh)
    assert rel_err(zs[0], zs[1]) <= 1e-5, rel_err(zs[0], zs[1])


@pytest.mark.parametrize("n_tokens,d_model,d_ff_shared", [
    (100, 256, 192),     # under 128 rows: 64-row tiles only
    (200, 256, 192),     # one 256-row tile (at least 128 rows), no 64-row tile
    (512, 2048, 256),    # two whole 256-row tiles, few units: K-split, fix-up
    (600, 256, 192),     # 256-row tiles and a 64-row tail
    (1300, 512, 2048),   # 256-row tiles (a tail of 20 rows in 64-row tiles), many units
])
def test_shared_ffn_dense_plans(n_tokens, d_model, d_ff_shared):
    """The shared expert is one dense segment whose tile counts and K-split plan the host
    knows, so only the kernels that have work are launched.  Every row of y_sh against
    the oracle's SwiGLU, over row counts that need 64-row tiles only, 256-row tiles only,
    both, and with and without K-parts."""
    import torch
    import mixture_experts_layer_histogram_amd as M
    from workloads import DEEPSEEK_V3
    cfg = DEEPSEEK_V3.scaled(name=f"shared_{n_tokens}_{d_model}_{d_ff_shared}", n_tokens=n_tokens,
                             d_model=d_model, n_experts=8, top_k=2, d_ff=64, d_ff_shared=d_ff_shared)
    inp = make_inputs(cfg)
    c = M.config_from(cfg)
    N, d, Fs = cfg.n_tokens, cfg.d_model, cfg.d_ff_shared
    dt = cfg.dtype
    x = M.to_device(inp.x, "cuda", dt)
    w1, w3, w2 = (M.to_device(a, "cuda", dt) for a in (inp.sh_w1, inp.sh_w3, inp.sh_w2))
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device="cuda")
    h = torch.empty((N, Fs), dtype=torch.bfloat16, device="cuda")
    y = torch.full((N, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.shared_ffn(c, x, w1, w3, w2, h, y, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.ffn_swiglu(oracle.to_f64(inp.x, dt), oracle.to_f64(inp.sh_w1, dt), oracle.to_f64(inp.sh_w3, dt),
                            oracle.to_f64(inp.sh_w2, dt))
    yh = host(y)
    assert np.isfinite(yh).all(), "rows left unwritten"
    err = rel_err(yh, ref)
    say(f"shared N={N} d={d} Fs={Fs}: rel err {err:.3e}")
    assert err <= TOL[dt], err
