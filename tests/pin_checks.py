"""Checks that pin the fp64 oracle to facts outside itself.

Each ``check_*`` raises AssertionError when the oracle disagrees with what the
pages print, with a closed form, with brute force on tiny inputs, or with an
independent library routine.  ``test_oracle_pins.py`` runs them as they are;
``test_oracle_mutations.py`` plants plausible mistakes in the oracle and shows
that some check catches each one.
"""
from __future__ import annotations

import ast
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as TF

import oracle.moe_oracle as mo
from workloads import (TINY_TOP2_FP32, MoEConfig, make_inputs, GATE_TOPK_SOFTMAX,
                       GATE_SOFTMAX_RENORM, GATE_SWITCH_TOP1)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = ast.literal_eval(v.strip())
    return vals


# ----------------------------------------------------------------- printed example

def check_printed_example():
    """Glossary page, "Load balancing and expert capacity": the seeded top-2
    example prints the chosen expert pairs and the tokens per expert."""
    g = _golden("glossary_top2_example.txt")
    inp = make_inputs(TINY_TOP2_FP32)
    r, _ = mo.oracle_layer(TINY_TOP2_FP32, inp)
    assert r.topk_idx.tolist() == g["experts_per_token"], r.topk_idx.tolist()
    assert r.disp.counts.tolist() == g["tokens_per_expert"], r.disp.counts.tolist()


def check_printed_example_output():
    """The same example's layer output, computed here with torch's own fp32
    modules (every expert run densely on every token, then masked), agrees
    with the oracle to fp32 accuracy."""
    cfg = TINY_TOP2_FP32
    inp = make_inputs(cfg)
    _, out = mo.oracle_layer(cfg, inp)
    x = torch.from_numpy(inp.x)
    router = torch.nn.Linear(cfg.d_model, cfg.n_experts, bias=False)
    with torch.no_grad():
        router.weight.copy_(torch.from_numpy(inp.w_router))
        logits = router(x)
        top_val, top_idx = torch.topk(logits, cfg.top_k, dim=-1)
        w = torch.softmax(top_val, dim=-1)
        ref = torch.zeros_like(x)
        for e in range(cfg.n_experts):
            l1 = torch.nn.Linear(cfg.d_model, cfg.d_ff)
            l2 = torch.nn.Linear(cfg.d_ff, cfg.d_model)
            l1.weight.copy_(torch.from_numpy(inp.w1[e])); l1.bias.copy_(torch.from_numpy(inp.b1[e]))
            l2.weight.copy_(torch.from_numpy(inp.w2[e])); l2.bias.copy_(torch.from_numpy(inp.b2[e]))
            ye = l2(torch.nn.GELU()(l1(x)))                      # all tokens, dense
            mask = (top_idx == e).to(torch.float32)              # [N, k]
            ref += (mask * w).sum(dim=1, keepdim=True) * ye
    ref = ref.double().numpy()
    err = np.abs(out - ref).max() / np.abs(ref).max()
    assert err <= 1e-5, err


# ----------------------------------------------------------------- selection

def _brute_rank(key_row):
    """rank[e] = #{e' : key[e'] > key[e] or (key[e'] == key[e] and e' < e)}."""
    E = key_row.size
    return np.array([sum(1 for f in range(E) if key_row[f] > key_row[e] or (key_row[f] == key_row[e] and f < e))
                     for e in range(E)])


def _brute_topk(key, k):
    out = np.zeros((key.shape[0], k), np.int64)
    for t in range(key.shape[0]):
        rank = _brute_rank(key[t])
        for e in range(key.shape[1]):
            if rank[e] < k:
                out[t, rank[e]] = e
    return out


def _tiny_keys(seed, N=40, E=8, tie_heavy=True):
    rng = np.random.default_rng(seed)
    if tie_heavy:
        return rng.choice(np.array([-1.0, 0.25, 0.5]), size=(N, E))
    return rng.standard_normal((N, E))


def check_topk_brute_force():
    """Top-k with ties to the lower index equals an O(E^2) brute-force rank."""
    for seed in range(6):
        for E in (1, 3, 8):
            for k in range(1, E + 1):
                key = _tiny_keys(seed, E=E, tie_heavy=seed % 2 == 0)
                assert np.array_equal(mo.top_k_desc(key, k), _brute_topk(key, k)), (seed, E, k)


def check_route_selection_brute_force():
    """Each gate rule selects by its own key: A on z + b, B on softmax(z) + b,
    C on z alone; compared against the brute-force rank."""
    rng = np.random.default_rng(7)
    for E, k in ((8, 2), (6, 3), (5, 1)):
        z = rng.choice(np.array([-0.5, 0.0, 0.75, 1.0]), size=(30, E))
        b = rng.choice(np.array([0.0, 0.25]), size=E).astype(np.float32)
        idx, _, _ = mo.route(z, k, GATE_TOPK_SOFTMAX, b)
        assert np.array_equal(idx, _brute_topk(z + b.astype(np.float64), k))
        idx, _, _ = mo.route(z, k, GATE_SOFTMAX_RENORM, b)
        p = scipy.special.softmax(z, axis=1)
        assert np.array_equal(idx, _brute_topk(p + b.astype(np.float64), k))
        idx, _, _ = mo.route(z, 1, GATE_SWITCH_TOP1, None)
        assert np.array_equal(idx, _brute_topk(z, 1))


# ----------------------------------------------------------------- gates

def check_softmax_library():
    """Row softmax equals scipy's, including rows whose logits would overflow exp."""
    rng = np.random.default_rng(3)
    z = rng.standard_normal((20, 9)) * 4
    z[0] = 1000.0 + np.arange(9)
    z[1] = -1000.0 - np.arange(9)
    ref = scipy.special.softmax(z, axis=1)
    got = mo.softmax_rows(z)
    assert np.all(np.isfinite(got))
    assert np.allclose(got, ref, rtol=1e-13, atol=0)


def check_gate_closed_forms():
    rng = np.random.default_rng(11)
    N, E, k = 64, 8, 3
    z = rng.standard_normal((N, E)) * 2
    # rule A: softmax over the selected raw logits (scipy on the selected values)
    idx, g, _ = mo.route(z, k, GATE_TOPK_SOFTMAX, None)
    ref = scipy.special.softmax(np.take_along_axis(z, idx, 1), axis=1)
    assert np.allclose(g, ref, rtol=1e-13, atol=1e-15)
    assert np.allclose(g.sum(1), 1.0, rtol=0, atol=1e-14)
    # rule A == rule B without bias: softmax over S equals p_S / sum p_S
    idxb, gb, _ = mo.route(z, k, GATE_SOFTMAX_RENORM, None)
    assert np.array_equal(idx, idxb)
    assert np.allclose(g, gb, rtol=1e-12, atol=1e-15)
    # rule C: gate is the full-softmax probability of the argmax, at least 1/E
    idxc, gc, _ = mo.route(z, 1, GATE_SWITCH_TOP1, None)
    p = scipy.special.softmax(z, axis=1)
    assert np.array_equal(idxc[:, 0], np.argmax(z, axis=1))
    assert np.allclose(gc[:, 0], p[np.arange(N), idxc[:, 0]], rtol=1e-13)
    assert np.all(gc >= 1.0 / E - 1e-15)


def check_bias_moves_selection_not_gates():
    """[L] Step 1: the bias changes which experts are picked, never the gate
    values computed from the raw scores."""
    rng = np.random.default_rng(5)
    N, E, k = 200, 8, 2
    z = rng.standard_normal((N, E))
    b = (rng.random(E).astype(np.float32) - np.float32(0.5)) * np.float32(0.6)
    for rule in (GATE_TOPK_SOFTMAX, GATE_SOFTMAX_RENORM):
        i0, g0, _ = mo.route(z, k, rule, None)
        i1, g1, _ = mo.route(z, k, rule, b)
        same = np.array([set(i0[t]) == set(i1[t]) for t in range(N)])
        changed = ~same
        assert same.sum() > 0 and changed.sum() > 0
        for t in np.nonzero(same)[0]:
            m0 = dict(zip(i0[t], g0[t]))
            m1 = dict(zip(i1[t], g1[t]))
            assert all(abs(m0[e] - m1[e]) < 1e-14 for e in m0)
    # a bias large enough to force expert 5 in: its gate is the raw-logit softmax over the forced set
    bf = np.zeros(E, np.float32)
    bf[5] = 100.0
    i2, g2, _ = mo.route(z, k, GATE_TOPK_SOFTMAX, bf)
    assert np.all(i2[:, 0] == 5)
    ref = scipy.special.softmax(np.take_along_axis(z, i2, 1), axis=1)
    assert np.allclose(g2, ref, rtol=1e-13)


# ----------------------------------------------------------------- dispatch / capacity

def check_dispatch_invariants():
    rng = np.random.default_rng(9)
    for E, k, N in ((8, 2, 50), (16, 4, 33), (5, 1, 17)):
        z = rng.standard_normal((N, E))
        idx, _, _ = mo.route(z, k, GATE_TOPK_SOFTMAX, None)
        d = mo.dispatch(idx, E, None)
        assert int(d.counts.sum()) == N * k                              # exactly k experts per token
        assert np.array_equal(d.counts, np.bincount(idx.reshape(-1), minlength=E))
        assert sorted(d.perm.tolist()) == list(range(N * k))            # a permutation of all slots
        assert d.offsets[0] == 0 and d.offsets[-1] == N * k
        for e in range(E):
            seg = d.perm[d.offsets[e]:d.offsets[e + 1]]
            assert np.all(np.diff(seg) > 0)                              # ascending slot id
            assert np.all(idx.reshape(-1)[seg] == e)
        assert np.array_equal(d.perm[d.slot_pos], np.arange(N * k))
        assert d.drop_count == 0


def check_capacity_brute_force():
    """Each expert keeps the first C of its slots in slot order; drop = sum max(0, count - C)."""
    rng = np.random.default_rng(21)
    for E, k, N, C in ((4, 1, 40, 6), (8, 2, 30, 5), (6, 3, 20, 0)):
        z = rng.standard_normal((N, E))
        z[:, 1] += 1.0                                                   # skew towards expert 1
        idx, _, _ = mo.route(z, k, GATE_TOPK_SOFTMAX, None)
        d = mo.dispatch(idx, E, C)
        es = idx.reshape(-1)
        for s in range(N * k):
            rank = int(np.sum(es[:s] == es[s]))                          # earlier slots on the same expert
            assert (d.slot_pos[s] >= 0) == (rank < C), (s, rank, C)
        assert np.array_equal(np.diff(d.offsets), np.minimum(d.counts, C))
        assert d.drop_count == int(np.maximum(d.counts - C, 0).sum())


def check_capacity_choice_priority_brute_force():
    """Choice priority: an over-full expert keeps the slots with the smallest
    (choice rank j, token t); its rows hold them in that order.  With k = 1 it
    coincides with slot priority."""
    rng = np.random.default_rng(22)
    for E, k, N, C in ((4, 2, 30, 6), (5, 3, 24, 4), (4, 1, 40, 7), (6, 3, 20, 0)):
        z = rng.standard_normal((N, E))
        z[:, 1] += 1.0
        idx, _, _ = mo.route(z, k, GATE_TOPK_SOFTMAX, None)
        d = mo.dispatch(idx, E, C, "packed", "choice")
        es = idx.reshape(-1)
        for s in range(N * k):
            t, j = divmod(s, k)
            ahead = sum(1 for s2 in range(N * k) if es[s2] == es[s] and (s2 % k, s2 // k) < (j, t))
            assert (d.slot_pos[s] >= 0) == (ahead < C), (s, ahead, C)
            if d.slot_pos[s] >= 0:
                assert d.slot_pos[s] == d.offsets[es[s]] + ahead
        assert d.drop_count == int(np.maximum(d.counts - C, 0).sum())
        if k == 1:
            d0 = mo.dispatch(idx, E, C)
            assert np.array_equal(d.perm, d0.perm) and np.array_equal(d.slot_pos, d0.slot_pos)


def check_padded_capacity_layout():
    """Padded layout: expert e owns rows [e C, (e+1) C), its kept slots first
    (same order as packed), padding rows marked -1; the layer output does not
    depend on the layout."""
    rng = np.random.default_rng(23)
    E, k, N, C = 4, 2, 30, 9
    z = rng.standard_normal((N, E))
    z[:, 2] += 1.5
    idx, _, _ = mo.route(z, k, GATE_TOPK_SOFTMAX, None)
    for pr in ("slot", "choice"):
        pk = mo.dispatch(idx, E, C, "packed", pr)
        pd = mo.dispatch(idx, E, C, "padded", pr)
        assert np.array_equal(pd.offsets, np.arange(E + 1) * C)
        for e in range(E):
            n = pk.kept[e]
            assert np.array_equal(pd.perm[e * C:e * C + n], pk.perm[pk.offsets[e]:pk.offsets[e + 1]])
            assert np.all(pd.perm[e * C + n:(e + 1) * C] == -1)
        assert np.array_equal(pd.slot_pos >= 0, pk.slot_pos >= 0)
        ok = pd.slot_pos >= 0
        assert np.array_equal(pd.perm[pd.slot_pos[ok]], np.nonzero(ok)[0])
    cfg = MoEConfig(name="padded", n_tokens=N, d_model=16, n_experts=E, top_k=k, d_ff=24, act="swiglu",
                    gate_rule=GATE_TOPK_SOFTMAX, dtype="f32", capacity_factor=C * E / N, residual=True)
    assert cfg.capacity == C
    inp, _ = _small_inputs(cfg, seed=4)
    import dataclasses
    _, out_packed = mo.oracle_layer(cfg, inp, logits_override=z.astype(np.float32))
    _, out_padded = mo.oracle_layer(dataclasses.replace(cfg, capacity_layout="padded"), inp,
                                    logits_override=z.astype(np.float32))
    assert np.array_equal(out_packed, out_padded)


# ----------------------------------------------------------------- layer reductions

def _small_inputs(cfg, w_override=None, seed=0):
    """fp32 inputs drawn directly (independent of the workload presets)."""
    rng = np.random.default_rng(seed)
    N, d, E, F = cfg.n_tokens, cfg.d_model, cfg.n_experts, cfg.d_ff

    class Inp:
        pass
    inp = Inp()
    inp.cfg = cfg
    inp.x = rng.standard_normal((N, d)).astype(np.float32)
    inp.w_router = (rng.standard_normal((E, d)) / np.sqrt(d)).astype(np.float32)
    inp.logit_bias = None
    inp.sel_bias = None
    ws = []
    for e in range(E):
        w = {"w1": (rng.standard_normal((F, d)) / np.sqrt(d)).astype(np.float32),
             "w2": (rng.standard_normal((d, F)) / np.sqrt(F)).astype(np.float32)}
        if cfg.act == "swiglu":
            w["w3"] = (rng.standard_normal((F, d)) / np.sqrt(d)).astype(np.float32)
        if cfg.ffn_bias:
            w["b1"] = rng.standard_normal(F).astype(np.float32) * np.float32(0.1)
            w["b2"] = rng.standard_normal(d).astype(np.float32) * np.float32(0.1)
        ws.append(w)
    if w_override == "identical":
        ws = [ws[0]] * E
    inp.expert = lambda e: ws[e]
    inp.sh_w1 = inp.sh_w3 = inp.sh_w2 = None
    return inp, ws


def _torch_dense_ffn(act, x, w):
    """Dense FFN in torch float64 (library ops, independent of the oracle)."""
    X = torch.from_numpy(x.astype(np.float64))
    t = {k: torch.from_numpy(v.astype(np.float64)) for k, v in w.items()}
    if act == "swiglu":
        h = TF.silu(TF.linear(X, t["w1"])) * TF.linear(X, t["w3"])
        return TF.linear(h, t["w2"]).numpy()
    h = TF.gelu(TF.linear(X, t["w1"], t.get("b1")), approximate="none")
    return TF.linear(h, t["w2"], t.get("b2")).numpy()


def check_single_expert_is_dense():
    """E = 1, k = 1: the layer is x + FFN(x) (the dense block of [L] "FFN swap")."""
    for act, bias in (("swiglu", False), ("gelu", True)):
        cfg = MoEConfig(name="dense", n_tokens=13, d_model=24, n_experts=1, top_k=1, d_ff=40,
                        act=act, ffn_bias=bias, dtype="f32", residual=True)
        inp, ws = _small_inputs(cfg, seed=1)
        _, out = mo.oracle_layer(cfg, inp)
        ref = inp.x.astype(np.float64) + _torch_dense_ffn(act, inp.x, ws[0])
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12), np.abs(out - ref).max()


def check_identical_experts_are_dense():
    """With every expert identical, gates summing to 1 make any top-k layer dense
    (rules A and B); rule C scales the dense FFN by the chosen probability."""
    for rule, k in ((GATE_TOPK_SOFTMAX, 3), (GATE_SOFTMAX_RENORM, 2), (GATE_SWITCH_TOP1, 1)):
        for act, bias in (("swiglu", False), ("gelu", True)):
            cfg = MoEConfig(name="ident", n_tokens=11, d_model=16, n_experts=5, top_k=k, d_ff=20,
                            act=act, ffn_bias=bias, dtype="f32", residual=True, gate_rule=rule)
            inp, ws = _small_inputs(cfg, w_override="identical", seed=2)
            r, out = mo.oracle_layer(cfg, inp)
            dense = _torch_dense_ffn(act, inp.x, ws[0])
            scale = np.ones((cfg.n_tokens, 1))
            if rule == GATE_SWITCH_TOP1:
                z = inp.x.astype(np.float64) @ inp.w_router.astype(np.float64).T
                scale = scipy.special.softmax(z, axis=1).max(axis=1, keepdims=True)
            ref = inp.x.astype(np.float64) + scale * dense
            assert np.allclose(out, ref, rtol=1e-12, atol=1e-12), (rule, act, np.abs(out - ref).max())


def check_dropped_tokens_pass_residual():
    """[N] item 2 / [G]: overflow tokens skip the experts and keep the residual."""
    cfg = MoEConfig(name="cap", n_tokens=40, d_model=16, n_experts=4, top_k=1, d_ff=12, act="gelu",
                    ffn_bias=True, dtype="f32", residual=True, gate_rule=GATE_SWITCH_TOP1,
                    capacity_factor=0.5)
    inp, _ = _small_inputs(cfg, seed=4)
    inp.logit_bias = np.array([0, 3.0, 0, 0], np.float32)              # most tokens want expert 1
    r, out = mo.oracle_layer(cfg, inp)
    dropped = np.nonzero(r.disp.slot_pos < 0)[0]
    assert dropped.size > 0 and cfg.capacity == 5
    x64 = inp.x.astype(np.float64)
    assert np.array_equal(out[dropped], x64[dropped])
    kept = np.nonzero(r.disp.slot_pos >= 0)[0]
    assert not np.array_equal(out[kept], x64[kept])


def _torch_layer_independent(cfg, inp):
    """The whole forward in torch float64, routing included, written without
    the oracle: logits by torch.linear; rule B keys softmax(z) + bias, ranked by
    a stable descending torch.sort; capacity by walking the slots t*k + j in
    ascending order with a per-expert counter; the shared SwiGLU added to every
    token with weight 1 ([L] "Shared experts": every token passes through it)."""
    N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
    bits = lambda a: torch.from_numpy(np.asarray(a, np.uint16).view(np.int16)).view(torch.bfloat16).double()
    cv = (bits if cfg.dtype == "bf16" else lambda a: torch.from_numpy(np.asarray(a, np.float32)).double())
    x = cv(inp.x)
    z = TF.linear(x, cv(inp.w_router))
    if inp.logit_bias is not None:
        z = z + torch.from_numpy(np.asarray(inp.logit_bias, np.float32)).double()
    b = torch.zeros(E, dtype=torch.float64) if inp.sel_bias is None else \
        torch.from_numpy(np.asarray(inp.sel_bias, np.float32)).double()
    p = torch.softmax(z, dim=1)
    assert cfg.gate_rule == GATE_SOFTMAX_RENORM
    idx = torch.sort(p + b, dim=1, descending=True, stable=True).indices[:, :k]
    ps = p.gather(1, idx)
    g = ps / ps.sum(dim=1, keepdim=True)
    C = cfg.capacity if cfg.capacity is not None else N * k
    taken = [0] * E
    kept = np.zeros((N, k), dtype=bool)
    for s in range(N * k):
        e = int(idx[s // k, s % k])
        if taken[e] < C:
            kept[s // k, s % k] = True
            taken[e] += 1
    out = x.clone() if cfg.residual else torch.zeros_like(x)
    if cfg.d_ff_shared:
        out = out + TF.linear(TF.silu(TF.linear(x, cv(inp.sh_w1))) * TF.linear(x, cv(inp.sh_w3)), cv(inp.sh_w2))
    for e in range(E):
        w = {n: cv(v) for n, v in inp.expert(e).items()}
        for t in range(N):
            for j in range(k):
                if kept[t, j] and int(idx[t, j]) == e:
                    xt = x[t:t + 1]
                    y = TF.linear(TF.silu(TF.linear(xt, w["w1"])) * TF.linear(xt, w["w3"]), w["w2"])
                    out[t] += g[t, j] * y[0]
    return out.numpy(), idx.numpy(), kept


def check_shared_expert_term():
    """The forward with a shared expert, rule B, a selection bias and capacity
    drops (so some tokens lose some or all of their slots) against the layer
    computed independently in torch: every token, dropped or not, gets the
    shared SwiGLU with weight 1 on top of its residual."""
    cfg = MoEConfig(name="shared_cap", n_tokens=48, d_model=32, n_experts=6, top_k=2, d_ff=24, d_ff_shared=40,
                    act="swiglu", gate_rule=GATE_SOFTMAX_RENORM, capacity_factor=1.0, dtype="bf16",
                    residual=True, sel_bias_range=0.2, seed=41)
    inp = make_inputs(cfg)
    inp.sel_bias = inp.sel_bias.copy()
    inp.sel_bias[2] += np.float32(0.5)                          # expert 2 over-full: drops
    r, out = mo.oracle_layer(cfg, inp)
    ref, idx, kept = _torch_layer_independent(cfg, inp)
    assert np.array_equal(r.topk_idx, idx)
    assert np.array_equal(r.disp.slot_pos.reshape(cfg.n_tokens, cfg.top_k) >= 0, kept)
    all_dropped = np.nonzero(~kept.any(axis=1))[0]
    part_dropped = np.nonzero(kept.any(axis=1) & ~kept.all(axis=1))[0]
    assert all_dropped.size > 0 and part_dropped.size > 0, (all_dropped.size, part_dropped.size)
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max(), np.abs(out - ref).max()


def check_rows_path():
    """``oracle_layer(rows=S)`` (the sampled form the full-size tests use) gives
    the rows S of the whole-batch output and the same routing, on shapes with a
    shared expert, capacity drops and the padded layout.  Equal up to the
    rounding of the matrix products only: BLAS picks its kernel by shape, so a
    product over fewer rows may round differently (measured: one ulp)."""
    cases = [
        MoEConfig(name="rows_b", n_tokens=40, d_model=16, n_experts=6, top_k=3, d_ff=20, d_ff_shared=12,
                  gate_rule=GATE_SOFTMAX_RENORM, capacity_factor=1.2, sel_bias_range=0.1, dtype="bf16", seed=42),
        MoEConfig(name="rows_c", n_tokens=33, d_model=12, n_experts=4, top_k=1, d_ff=8, act="gelu", ffn_bias=True,
                  gate_rule=GATE_SWITCH_TOP1, capacity_factor=0.75, capacity_layout="padded",
                  logit_offset=(1, 1.0), init="uniform_experts", dtype="f32", seed=43),
    ]
    for cfg in cases:
        inp = make_inputs(cfg)
        r_all, out_all = mo.oracle_layer(cfg, inp)
        assert r_all.disp.drop_count > 0, cfg.name
        for S in (np.array([0]), np.array([cfg.n_tokens - 1, 3, 17]), np.arange(1, cfg.n_tokens, 2),
                  np.nonzero(r_all.disp.slot_pos.reshape(cfg.n_tokens, cfg.top_k).min(axis=1) < 0)[0]):
            r_s, out_s = mo.oracle_layer(cfg, inp, rows=S)
            assert np.array_equal(r_s.topk_idx, r_all.topk_idx) and np.array_equal(r_s.disp.perm, r_all.disp.perm)
            assert out_s.shape == (S.size, cfg.d_model)
            assert np.abs(out_s - out_all[S]).max() <= 1e-14 * np.abs(out_all).max(), (cfg.name, S)


def check_bf16_decode_library():
    """Every one of the 65536 bfloat16 bit patterns decodes to torch's own
    bfloat16 value (NaN patterns to NaN, both zeros with their sign)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):                         # signalling-NaN patterns
        got = mo.to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got), np.signbit(ref))


# ----------------------------------------------------------------- balancing

def check_aux_uniform_is_one():
    """[G]: the Switch term is smallest (here: exactly 1) when the router
    probabilities are uniform, whatever the counts; and it reaches E when all
    tokens and all probability mass sit on one expert."""
    for E, k, N in ((8, 2, 30), (64, 1, 100), (5, 1, 7)):
        z = np.zeros((N, E))
        idx, _, p = mo.route(z, k, GATE_TOPK_SOFTMAX if k > 1 else GATE_SWITCH_TOP1, None)
        d = mo.dispatch(idx, E, max(1, N // (4 * E)))                  # heavy dropping on purpose
        assert abs(mo.aux_loss(d.counts, p, k) - 1.0) < 1e-12
    E, N = 16, 50
    z = np.full((N, E), -60.0)
    z[:, 3] = 60.0
    idx, _, p = mo.route(z, 1, GATE_SWITCH_TOP1, None)
    d = mo.dispatch(idx, E, None)
    assert abs(mo.aux_loss(d.counts, p, 1) - E) < 1e-9


def check_bias_step_signs():
    """[L] DeepSeek-V3 approach: over-target experts move down by gamma,
    under-target up by gamma, on-target stay."""
    E, N, k = 8, 12, 2                                                  # target N k / E = 3
    counts = np.array([3, 4, 2, 0, 9, 3, 1, 2])
    b = np.array([0.01, -0.02, 0, 0.5, -0.5, 0.25, 1.0, -1.0], np.float32)
    gamma = 1e-3
    signs, nb = mo.bias_step(counts, b, gamma, N, k)
    assert signs.tolist() == [0, 1, -1, -1, 1, 0, -1, -1]
    g32 = float(np.float32(gamma))
    for e in range(E):
        want = float(b[e]) - g32 * (1 if counts[e] > 3 else -1 if counts[e] < 3 else 0)
        assert abs(nb[e] - want) < 1e-15


def check_bias_loop_equalises():
    """[L] Step 2 / Exercises: repeated bias steps even out expert usage on a
    DeepSeek-V3-shaped batch (256 experts, top-8, bias ~ U(+-0.05), gamma 1e-3).
    The pages give no number; the bar here is a 10x drop of the load spread."""
    rng = np.random.default_rng(1234)
    N, E, k, gamma = 4096, 256, 8, 1e-3
    z = rng.standard_normal((N, E))
    b = ((rng.random(E) * 2 - 1) * 0.05).astype(np.float32)
    std0 = None
    for _ in range(50):
        idx, _, _ = mo.route(z, k, GATE_SOFTMAX_RENORM, b)
        counts = np.bincount(idx.reshape(-1), minlength=E)
        if std0 is None:
            std0 = counts.std()
        _, nb = mo.bias_step(counts, b, gamma, N, k)
        b = nb.astype(np.float32)
    idx, _, _ = mo.route(z, k, GATE_SOFTMAX_RENORM, b)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert counts.min() > 0
    assert counts.std() * 10 <= std0, (std0, counts.std())


def check_activation_library():
    """SiLU and exact GELU against 40-digit mpmath evaluations over [-30, 30]
    (relative error), and against torch's float64 ops where those are accurate."""
    import mpmath
    mpmath.mp.dps = 40
    u = np.linspace(-30, 30, 601)
    s_ref = np.array([float(mpmath.mpf(v) / (1 + mpmath.exp(-mpmath.mpf(v)))) for v in u])
    g_ref = np.array([float(mpmath.mpf(v) * mpmath.erfc(-mpmath.mpf(v) / mpmath.sqrt(2)) / 2) for v in u])
    nz = (g_ref != 0) & (s_ref != 0)
    assert np.max(np.abs(mo.silu(u)[nz] - s_ref[nz]) / np.abs(s_ref[nz])) < 1e-14
    assert np.max(np.abs(mo.gelu(u)[nz] - g_ref[nz]) / np.abs(g_ref[nz])) < 1e-12
    v = np.linspace(-6, 6, 1201)
    V = torch.from_numpy(v)
    assert np.allclose(mo.silu(v), TF.silu(V).numpy(), rtol=1e-14, atol=1e-16)
    assert np.allclose(mo.gelu(v), TF.gelu(V, approximate="none").numpy(), rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------- backward

def _torch_layer_loss(cfg, inp, idx, kept, counts, dout, d_aux, params):
    """The layer's forward written with torch ops (fp64) for fixed routing
    decisions, and the scalar <out, dout> + d_aux * aux whose gradients
    torch.autograd computes."""
    E, k = cfg.n_experts, cfg.top_k
    x, wr = params["x"], params["w_router"]
    z = x @ wr.T + params["logit_bias"][None, :]
    p = torch.softmax(z, dim=1)
    it = torch.from_numpy(idx)
    if cfg.gate_rule == GATE_TOPK_SOFTMAX:
        g = torch.softmax(z.gather(1, it), dim=1)
    elif cfg.gate_rule == GATE_SOFTMAX_RENORM:
        ps = p.gather(1, it)
        g = ps / ps.sum(dim=1, keepdim=True)
    else:
        g = p.gather(1, it)
    out = x.clone() if cfg.residual else torch.zeros_like(x)
    if cfg.d_ff_shared:
        out = out + TF.linear(TF.silu(TF.linear(x, params["sh_w1"])) * TF.linear(x, params["sh_w3"]),
                              params["sh_w2"])
    for t in range(cfg.n_tokens):
        for j in range(k):
            if not kept[t, j]:
                continue
            e = int(idx[t, j])
            xt = x[t:t + 1]
            if cfg.act == "swiglu":
                y = TF.linear(TF.silu(TF.linear(xt, params[f"w1_{e}"])) * TF.linear(xt, params[f"w3_{e}"]),
                              params[f"w2_{e}"])
            else:
                h = TF.gelu(TF.linear(xt, params[f"w1_{e}"], params.get(f"b1_{e}")), approximate="none")
                y = TF.linear(h, params[f"w2_{e}"], params.get(f"b2_{e}"))
            out = out.index_add(0, torch.tensor([t]), g[t, j] * y)
    loss = (out * torch.from_numpy(dout)).sum()
    if cfg.aux_loss:
        f = torch.from_numpy(counts.astype(np.float64)) / float(cfg.n_tokens * k)
        loss = loss + d_aux * E * (f * p.mean(dim=0)).sum()
    return loss


_BW_CASES = [
    MoEConfig(name="bw_a", n_tokens=20, d_model=12, n_experts=5, top_k=2, d_ff=16, act="swiglu",
              gate_rule=GATE_TOPK_SOFTMAX, dtype="f32", capacity_factor=1.5, residual=True, seed=31),
    MoEConfig(name="bw_b", n_tokens=18, d_model=12, n_experts=6, top_k=3, d_ff=10, d_ff_shared=14,
              act="swiglu", gate_rule=GATE_SOFTMAX_RENORM, dtype="f32", residual=True,
              sel_bias_range=0.05, seed=32),
    MoEConfig(name="bw_c", n_tokens=22, d_model=10, n_experts=4, top_k=1, d_ff=14, act="gelu", ffn_bias=True,
              gate_rule=GATE_SWITCH_TOP1, dtype="f32", capacity_factor=1.0, residual=True, aux_loss=True,
              logit_offset=(1, 0.7), init="uniform_experts", seed=33),
]


def _autograd_cases():
    """For each backward case: inputs, dout, d_aux and the torch.autograd leaves
    (x, w_router, logit_bias, every expert's weights, shared weights) after
    backward() of the layer's forward written with torch ops."""
    rng = np.random.default_rng(34)
    for cfg in _BW_CASES:
        inp = make_inputs(cfg)
        dout = rng.standard_normal((cfg.n_tokens, cfg.d_model))
        d_aux = 0.37 if cfg.aux_loss else 0.0
        r, _ = mo.oracle_layer(cfg, inp)
        kept = (r.disp.slot_pos >= 0).reshape(cfg.n_tokens, cfg.top_k)
        dt = cfg.dtype
        P = {"x": mo.to_f64(inp.x, dt), "w_router": mo.to_f64(inp.w_router, dt),
             "logit_bias": np.zeros(cfg.n_experts) if inp.logit_bias is None
             else np.asarray(inp.logit_bias, np.float64)}
        for e in range(cfg.n_experts):
            for n, v in inp.expert(e).items():
                P[f"{n}_{e}"] = mo.to_f64(v, dt)
        if cfg.d_ff_shared:
            for n in ("sh_w1", "sh_w3", "sh_w2"):
                P[n] = mo.to_f64(getattr(inp, n), dt)
        T = {n: torch.tensor(v, dtype=torch.float64, requires_grad=True) for n, v in P.items()}
        loss = _torch_layer_loss(cfg, inp, r.topk_idx, kept, r.disp.counts, dout, d_aux, T)
        loss.backward()
        yield cfg, inp, dout, d_aux, {n: t.grad.numpy() for n, t in T.items()}


def _close(a, b, what):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, what
    assert np.abs(a - b).max() <= 1e-11 * max(1.0, np.abs(b).max()), what


def check_backward_autograd():
    """The fp64 backward (router, gates for every rule, aux loss, experts with
    capacity drops, GELU biases, shared expert, residual) against
    torch.autograd on the same forward written with torch ops."""
    for cfg, inp, dout, d_aux, G in _autograd_cases():
        gr = mo.oracle_layer_backward(cfg, inp, dout, d_aux=d_aux)
        _close(gr["x"], G["x"], (cfg.name, "x"))
        _close(gr["w_router"], G["w_router"], (cfg.name, "w_router"))
        _close(gr["logit_bias"], G["logit_bias"], (cfg.name, "logit_bias"))
        for e in range(cfg.n_experts):
            for n in ("w1", "w3", "w2", "b1", "b2"):
                if f"{n}_{e}" in G:
                    _close(gr[n][e], G[f"{n}_{e}"], (cfg.name, f"{n}_{e}"))
        if cfg.d_ff_shared:
            for n in ("sh_w1", "sh_w3", "sh_w2"):
                _close(gr[n], G[n], (cfg.name, n))


def check_sampled_backward_autograd():
    """The sampled backward used at full sizes (a subset of token rows; a
    subset of each expert's hidden units) against torch.autograd: dx rows,
    expert and shared-expert weight-gradient columns and biases.  Its gate and
    logit gradients equal the whole-batch oracle's rows."""
    for cfg, inp, dout, d_aux, G in _autograd_cases():
        N, F = cfg.n_tokens, cfg.d_ff
        rows = np.arange(1, N, 3)                       # a strict subset (the aux term's N must stay N)
        rb = mo.oracle_backward_rows(cfg, inp, dout, rows, d_aux=d_aux)
        _close(rb["x"], G["x"][rows], (cfg.name, "rows x"))
        full = mo.oracle_layer_backward(cfg, inp, dout, d_aux=d_aux)
        _close(rb["gates"], full["gates"][rows], (cfg.name, "rows gates"))
        _close(rb["logits"], full["logits"][rows], (cfg.name, "rows logits"))
        cols = np.array([F - 1, 0, F // 2])
        for e in range(cfg.n_experts):
            gc = mo.oracle_expert_grad_columns(cfg, inp, dout, e, cols, rb["route"])
            _close(gc["w1"], G[f"w1_{e}"][cols], (cfg.name, e, "w1 cols"))
            _close(gc["w2"], G[f"w2_{e}"][:, cols], (cfg.name, e, "w2 cols"))
            if cfg.act == "swiglu":
                _close(gc["w3"], G[f"w3_{e}"][cols], (cfg.name, e, "w3 cols"))
            if cfg.ffn_bias:
                _close(gc["b1"], G[f"b1_{e}"][cols], (cfg.name, e, "b1 cols"))
                _close(gc["b2"], G[f"b2_{e}"], (cfg.name, e, "b2"))
        if cfg.d_ff_shared:
            sc = np.array([cfg.d_ff_shared - 1, 2])
            gs = mo.oracle_shared_grad_columns(cfg, inp, dout, sc)
            _close(gs["w1"], G["sh_w1"][sc], (cfg.name, "sh_w1 cols"))
            _close(gs["w3"], G["sh_w3"][sc], (cfg.name, "sh_w3 cols"))
            _close(gs["w2"], G["sh_w2"][:, sc], (cfg.name, "sh_w2 cols"))


def check_activation_grads_library():
    """SiLU' and GELU' against torch.autograd on a grid, including the tails."""
    u = np.linspace(-12, 12, 2001)
    ut = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    TF.silu(ut).sum().backward()
    assert np.abs(mo.silu_grad(u) - ut.grad.numpy()).max() <= 1e-14
    ut = torch.tensor(u, dtype=torch.float64, requires_grad=True)
    TF.gelu(ut, approximate="none").sum().backward()
    assert np.abs(mo.gelu_grad(u) - ut.grad.numpy()).max() <= 1e-14


# ----------------------------------------------------------------- fp8 weight-only experts

def check_e4m3_closed_forms():
    """OCP E4M3 values fixed by the format: 448 the largest finite, 2^-6 the
    smallest normal, 2^-9 the smallest subnormal, 1.0 = 0x38, S.1111.111 NaN;
    the 127 non-negative finite codes increase strictly with the code."""
    v = mo.e4m3_value(np.arange(256))
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x38] == 1.0
    assert v[0x07] == 7 * 2.0 ** -9 and v[0x3F] == 1.875 and v[0xB8] == -1.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF]) and np.isnan(v).sum() == 2
    assert np.all(np.diff(v[:127]) > 0)
    fin = ~np.isnan(v)
    assert np.array_equal(mo.e4m3_round(v[fin]), np.arange(256)[fin].astype(np.uint8))


def check_e4m3_ties_to_even():
    """A value halfway between two neighbouring codes takes the even one."""
    v = mo.e4m3_value(np.arange(127))
    mid = (v[:-1] + v[1:]) / 2
    got = mo.e4m3_round(mid.astype(np.float32))
    want = np.where(np.arange(126) % 2 == 0, np.arange(126), np.arange(1, 127))
    assert np.array_equal(got, want.astype(np.uint8)), np.nonzero(got != want)
    assert np.array_equal(mo.e4m3_round(-mid.astype(np.float32)), (want | 0x80).astype(np.uint8))


def check_e4m3_rounding_library():
    """Against torch's float8_e4m3fn cast (round to nearest even) on values of
    every binade, the subnormal range and exact midpoints, all within +-448."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(20000) * 40.0, rng.uniform(-2 ** -5, 2 ** -5, 20000),
                        np.exp2(rng.uniform(-12, 8.8, 20000)) * rng.choice([-1, 1], 20000)])
    v = mo.e4m3_value(np.arange(127))
    x = np.concatenate([x, (v[:-1] + v[1:]) / 2, v]).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mo.e4m3_round(x), lib)


def check_fp8_quantize_rows():
    """Per-row round trip: the row maximum lands on +-448 exactly, every element
    is within half a code step of the original, an all-zero row stays zero."""
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((40, 96)) * np.exp2(rng.uniform(-8, 4, (40, 1)))).astype(np.float32)
    w[3] = 0.0
    q, sc = mo.quantize_fp8_rows(w)
    assert q.dtype == np.uint8 and sc.dtype == np.float32
    amax = np.abs(w).max(axis=1)
    nz = amax > 0
    assert np.array_equal(sc[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    j = np.abs(w).argmax(axis=1)
    assert np.all(np.abs(mo.e4m3_value(q[np.arange(40), j]))[nz] == 448.0)
    deq = mo.dequantize_fp8_rows(q, sc)
    bound = np.maximum(2.0 ** -4 * np.abs(w), 2.0 ** -10 * sc[:, None].astype(np.float64)) * (1 + 1e-6)
    assert np.all(np.abs(deq - w) <= bound)
    assert np.all(q[3] == 0) and sc[3] == 1.0


def check_fp8_expert_is_dense_fp8_ffn():
    """One expert, k = 1: the layer with fp8 experts equals a dense SwiGLU FFN
    whose weights went through torch's own per-row fp8 round trip (fp32 scale
    amax / 448 and multiplier 448 / amax, float8_e4m3fn cast, back to fp64)."""
    cfg = MoEConfig(name="fp8_dense", n_tokens=9, d_model=64, n_experts=1, top_k=1, d_ff=96, act="swiglu",
                    gate_rule=GATE_TOPK_SOFTMAX, dtype="bf16", residual=False, seed=5)
    inp = make_inputs(cfg)
    _, out = mo.oracle_layer(cfg, inp, expert_weights="fp8")
    x = mo.to_f64(inp.x, "bf16")

    def rt(wb):
        w = torch.from_numpy(mo.to_f64(wb, "bf16").astype(np.float32))
        amax = w.abs().amax(dim=1, keepdim=True).double()
        # correctly rounded fp32 quotients (fp64 quotient rounded once to fp32)
        scale, inv = (amax / 448.0).float(), (448.0 / amax).float()
        return ((w * inv).to(torch.float8_e4m3fn).to(torch.float64) * scale.to(torch.float64)).numpy()
    e = inp.expert(0)
    w1, w3, w2 = rt(e["w1"]), rt(e["w3"]), rt(e["w2"])
    ref = (x @ w1.T) / (1 + np.exp(-(x @ w1.T))) * (x @ w3.T) @ w2.T
    assert np.abs(out - ref).max() <= 1e-12 * np.abs(ref).max()


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
