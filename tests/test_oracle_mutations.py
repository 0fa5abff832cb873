"""Plant plausible mistakes in the oracle (on the CPU) and show a pin catches each.

Every mutation replaces one oracle function with a subtly wrong variant; the
named checks must then fail.  This guards the pins themselves: a pin set that
still passed with a dropped term, a wrong sign or a swapped operand would not
be pinning anything.
"""
import numpy as np
import pytest

import oracle.moe_oracle as mo
import pin_checks as pc

_orig = {n: getattr(mo, n) for n in ("aux_loss_backward", "e4m3_round", "quantize_fp8_rows", "gate_backward", "silu_grad", "top_k_desc", "route", "ffn_swiglu", "ffn_gelu", "gelu", "dispatch",
                                       "aux_loss", "bias_step", "softmax_rows", "oracle_layer", "to_f64")}


def _ties_to_higher(key, k):
    E = key.shape[1]
    order = np.argsort(-key[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int64)


def _gates_from_biased_key(z, k, rule, sel_bias=None):
    if sel_bias is None or rule != mo.GATE_TOPK_SOFTMAX:
        return _orig["route"](z, k, rule, sel_bias)
    zb = z + np.asarray(sel_bias, np.float64)[None, :]
    idx, _, p = _orig["route"](z, k, rule, sel_bias)
    ch = np.take_along_axis(zb, idx, 1)
    ex = np.exp(ch - ch.max(1, keepdims=True))
    return idx, ex / ex.sum(1, keepdims=True), p


def _silu_on_w3(X, w1, w3, w2):
    return (mo.silu(X @ w3.T) * (X @ w1.T)) @ w2.T


def _gelu_tanh(u):
    return 0.5 * u * (1 + np.tanh(np.sqrt(2 / np.pi) * (u + 0.044715 * u ** 3)))


def _gelu_no_b2(X, w1, b1, w2, b2):
    return _orig["ffn_gelu"](X, w1, b1, w2, None)


def _keep_last(idx, E, C, *a):
    d = _orig["dispatch"](idx, E, None)
    if C is None:
        return d
    es = idx.reshape(-1)
    lists, drop = [], 0
    for e in range(E):
        s = np.nonzero(es == e)[0]
        if s.size > C:
            drop += s.size - C
            s = s[-C:] if C > 0 else s[:0]
        lists.append(s)
    perm = np.concatenate(lists)
    offs = np.zeros(E + 1, np.int64)
    offs[1:] = np.cumsum([len(s) for s in lists])
    sp = np.full(es.size, -1, np.int64)
    sp[perm] = np.arange(perm.size)
    return mo.Dispatch(d.counts, offs, perm, sp, drop, np.diff(offs))


def _descending_segments(idx, E, C, *a):
    d = _orig["dispatch"](idx, E, C, *a)
    perm = d.perm.copy()
    for e in range(E):
        perm[d.offsets[e]:d.offsets[e + 1]] = perm[d.offsets[e]:d.offsets[e + 1]][::-1]
    sp = np.full(d.slot_pos.size, -1, np.int64)
    sp[perm] = np.arange(perm.size)
    return mo.Dispatch(d.counts, d.offsets, perm, sp, d.drop_count, d.kept)


def _choice_as_slot(idx, E, C, layout="packed", priority="slot"):
    return _orig["dispatch"](idx, E, C, layout, "slot")


def _gate_backward_no_centering(rule, z, idx, gates, p, dg):
    if rule != "topk_softmax":
        return _orig["gate_backward"](rule, z, idx, gates, p, dg)
    dz = np.zeros(z.shape)
    np.put_along_axis(dz, idx, gates * dg, axis=1)          # drops the -<g, dg> term
    return dz


def _aux_backward_subset_n(counts, p, k, d_aux, n_tokens=None):
    return _orig["aux_loss_backward"](counts, p, k, d_aux)     # takes N from the rows it was given


def _silu_grad_sigmoid_only(u):
    return 1.0 / (1.0 + np.exp(-u))


def _aux_post_drop(counts, p, k):
    N, E = p.shape
    C = max(1, N // (4 * E))
    return _orig["aux_loss"](np.minimum(counts, C), p, k)


def _bias_sign_flipped(counts, b, gamma, N, k):
    s, nb = _orig["bias_step"](counts, b, gamma, N, k)
    return s, np.asarray(b, np.float32).astype(np.float64) + float(np.float32(gamma)) * s


def _softmax_no_max(z):
    ez = np.exp(z)
    return ez / ez.sum(1, keepdims=True)


def _layer_no_residual(cfg, inputs, *a, **kw):
    import dataclasses
    return _orig["oracle_layer"](dataclasses.replace(cfg, residual=False), inputs, *a, **kw)


def _e4m3_ties_away(x):
    xa = np.asarray(x, dtype=np.float64)
    c = _orig["e4m3_round"](xa)
    v = mo.e4m3_value(np.arange(127))
    mid = np.isin(np.abs(xa), (v[:-1] + v[1:]) / 2)
    up = np.searchsorted(v, np.abs(xa)).clip(0, 126)
    return np.where(mid, up | np.where(np.signbit(xa), 0x80, 0), c).astype(np.uint8)


def _quantize_fnuz_max(w):
    q, sc = _orig["quantize_fp8_rows"](np.asarray(w, dtype=np.float32) * np.float32(240.0 / 448.0))
    return q, (sc * np.float32(448.0 / 240.0)).astype(np.float32)


def _bf16_shift15(a, dtype):
    if dtype != "bf16":
        return _orig["to_f64"](a, dtype)
    bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    with np.errstate(invalid="ignore"):
        return bits.view(np.float32).astype(np.float64)


def _rows_off_by_one(cfg, inputs, logits_override=None, rows=None, **kw):
    if rows is not None:
        rows = np.minimum(np.asarray(rows, dtype=np.int64) + 1, cfg.n_tokens - 1)
    return _orig["oracle_layer"](cfg, inputs, logits_override, rows=rows, **kw)


def _shared_gated(cfg, inputs, logits_override=None, rows=None, **kw):
    """The shared expert scaled by the token's kept gate mass (1 unless slots were dropped)."""
    r, out = _orig["oracle_layer"](cfg, inputs, logits_override, rows=rows, **kw)
    if cfg.d_ff_shared:
        sel = np.arange(cfg.n_tokens) if rows is None else np.asarray(rows)
        x = mo.to_f64(inputs.x, cfg.dtype)[sel]
        sh = mo.ffn_swiglu(x, mo.to_f64(inputs.sh_w1, cfg.dtype), mo.to_f64(inputs.sh_w3, cfg.dtype),
                           mo.to_f64(inputs.sh_w2, cfg.dtype))
        kept = (r.disp.slot_pos.reshape(cfg.n_tokens, cfg.top_k) >= 0)[sel]
        mass = (r.gates[sel] * kept).sum(axis=1, keepdims=True)
        out = out - sh + mass * sh
    return r, out


MUTATIONS = [
    ("to_f64", _bf16_shift15, [pc.check_bf16_decode_library]),
    ("oracle_layer", _rows_off_by_one, [pc.check_rows_path]),
    ("oracle_layer", _shared_gated, [pc.check_shared_expert_term]),
    ("gate_backward", _gate_backward_no_centering, [pc.check_backward_autograd]),
    ("aux_loss_backward", _aux_backward_subset_n, [pc.check_sampled_backward_autograd]),
    ("silu_grad", _silu_grad_sigmoid_only, [pc.check_activation_grads_library, pc.check_backward_autograd]),
    ("e4m3_round", _e4m3_ties_away, [pc.check_e4m3_ties_to_even, pc.check_e4m3_rounding_library]),
    ("quantize_fp8_rows", _quantize_fnuz_max, [pc.check_fp8_quantize_rows]),
    ("top_k_desc", _ties_to_higher, [pc.check_topk_brute_force]),
    ("route", _gates_from_biased_key, [pc.check_bias_moves_selection_not_gates]),
    ("ffn_swiglu", _silu_on_w3, [pc.check_single_expert_is_dense, pc.check_identical_experts_are_dense]),
    ("gelu", _gelu_tanh, [pc.check_activation_library, pc.check_single_expert_is_dense]),
    ("ffn_gelu", _gelu_no_b2, [pc.check_single_expert_is_dense, pc.check_printed_example_output]),
    ("dispatch", _keep_last, [pc.check_capacity_brute_force]),
    ("dispatch", _descending_segments, [pc.check_dispatch_invariants]),
    ("dispatch", _choice_as_slot, [pc.check_capacity_choice_priority_brute_force]),
    ("aux_loss", _aux_post_drop, [pc.check_aux_uniform_is_one]),
    ("bias_step", _bias_sign_flipped, [pc.check_bias_step_signs, pc.check_bias_loop_equalises]),
    ("softmax_rows", _softmax_no_max, [pc.check_softmax_library]),
    ("oracle_layer", _layer_no_residual, [pc.check_single_expert_is_dense, pc.check_dropped_tokens_pass_residual]),
]


@pytest.mark.parametrize("name,fn,checks", MUTATIONS, ids=[f"{m[0]}:{m[1].__name__}" for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, fn, checks):
    monkeypatch.setattr(mo, name, fn)
    if name == "oracle_layer":
        monkeypatch.setattr(pc.mo, name, fn)
    for check in checks:
        with pytest.raises((AssertionError, FloatingPointError, ValueError)):
            check()
