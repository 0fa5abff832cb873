"""fp64 CPU oracle of one sparse Mixture-of-Experts FFN layer (forward pass).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this module.  It is the slow, obviously correct statement
of what the layer computes, and it shares no code with the HIP library.

Every value is computed in float64 from the exact values of the stored inputs
(fp32, or bfloat16 bit patterns).  A numpy matmul (BLAS dgemm), a stable sort
and ``scipy.special.erfc`` are the only library steps.

Sources (the pages describing the method; cited by title and section):

[L] "Mixture of Experts (MoE)", AI Engineering from Scratch, Phase 07 lesson 11
    (aiengineeringfromscratch.com): sections "Concept / FFN swap", "The load
    balance problem", "Shared experts", "Build it / Step 1: the router",
    "Step 2: run 100 tokens through the router", "Key terms".
[N] "MoE architecture: load balancing and gating implementation" (nextadmin.net):
    the same lesson, cleaner text: "Load balancing" items 1-3, "Shared experts".
[G] "Mixture of Experts (MoE)" glossary (ultralytics.com): "How an MoE layer
    works", "Load balancing and expert capacity" (seeded top-2 example and its
    printed output).
[X] "Expert Parallelism for MoE Serving" (aiunderstanding.org): "Deep dive",
    "Technical insight" (dispatch groups tokens by expert; capacity).
[S] "How sparse models scale" (ircnf.com): the part on running large MoE
    models, where quantised weights are the remedy for their memory size.

Readings taken where the pages leave a step open (each is also listed in the
design notes):

* top-k order: descending key, exact ties to the lower expert index ([L] Step 1
  sorts the experts with a stable sort on the negated key);
* softmax subtracts the row maximum before exponentiating ([L] Step 1);
* SwiGLU expert: ``(SiLU(X W1^T) * (X W3^T)) W2^T``, SiLU on W1, no biases;
* GELU expert: ``GELU(X W1^T + b1) W2^T + b2`` with the exact erf GELU;
* capacity ``C = floor(cf * N / E)``; each expert keeps its first C slots in
  ascending slot id ``s = t*k + j`` (or, as a variant, in choice order: all
  first choices by token, then second choices, ...); a dropped slot
  contributes nothing and the kept gates of that token are not renormalised;
  the kept rows are packed back to back or placed in fixed [E, C] buffers;
* dropped tokens still receive the residual (and the shared expert, if any);
* auxiliary loss ``E * sum_e f_e * P_e`` with ``f_e = counts_e / (N k)`` from
  the pre-drop counts and ``P_e`` the full-softmax probability averaged over
  all N tokens;
* bias step ``b_e <- b_e - gamma * sign(counts_e * E - N k)``, sign(0) = 0,
  applied after the forward pass (it feeds the next call only);
* fp8 weight-only experts ([S]; the pages name 8-bit weights, no format): OCP
  E4M3 codes, round to nearest with ties to even, saturating at 448, one fp32
  scale per output row (amax / 448), activations and accumulation unchanged.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.special import erfc

GATE_TOPK_SOFTMAX = "topk_softmax"
GATE_SOFTMAX_RENORM = "softmax_renorm"
GATE_SWITCH_TOP1 = "switch_top1"


# --------------------------------------------------------------------------- inputs

def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored fp32 values or bfloat16 bit patterns."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --------------------------------------------------------------------------- router

def router_logits(x: np.ndarray, w_router: np.ndarray, logit_bias=None) -> np.ndarray:
    """z[t, e] = x[t] . W_r[e] (+ a fixed per-expert logit offset).

    [L] "Build it / Step 1: the router": each expert's score is the dot product
    of the hidden vector with that expert's router row; [G] "How an MoE layer
    works": the router is one linear layer scoring every expert for every token.
    """
    z = x @ w_router.T
    if logit_bias is not None:
        z = z + np.asarray(logit_bias, dtype=np.float64)[None, :]
    return z


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row softmax with the row maximum subtracted first ([L] Step 1)."""
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def top_k_desc(key: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k column indices with the largest key, largest first,
    exact ties to the lower index: a full stable sort on the negated key
    ([L] Step 1 sorts all experts this way and keeps the first k)."""
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :k].astype(np.int64)


def route(z: np.ndarray, k: int, rule: str, sel_bias=None):
    """Selection and gate weights for every token.

    Returns ``(idx [N,k], gates [N,k], p [N,E])`` where ``p`` is the softmax
    over all E raw logits (used by the auxiliary loss).

    * ``topk_softmax`` ([L] Step 1; [G] example): key = z + selection bias;
      gate = softmax over the *raw* logits of the k selected experts.
    * ``softmax_renorm`` ([L] "The load balance problem", DeepSeek-V3 approach;
      [N] Load balancing item 3): p = softmax(z); key = p + bias; gate = p of
      the selected experts renormalised to sum 1.  The bias moves selection
      only; gates use the raw scores.
    * ``switch_top1`` ([G] "Load balancing and expert capacity": Switch sends
      each token to one expert): the argmax of z (ties to the lower index);
      gate = its full-softmax probability, not renormalised.
    """
    N, E = z.shape
    b = np.zeros(E) if sel_bias is None else np.asarray(sel_bias, dtype=np.float32).astype(np.float64)
    p = softmax_rows(z)
    if rule == GATE_TOPK_SOFTMAX:
        idx = top_k_desc(z + b[None, :], k)
        chosen = np.take_along_axis(z, idx, axis=1)
        m = chosen.max(axis=1, keepdims=True)
        ex = np.exp(chosen - m)
        gates = ex / ex.sum(axis=1, keepdims=True)
    elif rule == GATE_SOFTMAX_RENORM:
        idx = top_k_desc(p + b[None, :], k)
        ps = np.take_along_axis(p, idx, axis=1)
        gates = ps / ps.sum(axis=1, keepdims=True)
    elif rule == GATE_SWITCH_TOP1:
        if k != 1:
            raise ValueError("switch_top1 routes each token to exactly one expert")
        idx = top_k_desc(z, 1)
        gates = np.take_along_axis(p, idx, axis=1)
    else:
        raise ValueError(rule)
    return idx, gates, p


def selection_gap(z: np.ndarray, k: int, rule: str, sel_bias=None) -> np.ndarray:
    """Per token, key[k-th chosen] - key[(k+1)-th]: how far the selection is
    from a tie (inf when k == E).  Used to report near-ties."""
    N, E = z.shape
    if k >= E:
        return np.full(N, np.inf)
    b = np.zeros(E) if sel_bias is None else np.asarray(sel_bias, dtype=np.float32).astype(np.float64)
    if rule == GATE_TOPK_SOFTMAX:
        key = z + b[None, :]
    elif rule == GATE_SOFTMAX_RENORM:
        key = softmax_rows(z) + b[None, :]
    else:
        key = z
    s = -np.sort(-key, axis=1)
    return s[:, k - 1] - s[:, k]


# --------------------------------------------------------------------------- dispatch

@dataclass
class Dispatch:
    counts: np.ndarray      # [E] pre-drop tokens per expert (sum = N k)
    offsets: np.ndarray     # [E+1] start row of each expert's segment (packed: scan of kept counts; padded: e*C)
    perm: np.ndarray        # slot id s = t*k + j per row, grouped by expert (padded: -1 on padding rows)
    slot_pos: np.ndarray    # [N k] row of slot s, -1 if dropped
    drop_count: int
    kept: np.ndarray        # [E] kept slots per expert, min(counts, C)


def dispatch(idx: np.ndarray, n_experts: int, capacity: int | None, layout: str = "packed",
             priority: str = "slot") -> Dispatch:
    """Group the N*k slots by expert ([G] example: per expert, the tokens that
    chose it; [X] "Deep dive": tokens are sent to the holder of their expert).

    Within an expert, slots are ordered by priority: ascending slot id
    s = t*k + j ("slot"), or by choice rank first and token second
    ("choice": every token's first choice before any second choice).  With a
    capacity C ([N] Load balancing item 2: each expert takes at most C * N / E
    tokens; the overflow skips the experts), only the first C slots of each
    expert in that order are kept.

    Layout ([X] "Technical insight": fixed per-expert buffers, padded or
    dropped to a uniform shape): "packed" puts the experts' kept rows back to
    back; "padded" gives expert e rows [e*C, (e+1)*C), kept rows first and
    padding rows (perm = -1) after them.
    """
    expert_of_slot = idx.reshape(-1)
    n_slots = expert_of_slot.size
    k = idx.shape[1] if idx.ndim == 2 else 1
    counts = np.zeros(n_experts, dtype=np.int64)
    kept_lists = []
    drop = 0
    for e in range(n_experts):
        slots = np.nonzero(expert_of_slot == e)[0]          # ascending slot id
        if priority == "choice":
            slots = slots[np.lexsort((slots // k, slots % k))]   # by choice j, then token t
        elif priority != "slot":
            raise ValueError(priority)
        counts[e] = slots.size
        if capacity is not None and slots.size > capacity:
            drop += slots.size - capacity
            slots = slots[:capacity]
        kept_lists.append(slots)
    kept = np.array([len(s) for s in kept_lists], dtype=np.int64)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    if layout == "packed":
        offsets[1:] = np.cumsum(kept)
        perm = np.concatenate(kept_lists) if kept_lists else np.zeros(0, np.int64)
    elif layout == "padded":
        if capacity is None:
            raise ValueError("the padded layout needs a finite capacity")
        offsets = np.arange(n_experts + 1, dtype=np.int64) * capacity
        perm = np.full(n_experts * capacity, -1, dtype=np.int64)
        for e, sl in enumerate(kept_lists):
            perm[e * capacity:e * capacity + sl.size] = sl
    else:
        raise ValueError(layout)
    slot_pos = np.full(n_slots, -1, dtype=np.int64)
    rows = np.nonzero(perm >= 0)[0]
    slot_pos[perm[rows]] = rows
    return Dispatch(counts=counts, offsets=offsets, perm=perm.astype(np.int64),
                    slot_pos=slot_pos, drop_count=int(drop), kept=kept)


# --------------------------------------------------------------------------- experts

def silu(u: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def gelu(u: np.ndarray) -> np.ndarray:
    """Exact (erf) GELU, the form torch.nn.GELU() uses by default ([G] example):
    u * Phi(u) with Phi(u) = (1 + erf(u/sqrt 2))/2, written as erfc(-u/sqrt 2)/2
    so the negative tail keeps its relative precision."""
    return u * 0.5 * erfc(-u / math.sqrt(2.0))


def ffn_swiglu(X: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """SwiGLU feed-forward ([L] "FFN swap": each expert is usually a SwiGLU FFN)."""
    return (silu(X @ w1.T) * (X @ w3.T)) @ w2.T


def ffn_gelu(X: np.ndarray, w1: np.ndarray, b1, w2: np.ndarray, b2) -> np.ndarray:
    """Linear -> GELU -> Linear expert ([G] example's expert form)."""
    h = X @ w1.T
    if b1 is not None:
        h = h + b1[None, :]
    y = gelu(h) @ w2.T
    if b2 is not None:
        y = y + b2[None, :]
    return y


def expert_apply(act: str, X: np.ndarray, w: dict) -> np.ndarray:
    if act == "swiglu":
        return ffn_swiglu(X, w["w1"], w["w3"], w["w2"])
    if act == "gelu":
        return ffn_gelu(X, w["w1"], w.get("b1"), w["w2"], w.get("b2"))
    raise ValueError(act)


# --------------------------------------------------------------------------- balancing

def aux_loss(counts: np.ndarray, p: np.ndarray, k: int) -> float:
    """E * sum_e f_e * P_e: f_e = counts_e / (N k) (pre-drop), P_e = mean_t p[t,e].

    [G] "Load balancing and expert capacity": Switch adds a loss term that is
    smallest when tokens and router probabilities are spread evenly; [N] item 1.
    """
    N, E = p.shape
    f = counts.astype(np.float64) / float(N * k)
    P = p.sum(axis=0) / float(N)
    return float(E * np.sum(f * P))


def bias_step(counts: np.ndarray, sel_bias: np.ndarray, gamma: float, n_tokens: int, k: int):
    """Aux-loss-free balancing ([L] "The load balance problem", DeepSeek-V3
    approach; [L] Step 2): after a step, each expert whose load is above the
    target N k / E moves its selection bias down by gamma, one below it moves
    it up.  Returns (signs [E] int, updated bias [E] float64)."""
    E = counts.size
    diff = counts.astype(np.int64) * E - int(n_tokens) * int(k)   # load - target, times E
    signs = np.sign(diff).astype(np.int64)
    b = np.asarray(sel_bias, dtype=np.float32).astype(np.float64)
    g = float(np.float32(gamma))
    return signs, b - g * signs


# --------------------------------------------------------------------------- layer

@dataclass
class RouteResult:
    logits: np.ndarray
    topk_idx: np.ndarray
    gates: np.ndarray
    probs: np.ndarray
    disp: Dispatch
    aux: float | None
    signs: np.ndarray | None
    new_bias: np.ndarray | None
    min_gap: float


def oracle_route(cfg, logits: np.ndarray, sel_bias=None) -> RouteResult:
    """Everything the layer decides from the logits: selection, gates,
    counts, permutation, capacity, aux loss and the bias step."""
    z = np.asarray(logits, dtype=np.float64)
    idx, gates, p = route(z, cfg.top_k, cfg.gate_rule, sel_bias)
    d = dispatch(idx, cfg.n_experts, cfg.capacity, getattr(cfg, "capacity_layout", "packed"),
                 getattr(cfg, "capacity_priority", "slot"))
    aux = aux_loss(d.counts, p, cfg.top_k) if cfg.aux_loss else None
    signs = new_bias = None
    if cfg.gamma > 0:
        b = sel_bias if sel_bias is not None else np.zeros(cfg.n_experts, np.float32)
        signs, new_bias = bias_step(d.counts, b, cfg.gamma, cfg.n_tokens, cfg.top_k)
    gap = selection_gap(z, cfg.top_k, cfg.gate_rule, sel_bias)
    return RouteResult(logits=z, topk_idx=idx, gates=gates, probs=p, disp=d, aux=aux,
                       signs=signs, new_bias=new_bias, min_gap=float(gap.min()) if gap.size else math.inf)


def oracle_layer(cfg, inputs, logits_override=None, rows=None, sel_bias="inputs", expert_weights="stored",
                 progress=None):
    """The whole forward pass in fp64.

    ``inputs`` is a :class:`workloads.LayerInputs`.  ``logits_override`` replaces
    the router product (parity hook: the GPU's fp32 logits decide routing on
    both sides).  ``rows`` restricts the expert work and the output to those
    tokens (routing, counts and capacity still cover all N).
    ``expert_weights="fp8"`` runs the routed experts on their fp8 round trip
    (``fp8_expert_weights``); the router and the shared expert keep the stored
    weights.  ``progress(e)``, if given, is called after each expert's rows are
    done (long full-size runs report with it; it takes no part in the result).

    [L] "Concept / FFN swap": h + sum over the chosen experts of gate * expert(h);
    [G] example: out[tokens of e] += weight * expert_e(tokens of e) for each e;
    [L] "Shared experts": every token also passes through the shared expert.
    """
    dt = cfg.dtype
    N, E, k = cfg.n_tokens, cfg.n_experts, cfg.top_k
    x = to_f64(inputs.x, dt)
    if logits_override is None:
        z = router_logits(x, to_f64(inputs.w_router, dt), inputs.logit_bias)
    else:
        z = np.asarray(logits_override, dtype=np.float32).astype(np.float64)
    sb = inputs.sel_bias if isinstance(sel_bias, str) else sel_bias
    r = oracle_route(cfg, z, sb)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    want = np.zeros(N, dtype=bool)
    want[rows] = True

    d_model = cfg.d_model
    y_slot = {}
    expert_of_slot = r.topk_idx.reshape(-1)
    for e in range(E):
        lo, hi = r.disp.offsets[e], r.disp.offsets[e + 1]
        slots = r.disp.perm[lo:hi]
        slots = slots[slots >= 0]                       # padded layout: skip padding rows
        slots = slots[want[slots // k]]
        if slots.size == 0:
            continue
        assert np.all(expert_of_slot[slots] == e)
        w = {n: to_f64(v, dt) for n, v in inputs.expert(e).items()}
        if expert_weights == "fp8":
            w = fp8_expert_weights(w)
        Y = expert_apply(cfg.act, x[slots // k], w)
        for s, yrow in zip(slots, Y):
            y_slot[int(s)] = yrow
        if progress is not None:
            progress(e)

    out = np.zeros((rows.size, d_model))
    if cfg.residual:
        out += x[rows]
    if cfg.d_ff_shared > 0:
        sw = {"w1": to_f64(inputs.sh_w1, dt), "w3": to_f64(inputs.sh_w3, dt), "w2": to_f64(inputs.sh_w2, dt)}
        out += ffn_swiglu(x[rows], sw["w1"], sw["w3"], sw["w2"])
    for i, t in enumerate(rows):
        for j in range(k):
            s = int(t) * k + j
            if r.disp.slot_pos[s] >= 0:
                out[i] += r.gates[t, j] * y_slot[s]
    return r, out


# --------------------------------------------------------------------------- fp8 weight-only experts

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent field 0 holds subnormals m/8 * 2^-6; S.1111.111 is NaN)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return s * mag


_E4M3_POS = e4m3_value(np.arange(127))          # codes 0..126: every non-negative finite value, ascending


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 code to each value (compared exactly in fp64), an exact tie
    going to the code with an even mantissa; magnitudes above 448 saturate to
    448.  The sign bit follows the sign of x (so -0.0 and negative values that
    round to zero give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 126)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _E4M3_POS[lo], _E4M3_POS[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def quantize_fp8_rows(w) -> tuple[np.ndarray, np.ndarray]:
    """Round-to-nearest fp8 weights with one scale per output row (a row of a
    weight stored [out, in]).  In fp32, as the kernel computes it:
    amax = max |w|, scale = amax / 448, inv = 448 / amax (scale = inv = 1 for
    an all-zero row), code = e4m3_round(w * inv)."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    scale = np.where(zero, np.float32(1), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1), np.float32(E4M3_MAX) / safe).astype(np.float32)
    codes = e4m3_round((w * inv[:, None]).astype(np.float32))
    return codes, scale


def dequantize_fp8_rows(codes, scales) -> np.ndarray:
    """fp64 weights the fp8 experts compute with: value(code) * row scale (exact)."""
    return e4m3_value(codes) * np.asarray(scales, dtype=np.float64)[:, None]


def fp8_expert_weights(w: dict) -> dict:
    """An expert's weight dict with every matrix replaced by its fp8 round trip
    (biases unchanged).  Input matrices are the exact fp64 values of bf16/fp32
    storage, hence exactly representable in fp32."""
    out = {}
    for n, v in w.items():
        if n.startswith("b"):
            out[n] = v
        else:
            q, sc = quantize_fp8_rows(np.asarray(v, dtype=np.float32))
            out[n] = dequantize_fp8_rows(q, sc)
    return out


# --------------------------------------------------------------------------- backward

def silu_grad(u: np.ndarray) -> np.ndarray:
    """d/du u*sigmoid(u) = sigmoid(u) * (1 + u * (1 - sigmoid(u)))."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * (1.0 - s))


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d/du u*Phi(u) = Phi(u) + u*phi(u) (exact erf GELU)."""
    return 0.5 * erfc(-u / math.sqrt(2.0)) + u * np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)


def softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """Row softmax Jacobian-vector product: dz = p * (dp - <p, dp>)."""
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def gate_backward(rule: str, z: np.ndarray, idx: np.ndarray, gates: np.ndarray, p: np.ndarray,
                  dg: np.ndarray) -> np.ndarray:
    """dL/dz from dL/dgates; the selection itself is piecewise constant in z.

    rule A (gate = softmax of the selected raw logits): dz_S = g * (dg - <g, dg>);
    rule B (gate = p_S / sum p_S, p = softmax(z)): dp_S = (dg - <g, dg>) / sum p_S,
    then the full softmax Jacobian; rule C (gate = p of the argmax): dp = dg at
    the argmax, then the softmax Jacobian."""
    N, E = z.shape
    dz = np.zeros((N, E))
    if rule == GATE_TOPK_SOFTMAX:
        dzs = gates * (dg - np.sum(gates * dg, axis=1, keepdims=True))
        np.put_along_axis(dz, idx, dzs, axis=1)
    elif rule == GATE_SOFTMAX_RENORM:
        ps = np.take_along_axis(p, idx, axis=1)
        dps = (dg - np.sum(gates * dg, axis=1, keepdims=True)) / ps.sum(axis=1, keepdims=True)
        dp = np.zeros((N, E))
        np.put_along_axis(dp, idx, dps, axis=1)
        dz = softmax_backward(p, dp)
    elif rule == GATE_SWITCH_TOP1:
        dp = np.zeros((N, E))
        np.put_along_axis(dp, idx, dg, axis=1)
        dz = softmax_backward(p, dp)
    else:
        raise ValueError(rule)
    return dz


def aux_loss_backward(counts: np.ndarray, p: np.ndarray, k: int, d_aux: float, n_tokens=None) -> np.ndarray:
    """dL/dz of d_aux * E * sum_e f_e P_e: f (from the discrete counts) is constant,
    dP_e/dp[t,e] = 1/N, then the softmax Jacobian.  ``p`` may hold a subset of
    the N tokens' rows when ``n_tokens`` gives N."""
    N, E = p.shape
    N = N if n_tokens is None else int(n_tokens)
    f = counts.astype(np.float64) / float(N * k)
    dp = np.broadcast_to(d_aux * E * f / float(N), p.shape)
    return softmax_backward(p, dp)


def expert_backward(act: str, X: np.ndarray, w: dict, dY: np.ndarray, weights: bool = True) -> dict:
    """Gradients of one expert FFN on its rows X given dL/dY: dX and (unless
    ``weights`` is False) the weight and bias gradients.  SwiGLU: H = SiLU(A1)
    * A3, A1 = X W1^T, A3 = X W3^T, Y = H W2^T.  GELU: H = GELU(A), A = X W1^T
    + b1, Y = H W2^T + b2."""
    g = {}
    if act == "swiglu":
        A1, A3 = X @ w["w1"].T, X @ w["w3"].T
        H = silu(A1) * A3
        dH = dY @ w["w2"]
        dA1 = dH * A3 * silu_grad(A1)
        dA3 = dH * silu(A1)
        g["x"] = dA1 @ w["w1"] + dA3 @ w["w3"]
        if not weights:
            return g
        g["w2"] = dY.T @ H
        g["w1"] = dA1.T @ X
        g["w3"] = dA3.T @ X
    elif act == "gelu":
        A = X @ w["w1"].T
        if w.get("b1") is not None:
            A = A + w["b1"][None, :]
        H = gelu(A)
        dH = dY @ w["w2"]
        dA = dH * gelu_grad(A)
        g["x"] = dA @ w["w1"]
        if not weights:
            return g
        g["w2"] = dY.T @ H
        g["w1"] = dA.T @ X
        if w.get("b1") is not None:
            g["b1"] = dA.sum(axis=0)
        if w.get("b2") is not None:
            g["b2"] = dY.sum(axis=0)
    else:
        raise ValueError(act)
    return g


def oracle_layer_backward(cfg, inputs, dout, d_aux: float = 0.0, logits_override=None,
                          expert_weights="stored") -> dict:
    """Gradients of the layer's forward pass (``oracle_layer``) in fp64, for an
    upstream gradient ``dout`` [N, d] of ``out`` and ``d_aux`` of the aux loss.

    The routing decisions (selection, capacity) are taken as fixed, since they
    are piecewise constant in the inputs; gradients flow through the gate
    weights into the logits and the router, through the kept slots' expert
    FFNs, the shared expert and the residual ([L] "The load balance problem":
    the auxiliary loss is a second gradient signal into the router).

    Returns dx [N, d], w_router [E, d], logit_bias [E], w1/w3 [E, F, d],
    w2 [E, d, F], b1 [E, F] / b2 [E, d] (GELU with biases), sh_w1/sh_w3
    [Fs, d] and sh_w2 [d, Fs] (with a shared expert)."""
    dt = cfg.dtype
    N, E, k, d, F = cfg.n_tokens, cfg.n_experts, cfg.top_k, cfg.d_model, cfg.d_ff
    x = to_f64(inputs.x, dt)
    wr = to_f64(inputs.w_router, dt)
    z = router_logits(x, wr, inputs.logit_bias) if logits_override is None else \
        np.asarray(logits_override, dtype=np.float32).astype(np.float64)
    r = oracle_route(cfg, z, inputs.sel_bias)
    dout = np.asarray(dout, dtype=np.float64)
    grads = {"x": np.zeros((N, d)), "w1": np.zeros((E, F, d)), "w2": np.zeros((E, d, F))}
    if cfg.act == "swiglu":
        grads["w3"] = np.zeros((E, F, d))
    if cfg.ffn_bias:
        grads["b1"] = np.zeros((E, F))
        grads["b2"] = np.zeros((E, d))
    if cfg.residual:
        grads["x"] += dout
    dg = np.zeros((N, k))
    for e in range(E):
        lo, hi = r.disp.offsets[e], r.disp.offsets[e + 1]
        slots = r.disp.perm[lo:hi]
        slots = slots[slots >= 0]
        if slots.size == 0:
            continue
        w = {n: to_f64(v, dt) for n, v in inputs.expert(e).items()}
        if expert_weights == "fp8":
            w = fp8_expert_weights(w)
        t, j = slots // k, slots % k
        X = x[t]
        Y = expert_apply(cfg.act, X, w)
        dg[t, j] = np.sum(dout[t] * Y, axis=1)
        dY = r.gates[t, j][:, None] * dout[t]
        g = expert_backward(cfg.act, X, w, dY)
        np.add.at(grads["x"], t, g["x"])
        for n in ("w1", "w3", "w2", "b1", "b2"):
            if n in g:
                grads[n][e] += g[n]
    dz = gate_backward(cfg.gate_rule, z, r.topk_idx, r.gates, r.probs, dg)
    if cfg.aux_loss and d_aux != 0.0:
        dz = dz + aux_loss_backward(r.disp.counts, r.probs, k, d_aux)
    grads["logits"] = dz
    grads["w_router"] = dz.T @ x
    grads["logit_bias"] = dz.sum(axis=0)
    grads["x"] += dz @ wr
    if cfg.d_ff_shared > 0:
        sw = {"w1": to_f64(inputs.sh_w1, dt), "w3": to_f64(inputs.sh_w3, dt), "w2": to_f64(inputs.sh_w2, dt)}
        g = expert_backward("swiglu", x, sw, dout)
        grads["x"] += g["x"]
        grads["sh_w1"], grads["sh_w3"], grads["sh_w2"] = g["w1"], g["w3"], g["w2"]
    grads["gates"] = dg
    return grads


# --------------------------------------------------------------------------- sampled backward (full sizes)

def oracle_backward_rows(cfg, inputs, dout, rows, d_aux: float = 0.0, logits_override=None) -> dict:
    """The per-token part of ``oracle_layer_backward`` for the tokens ``rows``
    only: dx [rows, d], the gate gradients [rows, k] and dL/dlogits [rows, E].

    Each of these rows depends on its own token alone once routing is fixed
    (the aux-loss gradient only through the batch counts): the token's kept
    experts give dgates and their input gradient, the gate rule maps dgates
    to dlogits, the router adds dz W_router, plus the shared expert and the
    residual.  Routing, counts and capacity still cover all N tokens."""
    dt = cfg.dtype
    N, k = cfg.n_tokens, cfg.top_k
    rows = np.asarray(rows, dtype=np.int64)
    x = to_f64(inputs.x, dt)
    wr = to_f64(inputs.w_router, dt)
    z = router_logits(x, wr, inputs.logit_bias) if logits_override is None else \
        np.asarray(logits_override, dtype=np.float32).astype(np.float64)
    r = oracle_route(cfg, z, inputs.sel_bias)
    xr = x[rows]
    dr = np.asarray(dout, dtype=np.float64)[rows]
    dx = dr.copy() if cfg.residual else np.zeros_like(xr)
    dg = np.zeros((rows.size, k))
    chosen = r.topk_idx[rows]
    kept = r.disp.slot_pos[rows[:, None] * k + np.arange(k)[None, :]] >= 0
    for e in np.unique(chosen[kept]):
        ii, jj = np.nonzero(kept & (chosen == e))
        w = {n: to_f64(v, dt) for n, v in inputs.expert(int(e)).items()}
        dg[ii, jj] = np.sum(dr[ii] * expert_apply(cfg.act, xr[ii], w), axis=1)
        dY = r.gates[rows[ii], jj][:, None] * dr[ii]
        np.add.at(dx, ii, expert_backward(cfg.act, xr[ii], w, dY, weights=False)["x"])
    dz = gate_backward(cfg.gate_rule, z[rows], chosen, r.gates[rows], r.probs[rows], dg)
    if cfg.aux_loss and d_aux != 0.0:
        dz = dz + aux_loss_backward(r.disp.counts, r.probs[rows], k, d_aux, n_tokens=N)
    dx += dz @ wr
    if cfg.d_ff_shared > 0:
        sw = {"w1": to_f64(inputs.sh_w1, dt), "w3": to_f64(inputs.sh_w3, dt), "w2": to_f64(inputs.sh_w2, dt)}
        dx += expert_backward("swiglu", xr, sw, dr, weights=False)["x"]
    return {"x": dx, "gates": dg, "logits": dz, "route": r}


def _hidden_subset(w: dict, cols, dt: str) -> dict:
    cols = np.asarray(cols, dtype=np.int64)
    sub = {"w1": to_f64(w["w1"][cols], dt), "w2": to_f64(w["w2"][:, cols], dt)}
    if w.get("w3") is not None:
        sub["w3"] = to_f64(w["w3"][cols], dt)
    if w.get("b1") is not None:
        sub["b1"] = to_f64(w["b1"][cols], dt)
        sub["b2"] = to_f64(w["b2"], dt)
    return sub


def oracle_expert_grad_columns(cfg, inputs, dout, e: int, cols, route: RouteResult) -> dict:
    """Weight gradients of routed expert ``e`` restricted to its hidden units
    ``cols``: w1 / w3 [cols, d], w2 [d, cols], b1 [cols], and b2 [d].

    The activation acts on each hidden unit alone, so these entries are the
    weight gradients of the smaller FFN that keeps only the units ``cols``,
    fed the same rows (every kept slot of e) and the same dL/dY = gate * dout."""
    k = cfg.top_k
    lo, hi = route.disp.offsets[e], route.disp.offsets[e + 1]
    slots = route.disp.perm[lo:hi]
    slots = slots[slots >= 0]
    t, j = slots // k, slots % k
    X = to_f64(inputs.x[t], cfg.dtype)
    dY = route.gates[t, j][:, None] * np.asarray(dout, dtype=np.float64)[t]
    g = expert_backward(cfg.act, X, _hidden_subset(inputs.expert(e), cols, cfg.dtype), dY)
    g.pop("x")
    return g


def oracle_shared_grad_columns(cfg, inputs, dout, cols) -> dict:
    """Shared-expert weight gradients restricted to its hidden units ``cols``
    (the same argument as ``oracle_expert_grad_columns``; every token's row)."""
    w = {"w1": inputs.sh_w1, "w3": inputs.sh_w3, "w2": inputs.sh_w2}
    g = expert_backward("swiglu", to_f64(inputs.x, cfg.dtype), _hidden_subset(w, cols, cfg.dtype),
                        np.asarray(dout, dtype=np.float64))
    g.pop("x")
    return g
