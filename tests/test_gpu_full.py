"""GPU parity at the workloads' full sizes, in the configuration bench.py
times: routing, dispatch, aux and bias step compared bit-exactly (integers)
or to tolerance (floats) over the whole batch; the layer output compared on
sampled tokens that the oracle computes one by one."""
import numpy as np
import pytest

import oracle
from gpu_harness import FULL, TOL, rel_err, run_layer, say
from workloads import make_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _sample_rows(cfg, o, n=12):
    N = cfg.n_tokens
    rows = set(np.linspace(0, N - 1, min(n, N)).astype(int).tolist())
    dropped = np.nonzero((o["slot_pos"].reshape(N, cfg.top_k) < 0).all(axis=1))[0]
    rows.update(dropped[:4].tolist())                       # tokens that skipped every expert
    return np.array(sorted(rows))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_prefill", "mixtral_decode", "switch_skewed", "deepseek_v3"])
def test_full_size_parity(name):
    cfg = FULL[name]
    say(f"full {name}: generating inputs")
    inp = make_inputs(cfg)
    say(f"full {name}: running layer")
    inp, o, _ = run_layer(cfg, inp)
    tol = TOL[cfg.dtype]
    r = oracle.oracle_route(cfg, o["logits"], inp.sel_bias)
    say(f"full {name}: min selection gap {r.min_gap:.3e}, drop {r.disp.drop_count}, kept {r.disp.offsets[-1]}")
    assert np.array_equal(o["topk_idx"], r.topk_idx)
    assert rel_err(o["gates"], r.gates) <= tol
    assert np.array_equal(o["counts"], r.disp.counts)
    assert np.array_equal(o["offsets"], r.disp.offsets)
    kept = int(r.disp.offsets[-1])
    assert np.array_equal(o["perm"][:kept], r.disp.perm)
    assert np.array_equal(o["slot_pos"], r.disp.slot_pos)
    assert int(o["drop_count"][0]) == r.disp.drop_count
    if cfg.aux_loss:
        assert abs(float(o["aux"][0]) - r.aux) <= tol * abs(r.aux)
    if cfg.gamma > 0:
        assert np.array_equal(o["signs"].astype(np.int64), r.signs)
        assert rel_err(o["sel_bias_next"], r.new_bias) <= 1e-6
    rows = _sample_rows(cfg, o)
    dt = cfg.dtype
    z_ref = oracle.router_logits(oracle.to_f64(inp.x[rows], dt), oracle.to_f64(inp.w_router, dt), inp.logit_bias)
    assert rel_err(o["logits"][rows], z_ref) <= tol
    say(f"full {name}: oracle on {rows.size} sampled tokens")
    _, ref = oracle.oracle_layer(cfg, inp, logits_override=o["logits"], rows=rows)
    err = rel_err(o["out"][rows], ref)
    say(f"full {name}: out rel err {err:.3e}")
    assert err <= tol
