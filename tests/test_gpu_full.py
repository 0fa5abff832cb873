"""GPU parity at the workloads' full sizes, in the configuration bench.py
times: routing, dispatch, aux and bias step compared bit-exactly (integers)
or to tolerance (floats) over the whole batch, and the layer output of every
token against the oracle (which streams the experts one at a time)."""
import numpy as np
import pytest

import oracle
from gpu_harness import FULL, TOL, rel_err, run_layer, say
from workloads import make_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["mixtral_prefill", "mixtral_decode", "switch_skewed", "deepseek_v3",
                                  "deepseek_v3_balanced"])
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
    dt = cfg.dtype
    z_ref = oracle.router_logits(oracle.to_f64(inp.x, dt), oracle.to_f64(inp.w_router, dt), inp.logit_bias)
    err_z = rel_err(o["logits"], z_ref)
    say(f"full {name}: logits rel err {err_z:.3e}")
    assert err_z <= tol
    say(f"full {name}: oracle on all {cfg.n_tokens} tokens")

    def progress(e):
        if e % 32 == 31 or e == cfg.n_experts - 1:
            say(f"full {name}: oracle through expert {e}")
    _, ref = oracle.oracle_layer(cfg, inp, logits_override=o["logits"], progress=progress)
    err = rel_err(o["out"], ref)
    say(f"full {name}: out rel err {err:.3e} over every token")
    assert err <= tol
    # tokens that skipped every expert keep exactly their residual (+ shared expert)
    dropped = np.nonzero((o["slot_pos"].reshape(cfg.n_tokens, cfg.top_k) < 0).all(axis=1))[0]
    if dropped.size:
        err_d = rel_err(o["out"][dropped], ref[dropped])
        say(f"full {name}: {dropped.size} fully dropped tokens, rel err {err_d:.3e}")
        assert err_d <= tol
