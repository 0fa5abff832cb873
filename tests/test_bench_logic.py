"""bench.py's host-side arithmetic, without a GPU: the measured-ceiling fractions divide the
same achieved rates (or roofline times) by the measured ceilings instead of the published
peaks, and the `--gpus N > 1` guard refuses before touching a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

CEIL = {"hbm_read": {"GBps": 7200.0}, "mfma_bf16": {"TFLOPs": 1800.0}}


def test_frac_of_measured_hbm_and_mfma():
    res = {"roofline": {"bound": "hbm", "achieved": 3600.0}, "expert_gemms": None}
    bench.add_measured_fracs(res, CEIL)
    assert res["roofline"]["frac_of_measured"] == pytest.approx(0.5)
    res = {"roofline": {"bound": "mfma", "achieved": 900.0}}
    bench.add_measured_fracs(res, CEIL)
    assert res["roofline"]["frac_of_measured"] == pytest.approx(0.5)


def test_frac_of_measured_expert_gemms_takes_the_longer_bound():
    # 1.8 TFLOP at 1.8 PFLOP/s = 1 ms; 3.6 GB at 7.2 TB/s = 0.5 ms: the MFMA time bounds it
    g = {"algorithmic_flop": 1.8e12, "algorithmic_bytes": 3.6e9, "ms": 2.0}
    res = {"roofline": {"bound": "alu", "achieved": 1.0}, "expert_gemms": g}
    bench.add_measured_fracs(res, CEIL)
    assert g["frac_of_measured"] == pytest.approx(0.5)
    assert "frac_of_measured" not in res["roofline"]          # the vector-ALU bound has no probe
    g2 = {"algorithmic_flop": 1.8e11, "algorithmic_bytes": 1.44e10, "ms": 4.0}   # 0.1 ms vs 2 ms: bytes
    bench.add_measured_fracs({"expert_gemms": g2}, CEIL)
    assert g2["frac_of_measured"] == pytest.approx(0.5)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
