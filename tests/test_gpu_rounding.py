"""GPU: the epilogues' fp32 -> bf16 rounding is round-to-nearest-even, bit for bit.

The down projection's output element y[r, c] = sum_k h[r, k] W2[c, k]; with h[r] holding 1 at two
positions and 0 elsewhere it is the sum of two bf16 weights, which fp32 holds exactly when their
exponents are close (here within 4 binades).  So the kernel's result must equal that exact sum
rounded to bf16 with ties to even, computed below with integer arithmetic on the fp32 bits.  Half
of the columns are built as exact ties (a weight plus half a bf16 unit in its last place), the
rest are random pairs; two segments (300 and 50 rows) take the 256-row kernel (with a K-part
fix-up, as the few units are split over K) and the 64-row kernel."""
import numpy as np
import pytest

from gpu_harness import host, say
from workloads import MIXTRAL_PREFILL

pytestmark = pytest.mark.gpu


def _rne_bf16_bits(x32: np.ndarray) -> np.ndarray:
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def test_epilogue_rounding_is_nearest_even():
    import torch
    import mixture_experts_layer_histogram_amd as M
    rows = [300, 50]
    R, E, d, F = sum(rows), len(rows), 2048, 256
    cfg = MIXTRAL_PREFILL.scaled(name="rounding", n_tokens=R, n_experts=E, top_k=1, d_model=d, d_ff=F)
    c = M.config_from(cfg)
    rng = np.random.default_rng(11)
    # weights: bf16 values with exponents in [-2, 2), random signs and mantissas
    mant = rng.integers(0, 128, size=(E, d, F))
    expo = rng.integers(125, 129, size=(E, d, F))
    sign = rng.integers(0, 2, size=(E, d, F))
    w_bits = ((sign << 15) | (expo << 7) | mant).astype(np.uint16)
    # tie columns (c even): the odd K entry is +-half a bf16 ulp of the even entry before it
    half_ulp_exp = expo[:, 0::2, 0::2] - 8                      # 2^(e - 127 - 8): half of 2^(e - 127 - 7)
    tie = ((rng.integers(0, 2, size=half_ulp_exp.shape) << 15) | (half_ulp_exp << 7)).astype(np.uint16)
    w_bits[:, 0::2, 1::2] = tie
    w32 = (w_bits.astype(np.uint32) << 16).view(np.float32)
    # h row r picks the K pair (2 (r mod 128), 2 (r mod 128) + 1)
    h = np.zeros((R, F), np.float32)
    kk = 2 * (np.arange(R) % (F // 2))
    h[np.arange(R), kk] = 1.0
    h[np.arange(R), kk + 1] = 1.0
    offs = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    seg = np.repeat(np.arange(E), rows)
    exact = w32[seg[:, None], np.arange(d)[None, :], kk[:, None]].astype(np.float64) + \
        w32[seg[:, None], np.arange(d)[None, :], kk[:, None] + 1].astype(np.float64)
    s32 = exact.astype(np.float32)
    assert np.array_equal(s32.astype(np.float64), exact), "test construction: sums must be exact in fp32"
    want = _rne_bf16_bits(s32)
    ties = ((s32.view(np.uint32) & 0xFFFF) == 0x8000)
    say(f"rounding: {want.size} outputs, {int(ties.sum())} exact ties")
    assert ties.sum() > 10000
    half_up = ((s32.view(np.uint32).astype(np.uint64) + 0x8000) >> 16).astype(np.uint16)
    assert (half_up != want).sum() > 10000, "the outputs must tell ties-to-even from ties-away rounding"
    dev = torch.device("cuda")
    hd = torch.from_numpy(h).to(torch.bfloat16).to(dev)
    w2 = torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.full((R, d), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M.workspace_size(c), dtype=torch.uint8, device=dev)
    M.expert_down(c, hd, torch.from_numpy(offs).to(dev), w2, y, ws=ws)
    torch.cuda.synchronize()
    got = host(y.view(torch.int16)).view(np.uint16)
    bad = got != want
    assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:5])
