"""The measurement probes run on the GPU: the read probe leaves its buffer as it was and
reads every byte once at a rate near the HBM peak at most; the MFMA probe's FLOP count per iteration is
the chip's wavefronts times two 32x32x16 products, and its rate stays below the
published dense bf16 peak."""
import pytest

pytestmark = pytest.mark.gpu


def test_probes_run():
    import torch
    import mixture_experts_layer_histogram_amd as M
    buf = torch.randint(0, 255, (1 << 30,), dtype=torch.uint8, device="cuda")   # 4x the last-level cache
    ref = buf.clone()
    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    M.probe_hbm_read(buf, sink)
    e0.record()
    M.probe_hbm_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    assert torch.equal(buf, ref)
    # near the published HBM peak at most (the part of the buffer the last-level cache may still
    # hold from the first call reads faster)
    assert 100.0 < gbs <= 8000.0 * 1.25, gbs

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert M.probe_mfma_flop_per_iter() == cus * 8 * 2 * 2 * 32 * 32 * 16
    ops = torch.randn(4096, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()
    iters = 20000
    M.probe_mfma_bf16(ops, iters, sink)
    e0.record()
    M.probe_mfma_bf16(ops, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    tflops = M.probe_mfma_flop_per_iter() * iters / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 100.0 < tflops <= 2500.0 * 1.02, tflops
