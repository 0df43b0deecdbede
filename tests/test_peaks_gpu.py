"""The measured-peak kernels on the GPU: they run, read every byte they are
given (a rate bounded by the published HBM peak), keep their sink untouched
on zero data, and the MFMA loop stays under the published bf16 peak."""
import pytest

import prefill_decode_hybrid_amd as pod

pytestmark = pytest.mark.gpu


def _time(torch, fn, n=3):
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / n


def test_peak_read_and_mfma():
    import torch
    nbytes, wgs = 1 << 30, 256
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    t = _time(torch, lambda: pod.pod_attn_peak_read(buf, nbytes, wgs, sink))
    rate = nbytes / t
    print(f"peak read: {rate / 1e12:.2f} TB/s")
    assert 0.5e12 < rate < 8.0e12 * 1.05
    iters = 256
    t = _time(torch, lambda: pod.pod_attn_peak_mfma(wgs, iters, sink))
    flops = wgs * 4 * iters * pod.PEAK_MFMA_FLOPS_PER_ITER_WAVE / t
    print(f"peak mfma: {flops / 1e12:.0f} TFLOP/s")
    assert 100e12 < flops < 2516.6e12 * 1.05
    assert int(sink.item()) == 0
