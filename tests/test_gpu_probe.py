"""The MFMA measurement probe (gau_probe_mfma) runs and reports a rate within
the chip's published bf16 peak."""

import pytest
import torch

import chunked_linear_attention_amd as g

pytestmark = pytest.mark.gpu


def test_mfma_probe_rate_is_below_the_published_peak():
    out = torch.zeros(1, dtype=torch.float32, device="cuda")
    g.probe_mfma(256, 50, out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    flops = g.probe_mfma(1024, 400, out)
    b.record()
    torch.cuda.synchronize()
    tflops = flops / (a.elapsed_time(b) * 1e-3) / 1e12
    print(f"mfma probe: {tflops:.0f} TFLOP/s", flush=True)
    assert 100.0 < tflops < 2516.6 * 1.02
    assert out.item() == 0.0  # the sentinel store never happens
