"""gau_forward_noalloc (the forward with its workspace in the library's device
scratch array) against gau_forward through the C ABI: two calls in a row, the
second smaller, each bitwise equal to gau_forward's output on the same inputs
(the same kernels in the same order), and the size check without a launch."""

import numpy as np
import pytest
import torch

import chunked_linear_attention_amd as g

from _gpu import make, torch_dtype

pytestmark = pytest.mark.gpu


def _pair(B, T, d, e, s, C, dtype, causal, seed):
    print(f"noalloc case B={B} T={T} d={d} e={e} s={s} C={C} {dtype} causal={causal}", flush=True)
    inp = make(B, T, d, e, s, C, dtype, seed=seed, heads="wide")
    tdt = torch_dtype(dtype)
    dev = g.device_layer(inp, tdt)
    cfg = g.make_config(B, T, d, e, s, C, causal, g.GAU_BF16 if dtype == "bf16" else g.GAU_F32)
    assert g.workspace_bytes(cfg) <= g.NOALLOC_SCRATCH_BYTES
    args = (dev["X"], dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"], dev["relpos"])
    ws = torch.empty(g.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    ref = torch.empty((B, T, d), dtype=tdt, device="cuda")
    g.forward(cfg, *args, ref, ws)
    got = torch.full((B, T, d), float("nan"), dtype=tdt, device="cuda")
    g.forward_noalloc(cfg, *args, got)
    torch.cuda.synchronize()
    a, b = ref.float().cpu().numpy(), got.float().cpu().numpy()
    assert np.all(np.isfinite(b))
    np.testing.assert_array_equal(b, a)


def test_noalloc_forward_equals_forward_on_two_calls():
    # first call: B*T = 4096 tokens at the benchmark width (36 MiB of the 64)
    _pair(2, 2048, 768, 1536, 128, 256, "bf16", True, seed=901)
    # second call, smaller, non-causal: the array still holds the first
    # call's intermediates, none of which may leak into this result
    _pair(1, 512, 256, 512, 128, 128, "bf16", False, seed=902)
    # and an fp32 layer after both
    _pair(1, 256, 128, 256, 128, 64, "f32", True, seed=903)


def test_noalloc_forward_rejects_more_than_its_scratch():
    """B*T = 8192 at d = 768 needs 72 MiB: GAU_ERR_WORKSPACE, nothing queued
    (the output keeps its sentinel)."""
    B, T, d, e, s, C = 1, 8192, 768, 1536, 128, 256
    cfg = g.make_config(B, T, d, e, s, C, True, g.GAU_BF16)
    assert g.workspace_bytes(cfg) > g.NOALLOC_SCRATCH_BYTES
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(shape, dtype=dt, device="cuda")
    O = torch.full((B, T, d), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(g.GauError) as ei:
        g.forward_noalloc(cfg, z(B, T, d), z(e, d), z(e, d), z(s, d), z(d, e), z(4, s, dt=torch.float32),
                          z(4, s, dt=torch.float32), z(2 * C - 1, dt=torch.float32), O)
    assert ei.value.status == 5
    torch.cuda.synchronize()
    assert bool(torch.all(O == 7.0))
