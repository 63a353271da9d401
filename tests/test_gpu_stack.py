"""GPU parity of the layer stack (RMS pre-norm, FLASH layer, residual add)
against the float64 oracle."""

import numpy as np
import pytest
import torch

import chunked_linear_attention_amd as g
from chunked_linear_attention_amd import inputs
from oracle import gau_oracle as orc

from _gpu import assert_close, chunk_errors, torch_dtype

pytestmark = pytest.mark.gpu


def _run_stack(X, layers, B, T, d, e, s, C, dtype, causal=True):
    tdt = torch_dtype(dtype)
    cfg = g.make_config(B, T, d, e, s, C, causal, g.GAU_BF16 if dtype == "bf16" else g.GAU_F32)
    dev = [g.device_layer(L, tdt) for L in layers]
    x = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).cuda()
    ws = torch.empty(g.stack_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    g.stack_forward(cfg, x, dev, ws)
    torch.cuda.synchronize()
    return x.cpu().numpy().astype(np.float64)


STACK_SHAPES = [
    # B, T, d, e, s, C, layers
    (2, 512, 256, 512, 128, 128, 3),
    (3, 192, 384, 768, 128, 64, 2),   # B*T = 576: the output tiles' last token tile ragged, d not a power of two
]


@pytest.mark.parametrize("shape", STACK_SHAPES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_L{}".format(*c))
@pytest.mark.parametrize("heads", ["workload", "wide"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_stack_matches_oracle(dtype, heads, shape):
    B, T, d, e, s, C, nl = shape
    X, layers = inputs.make_stack_inputs(B, T, d, e, s, C, nl, weight_seed=300, x_seed=301, dtype=dtype,
                                         heads=heads)
    got = _run_stack(X, layers, B, T, d, e, s, C, dtype)
    ref = orc.flash_stack_forward(X, layers, C, True)
    tol = 1e-4 if dtype == "f32" else 2e-2
    assert_close(got, ref, tol, "stack")
    # the tolerance applied to what the layers added to the residual stream
    # (X is exact on both sides), and that contribution is not small
    assert_close(got - X, ref - X, tol, "stack minus its input")
    assert np.max(np.abs(ref - X)) > 0.1 * np.max(np.abs(X))


def test_full_stack_workload():
    """24 layers at d=1024, B=2, T=8192, C=256: every token of both
    sequences against the oracle, the output and the layers' contribution
    (output minus input) each under the bf16 gate, and every chunk of that
    contribution under the gate relative to its own largest value."""
    cfg = inputs.WORKLOADS["stack24_bf16_B2_T8192_d1024_C256"]
    B, T, d, e, s, C, nl = (cfg[k] for k in ("B", "T", "d", "e", "s", "C", "layers"))
    X, layers = inputs.make_stack_inputs(**cfg)
    print("stack24 B=2 T=8192 d=1024: GPU run", flush=True)
    got = _run_stack(X, layers, B, T, d, e, s, C, "bf16")
    assert np.all(np.isfinite(got))
    print("stack24: oracle", flush=True)
    ref = orc.flash_stack_forward(X, layers, C, True)
    assert_close(got, ref, 2e-2, "stack24")
    err = assert_close(got - X, ref - X, 2e-2, "stack24 minus its input")
    ce = chunk_errors(got - X, ref - X, C)
    print(f"stack24: delta {err:.2e}, worst per-chunk {ce.max():.2e} (chunk {int(ce.argmax())})", flush=True)
    assert ce.max() <= 2e-2, f"chunk {int(ce.argmax())}: {ce.max():.3e}"
