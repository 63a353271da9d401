"""Helpers for the GPU parity tests: run libgau on seeded inputs and read its
outputs and workspace intermediates back to the host."""

import numpy as np
import torch

import chunked_linear_attention_amd as g
from chunked_linear_attention_amd import inputs
from oracle import gau_oracle as orc

BF16_TOL = 2e-2   # max|err| <= 2e-2 * max|ref|, bf16 storage with fp32 accumulation
F32_TOL = 1e-4    # max|err| <= 1e-4 * max|ref|, fp32


def tol_for(dtype):
    return BF16_TOL if dtype == "bf16" else F32_TOL


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def run_layer(inp, B, T, d, e, s, C, causal, dtype, quad_scale=None, lin_scale=None, stream=None, rope=False,
              parts="both", stagewise=False):
    """Forward on the GPU; returns (O as float64 numpy, workspace, cfg, layout).

    The forward reuses two regions in place (Y overwrites U; causal: P
    overwrites S).  With stagewise=True the workspace returned is the pair
    (after the full forward, after a second run of the stages up to the chunk
    states alone), and ws_array reads U and S from the second one."""
    tdt = torch_dtype(dtype)
    dev = g.device_layer(inp, tdt)
    cfg = g.make_config(B, T, d, e, s, C, causal, g.GAU_BF16 if dtype == "bf16" else g.GAU_F32,
                        quad_scale, lin_scale, rope, parts)
    ws = torch.zeros(g.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    O = torch.empty((B, T, d), dtype=tdt, device="cuda")
    args = (dev["X"], dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"], dev["relpos"])
    g.forward(cfg, *args, O, ws, stream)
    if stagewise:
        mid = torch.zeros_like(ws)
        g.forward_stages(cfg, g.STAGE_PROJ, g.STAGE_STATE, *args, torch.empty_like(O), mid, stream=stream)
        ws = (ws, mid)
    torch.cuda.synchronize()
    return O.float().cpu().numpy().astype(np.float64), ws, cfg, g.workspace_layout(cfg)


# regions a later stage of the forward overwrites in place: name -> the region
# that takes its place
IN_PLACE = {"U": "Y", "S": "P"}


def ws_array(ws, layout, name, shape, dtype):
    """A workspace region as a float64 numpy array of `shape` (from the
    stages-up-to-the-states snapshot when the full forward overwrote it)."""
    if isinstance(ws, tuple):
        final, mid = ws
        ws = mid if (name in IN_PLACE and layout[name] == layout[IN_PLACE[name]]) else final
    n = int(np.prod(shape))
    tdt, eb = torch_dtype(dtype), (2 if dtype == "bf16" else 4)
    off = layout[name]
    t = ws[off:off + n * eb].view(tdt).reshape(shape)
    return t.float().cpu().numpy().astype(np.float64)


def oracle_layer(inp, C, causal, quad_scale=None, lin_scale=None, intermediates=False, rope=False, parts="both",
                 chunk_segments=None):
    return orc.flash_forward(inp["X"], inp["W_u"], inp["W_v"], inp["W_z"], inp["W_o"], inp["gamma"],
                             inp["beta"], inp["relpos"], C, causal, quad_scale, lin_scale,
                             return_intermediates=intermediates, use_rope=rope, parts=parts,
                             chunk_segments=chunk_segments)


def rel_err(got, ref):
    """max|got - ref| / max|ref|."""
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def assert_close(got, ref, tol, what=""):
    err = rel_err(got, ref)
    assert err <= tol, f"{what}: max|err|/max|ref| = {err:.3e} > {tol:.1e}"
    return err


def chunk_errors(got, ref, C):
    """Per-chunk max|err| / max|ref| (diagnostic; not the gate)."""
    B, T, _ = ref.shape
    G = T // C
    e = np.abs(got - ref).reshape(B, G, -1).max(axis=(0, 2))
    r = np.abs(ref).reshape(B, G, -1).max(axis=(0, 2))
    return e / np.maximum(r, 1e-300)


def make(B, T, d, e, s, C, dtype, seed, heads="workload"):
    """Seeded inputs with the workloads' recipe at a given shape (heads="wide":
    gamma ~ N(1, 0.5^2) and beta ~ N(0, 0.3^2), so the offsets count)."""
    return inputs.make_layer_inputs(B=B, T=T, d=d, e=e, s=s, C=C, seed=seed, dtype=dtype, heads=heads)
