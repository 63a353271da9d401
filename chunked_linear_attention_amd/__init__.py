"""MI355X-native FLASH gated attention unit with mixed chunk attention
("Transformer Quality in Linear Time"): the layer's forward pass, its
gradients, incremental decoding and the layer stack.

The computation lives in libgau.so: hand-written HIP kernels for gfx950 behind
the C ABI declared in include/gau.h.  This package is the thin Python binding
(ctypes; PyTorch tensors supply device memory and the HIP stream), the build
script, and the seeded synthetic input generator.
"""

import numpy as np

from . import inputs  # noqa: F401
from ._lib import (  # noqa: F401
    GAU_BF16, GAU_F32, GAU_FULL, GAU_GLOBAL_ONLY, GAU_LOCAL_ONLY, STAGE_ATTN, STAGE_OUT, STAGE_PROJ, STAGE_SCAN, STAGE_SCORES, STAGE_STATE, EXPORTS,
    GRAD_NAMES, NOALLOC_SCRATCH_BYTES, GauError, backward, backward_workspace_bytes, decode_reset, decode_step, decode_workspace_bytes, forward, forward_noalloc, forward_segmented, forward_stages, load, make_config,
    probe_mfma, rope_relpos, stack_forward, stack_workspace_bytes,
    status_string, workspace_bytes, workspace_layout,
)


def _torch():
    import torch
    return torch


def device_tensor(a, dtype, device="cuda"):
    """numpy float32 array -> contiguous device tensor of `dtype` (bf16 values
    are taken as exact bf16 bit patterns via round-to-nearest-even)."""
    torch = _torch()
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == torch.bfloat16:
        bits = inputs.bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def device_layer(inp, dtype, device="cuda"):
    """Upload one layer's inputs (numpy, pages' orientation) in the ABI layout:
    weights output-major (W transposed on the host), scale/offset/relpos fp32."""
    torch = _torch()
    out = {}
    if "X" in inp:
        out["X"] = device_tensor(inp["X"], dtype, device)
    for k in ("W_u", "W_v", "W_z", "W_o"):
        out[k] = device_tensor(np.ascontiguousarray(inp[k].T), dtype, device)
    out["scale"] = device_tensor(inp["gamma"], torch.float32, device)
    out["offset"] = device_tensor(inp["beta"], torch.float32, device)
    out["relpos"] = device_tensor(inp["relpos"], torch.float32, device)
    return out


def gau_forward(X, W_u, W_v, W_z, W_o, scale, offset, relpos, C, causal,
                quad_scale=None, lin_scale=None, out=None, workspace=None, stream=None, rope=False,
                parts="both"):
    """O = FLASH layer forward of X [B, T, d] (weights output-major).

    Allocates O and the workspace with torch.empty when not given; all
    arithmetic runs in libgau's kernels on the current (or given) stream.
    """
    torch = _torch()
    B, T, d = X.shape
    e = W_u.shape[0]
    s = W_z.shape[0]
    dt = GAU_BF16 if X.dtype == torch.bfloat16 else GAU_F32
    cfg = make_config(B, T, d, e, s, C, causal, dt, quad_scale, lin_scale, rope, parts)
    if out is None:
        out = torch.empty_like(X)
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(cfg), 1), dtype=torch.uint8, device=X.device)
    forward(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, out, workspace, stream)
    return out


def gau_backward(X, W_u, W_v, W_z, W_o, scale, offset, relpos, C, causal, dO,
                 quad_scale=None, lin_scale=None, workspace=None, stream=None, rope=False, parts="both",
                 chunk_segments=None):
    """Gradients of <dO, O> for O = gau_forward(X, ...) with the same rope and
    parts (with chunk_segments, an int32 device tensor [B, T / C], the
    segment-masked layer of forward_segmented): a dict of fp32 device tensors
    keyed X, W_u, W_v, W_z, W_o (output-major, like the weights), scale,
    offset, relpos.  Every step runs in libgau's kernels."""
    torch = _torch()
    B, T, d = X.shape
    e = W_u.shape[0]
    s = W_z.shape[0]
    dt = GAU_BF16 if X.dtype == torch.bfloat16 else GAU_F32
    cfg = make_config(B, T, d, e, s, C, causal, dt, quad_scale, lin_scale, rope, parts)
    like = {"X": X, "W_u": W_u, "W_v": W_v, "W_z": W_z, "W_o": W_o, "scale": scale, "offset": offset,
            "relpos": relpos}
    grads = {k: torch.empty(like[k].shape, dtype=torch.float32, device=X.device) for k in GRAD_NAMES}
    if workspace is None:
        workspace = torch.empty(max(backward_workspace_bytes(cfg), 1), dtype=torch.uint8, device=X.device)
    backward(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, dO, grads, workspace, stream,
             chunk_segments=chunk_segments)
    return grads
