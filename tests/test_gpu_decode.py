"""GPU parity of incremental decoding: gau_decode_step for t = 0, 1, ... gives
the causal layer's outputs token by token (float64 oracle)."""

import numpy as np
import pytest
import torch

import chunked_linear_attention_amd as g
from oracle import gau_oracle as orc

from _gpu import assert_close, make, oracle_layer, tol_for, torch_dtype

pytestmark = pytest.mark.gpu


def _decode(inp, B, T, d, e, s, C, dtype, steps, rope=False, reset_twice=False, parts="both"):
    tdt = torch_dtype(dtype)
    dev = g.device_layer(inp, tdt)
    cfg = g.make_config(B, T, d, e, s, C, True, g.GAU_BF16 if dtype == "bf16" else g.GAU_F32, rope=rope,
                        parts=parts)
    ws = torch.empty(g.decode_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # the reset must clear what the state needs
    X = dev["X"]
    runs = []
    for _ in range(2 if reset_twice else 1):
        g.decode_reset(cfg, ws)
        out = torch.empty((B, steps, d), dtype=tdt, device="cuda")
        o = torch.empty((B, d), dtype=tdt, device="cuda")
        for t in range(steps):
            x = X[:, t].contiguous()
            g.decode_step(cfg, t, x, dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"],
                          dev["relpos"], o, ws)
            out[:, t] = o
        torch.cuda.synchronize()
        runs.append(out.float().cpu().numpy().astype(np.float64))
    return runs


CASES = [
    # B, T, d, e, s, C, dtype, steps, rope
    (2, 192, 128, 256, 128, 64, "f32", 192, False),    # three chunks, state updated twice
    (2, 384, 256, 512, 128, 128, "bf16", 384, False),
    (1, 256, 128, 1024, 256, 128, "bf16", 256, True),  # s = 256, RoPE
    (3, 192, 128, 256, 128, 64, "bf16", 130, False),   # stop inside a chunk
    (8, 128, 128, 256, 128, 64, "f32", 128, True),     # the largest batch of the GEMV products
    (9, 128, 128, 256, 128, 64, "f32", 128, True),     # B >= 9: the products on the MFMA core
    (20, 128, 128, 256, 128, 64, "bf16", 128, False),
    (70, 128, 256, 512, 256, 64, "f32", 70, True),     # ... two token tiles, the second ragged
    (96, 128, 128, 1536, 128, 64, "f32", 128, False),   # attention with 8 features per thread
    (176, 128, 128, 1536, 128, 64, "bf16", 128, True),  # ... bf16 (16-byte loads), RoPE
    # gamma ~ N(1, 0.5^2), beta ~ N(0, 0.3^2): the heads' offsets count
    (2, 192, 128, 256, 128, 64, "f32", 192, False, "wide"),
    (2, 384, 256, 512, 128, 128, "bf16", 384, True, "wide"),
    (20, 128, 128, 256, 256, 64, "bf16", 128, False, "wide"),
    (96, 128, 128, 1536, 128, 64, "f32", 128, True, "wide"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}steps{}{}".format(
    *c[:7], c[7], "_rope" if c[8] else "", "_wide" if len(c) > 9 else ""))
def test_decoding_matches_the_causal_layer(case):
    B, T, d, e, s, C, dtype, steps, rope = case[:9]
    heads = case[9] if len(case) > 9 else "workload"
    inp = make(B, T, d, e, s, C, dtype, seed=B * 389 + T + C, heads=heads)
    got, = _decode(inp, B, T, d, e, s, C, dtype, steps, rope)
    ref = oracle_layer(inp, C, True, rope=rope)[:, :steps]
    assert_close(got, ref, tol_for(dtype), "decoded O")
    # also per chunk, so early chunks (small outputs) are checked too
    for c0 in range(0, steps, C):
        assert_close(got[:, c0:c0 + C], ref[:, c0:c0 + C], 2 * tol_for(dtype), f"chunk at {c0}")


def test_reset_restarts_the_state_bitwise():
    B, T, d, e, s, C = 2, 192, 128, 256, 128, 64
    inp = make(B, T, d, e, s, C, "bf16", seed=3)
    a, b = _decode(inp, B, T, d, e, s, C, "bf16", 150, reset_twice=True)
    assert np.array_equal(a, b)


def test_decoding_agrees_with_the_parallel_forward():
    """The same layer through gau_forward and through gau_decode_step."""
    B, T, d, e, s, C = 2, 512, 256, 512, 128, 128
    inp = make(B, T, d, e, s, C, "bf16", seed=4)
    got, = _decode(inp, B, T, d, e, s, C, "bf16", T)
    from _gpu import run_layer
    O, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16")
    assert_close(got, O, 2e-2, "decode vs forward")


@pytest.mark.parametrize("parts,B", [("local", 2), ("global", 2), ("global", 5)])
def test_decoding_local_only_and_global_only(parts, B):
    T, d, e, s, C = 192, 128, 256, 128, 64
    inp = make(B, T, d, e, s, C, "bf16", seed=17)
    got, = _decode(inp, B, T, d, e, s, C, "bf16", 140, parts=parts)
    ref = oracle_layer(inp, C, True, parts=parts)[:, :140]
    assert_close(got, ref, 2e-2, f"decoded O ({parts})")
