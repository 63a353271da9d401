"""GPU parity of the layer over packed sequences (gau_forward_segmented):
the segment-masked linear term (the listing's row-normalised chunk mask on
the summaries; the local part unmasked) against the float64 oracle, and the
packed row against its documents run alone."""

import numpy as np
import pytest
import torch

import chunked_linear_attention_amd as g

from _gpu import assert_close, chunk_errors, make, oracle_layer, tol_for, torch_dtype
from oracle import gau_oracle as orc

pytestmark = pytest.mark.gpu


def run_segmented(inp, seg, B, T, d, e, s, C, causal, dtype, parts="both"):
    """O and the per-chunk states P [B, G, e, s] the forward leaves in S's region."""
    tdt = torch_dtype(dtype)
    dev = g.device_layer(inp, tdt)
    cfg = g.make_config(B, T, d, e, s, C, causal, g.GAU_BF16 if dtype == "bf16" else g.GAU_F32, parts=parts)
    ws = torch.full((g.workspace_bytes(cfg),), 0xFF, dtype=torch.uint8, device="cuda")
    O = torch.empty((B, T, d), dtype=tdt, device="cuda")
    sg = torch.from_numpy(np.ascontiguousarray(seg, dtype=np.int32)).cuda()
    g.forward_segmented(cfg, sg, dev["X"], dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"],
                        dev["offset"], dev["relpos"], O, ws)
    torch.cuda.synchronize()
    L = g.workspace_layout(cfg)
    G = T // C
    eb = 2 if dtype == "bf16" else 4
    n = B * G * e * s
    P = ws[L["S"]:L["S"] + n * eb].view(tdt).reshape(B, G, e, s).float().cpu().numpy().astype(np.float64)
    return O.float().cpu().numpy().astype(np.float64), P


def random_runs(rng, B, G, max_run):
    """Per-row chunk ids: runs of 1..max_run chunks, ids increasing."""
    seg = np.zeros((B, G), np.int32)
    for b in range(B):
        g0, sid = 0, 0
        while g0 < G:
            n = int(rng.integers(1, max_run + 1))
            seg[b, g0:g0 + n] = sid
            g0, sid = g0 + n, sid + 1
    return seg


CASES = [
    # B, T, d, e, s, C, dtype, causal
    (1, 512, 128, 256, 128, 64, "f32", True),
    (2, 512, 128, 256, 128, 64, "f32", False),
    (2, 1024, 256, 512, 128, 128, "bf16", True),
    (1, 1024, 256, 512, 256, 128, "bf16", False),
    (1, 2048, 256, 512, 128, 512, "bf16", True),
    (2, 1024, 128, 1024, 128, 64, "bf16", True),     # Z formed inside the U tiles
    (1, 960, 128, 1536, 128, 64, "bf16", False),     # e = 1536 mapping, ragged last token tile
    (1, 1024, 128, 2048, 256, 256, "f32", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}".format(
    *c[:7], "causal" if c[7] else "full"))
def test_segmented_layer_matches_oracle(case):
    B, T, d, e, s, C, dtype, causal = case
    G = T // C
    rng = np.random.default_rng(B * 97 + T + C)
    seg = random_runs(rng, B, G, max(1, G // 3))
    seg[0, -1] = seg[0, -2] if G > 1 else seg[0, -1]
    print(f"segmented case {case} ids {seg.tolist()}", flush=True)
    inp = make(B, T, d, e, s, C, dtype, seed=B * 331 + T + C, heads="wide")
    O, P = run_segmented(inp, seg, B, T, d, e, s, C, causal, dtype)
    ref, im = oracle_layer(inp, C, causal, intermediates=True, chunk_segments=seg)
    tol = tol_for(dtype)
    assert_close(P, im["P"].transpose(0, 1, 3, 2), tol, "P")
    assert_close(O, ref, tol, "O")
    ce = chunk_errors(O, ref, C)
    assert ce.max() <= tol, f"chunk {int(ce.argmax())}: {ce.max():.3e}"
    # the mask matters: the plain layer differs
    plain = oracle_layer(inp, C, causal)
    assert np.max(np.abs(plain - ref)) > 10 * tol * np.max(np.abs(ref))


@pytest.mark.parametrize("parts", ["local", "global"])
def test_segmented_parts(parts):
    B, T, d, e, s, C = 2, 1024, 256, 512, 128, 128
    seg = np.array([[0, 0, 0, 1, 1, 2, 2, 2], [4, 4, 4, 4, 4, 4, 4, 4]], np.int32)
    inp = make(B, T, d, e, s, C, "bf16", seed=55, heads="wide")
    O, _ = run_segmented(inp, seg, B, T, d, e, s, C, True, "bf16", parts=parts)
    ref = oracle_layer(inp, C, True, chunk_segments=seg, parts=parts)
    assert_close(O, ref, 2e-2, f"segmented {parts}")


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_packed_row_equals_documents_alone_bitwise(causal):
    """Three documents packed into one row (each starting on a chunk
    boundary, not on a 256-token tile boundary) give, token for token, the
    bits each document gives alone as one segment."""
    C, d, e, s = 64, 256, 512, 128
    lens = [192, 448, 128]
    T = sum(lens)
    inp = make(1, T, d, e, s, C, "bf16", seed=61, heads="wide")
    seg = np.concatenate([np.full(n // C, i + 3, np.int32) for i, n in enumerate(lens)])[None, :]
    packed, _ = run_segmented(inp, seg, 1, T, d, e, s, C, causal, "bf16")
    t0 = 0
    for n in lens:
        one = dict(inp, X=inp["X"][:, t0:t0 + n].copy())
        alone, _ = run_segmented(one, np.zeros((1, n // C), np.int32), 1, n, d, e, s, C, causal, "bf16")
        np.testing.assert_array_equal(packed[:, t0:t0 + n], alone)
        t0 += n


def test_packed_benchmark_shape():
    """B=2, T=8192, d=768, C=256, bf16, causal, each row packed with
    documents of 1 to 8 chunks: every token against the oracle, every chunk
    under the gate relative to its own largest value."""
    B, T, d, e, s, C = 2, 8192, 768, 1536, 128, 256
    seg = random_runs(np.random.default_rng(8192), B, T // C, 8)
    inp = make(B, T, d, e, s, C, "bf16", seed=8193)
    print(f"packed benchmark shape: ids {seg.tolist()}", flush=True)
    O, _ = run_segmented(inp, seg, B, T, d, e, s, C, True, "bf16")
    ref = oracle_layer(inp, C, True, chunk_segments=seg)
    err = assert_close(O, ref, 2e-2, "packed B=2 T=8192")
    ce = chunk_errors(O, ref, C)
    print(f"packed B=2 T=8192: global {err:.2e}, worst per-chunk {ce.max():.2e}", flush=True)
    assert ce.max() <= 2e-2, f"chunk {int(ce.argmax())}: {ce.max():.3e}"
