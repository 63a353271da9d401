"""GPU parity: libgau (through its C ABI) against the float64 CPU oracle on the
same seeded inputs.  Gate: max|err| <= 1e-4 * max|ref| (fp32) and
<= 2e-2 * max|ref| (bf16 storage, fp32 accumulation), on the output and on
every stored intermediate."""

import numpy as np
import pytest
import torch

import chunked_linear_attention_amd as g
from chunked_linear_attention_amd import inputs
from oracle import gau_oracle as orc

from _gpu import (assert_close, chunk_errors, make, oracle_layer, run_layer, tol_for, ws_array,
                  torch_dtype)

pytestmark = pytest.mark.gpu


def _stagewise(ws, L, im, B, T, e, s, C, causal, dtype):
    tol = tol_for(dtype)
    G = T // C
    assert_close(ws_array(ws, L, "U", (B, T, e), dtype), im["U"], tol, "U")
    assert_close(ws_array(ws, L, "Vt", (B, e, T), dtype), im["V"].transpose(0, 2, 1), tol, "Vt")
    assert_close(ws_array(ws, L, "Q_quad", (B, T, s), dtype), im["Q_quad"], tol, "Q_quad")
    assert_close(ws_array(ws, L, "K_quad", (B, T, s), dtype), im["K_quad"], tol, "K_quad")
    assert_close(ws_array(ws, L, "Q_lin", (B, T, s), dtype), im["Q_lin"], tol, "Q_lin")
    assert_close(ws_array(ws, L, "K_lin_t", (B, s, T), dtype), im["K_lin"].transpose(0, 2, 1), tol, "K_lin_t")
    assert_close(ws_array(ws, L, "S", (B, G, e, s), dtype), im["S"].transpose(0, 1, 3, 2), tol, "S")
    Gp = G if causal else 1
    P = ws_array(ws, L, "P", (B, Gp, e, s), dtype)
    refP = im["P"].transpose(0, 1, 3, 2)[:, :Gp]
    if causal:
        assert np.all(P[:, 0] == 0.0), "P_0 must be exactly zero"
    if np.max(np.abs(refP)) > 0:
        assert_close(P, refP, tol, "P")
    A = ws_array(ws, L, "A", (B * G, C, C), dtype)
    refA = im["kernel"].reshape(B * G, C, C)
    if causal:  # key tiles above the diagonal are not written (and not read)
        ts = 128 if C >= 128 else 64
        t = np.arange(C) // ts
        keep = t[None, :] <= t[:, None]
        A, refA = A[:, keep], refA[:, keep]
    assert_close(A, refA, tol, "A")
    assert_close(ws_array(ws, L, "Y", (B, T, e), dtype), im["Y"], tol, "Y")


SMALL = [
    # B, T, d, e, s, C, dtype, causal
    (1, 256, 128, 256, 128, 64, "f32", True),
    (1, 256, 128, 256, 128, 64, "f32", False),
    (2, 512, 256, 512, 128, 128, "bf16", True),
    (2, 512, 256, 512, 128, 128, "bf16", False),
    (1, 320, 128, 256, 128, 64, "bf16", True),     # 320 rows: two full 128-row tiles + a ragged 64
    (1, 320, 128, 256, 128, 64, "f32", True),
    (1, 1024, 256, 512, 128, 512, "bf16", True),   # C = 512
    (1, 1024, 256, 512, 128, 512, "bf16", False),
    (1, 512, 256, 512, 256, 256, "bf16", True),    # s = 256
    (1, 256, 128, 256, 256, 128, "f32", False),
    (3, 128, 128, 256, 128, 128, "bf16", True),    # C = T: one chunk per sequence
    (2, 192, 384, 768, 128, 64, "bf16", True),     # d, e not powers of two
    (1, 256, 128, 1024, 128, 64, "f32", True),     # e >= 1024: Z formed inside the U tiles
    (1, 320, 256, 1024, 256, 64, "bf16", False),   # ... with s = 256 and a ragged row tile
    (2, 256, 128, 1280, 128, 128, "bf16", True),
    (1, 960, 128, 1536, 128, 64, "bf16", True),    # e = 1536: column halves per XCD, ragged last token tile
    (2, 512, 128, 1536, 128, 128, "f32", True),    # e = 1536 in fp32, four token tiles
    (1, 512, 256, 2048, 128, 128, "bf16", True),   # e = 2048: column quarters per XCD, two token tiles
    (1, 768, 128, 2048, 128, 128, "f32", False),   # e = 2048, three token tiles (the generic order)
    (1, 256, 2048, 4096, 128, 64, "bf16", True),   # wide layer: K = 2048 projection, 256-feature output tiles
    (1, 128, 1024, 3072, 256, 64, "f32", False),   # wide fp32 layer, s = 256, one token tile
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}".format(
    *c[:7], "causal" if c[7] else "full"))
def test_layer_matches_oracle(case):
    B, T, d, e, s, C, dtype, causal = case
    inp = make(B, T, d, e, s, C, dtype, seed=B * 7919 + T + C)
    O, ws, cfg, L = run_layer(inp, B, T, d, e, s, C, causal, dtype, stagewise=True)
    ref, im = oracle_layer(inp, C, causal, intermediates=True)
    _stagewise(ws, L, im, B, T, e, s, C, causal, dtype)
    assert_close(O, ref, tol_for(dtype), "O")


WIDE = [
    # B, T, d, e, s, C, dtype, causal, with gamma ~ N(1, 0.5^2), beta ~ N(0, 0.3^2):
    # every offset moves the output, so a dropped or misplaced +beta (or a mix-up
    # of two heads' scales) in the Z epilogues fails the gate
    (1, 256, 128, 256, 128, 64, "f32", True),      # Z tiles of their own (e < 1024), s = 128
    (2, 512, 256, 512, 128, 128, "bf16", False),
    (1, 512, 256, 512, 256, 256, "bf16", True),    # Z tiles, s = 256
    (1, 256, 128, 256, 256, 128, "f32", False),
    (1, 256, 128, 1024, 128, 64, "f32", True),     # Z formed inside the U tiles, s = 128
    (1, 320, 256, 1024, 256, 64, "bf16", False),   # ... s = 256, ragged row tile
    (1, 256, 128, 1024, 256, 128, "f32", True),
    (1, 960, 128, 1536, 128, 64, "bf16", True),    # e = 1536 mapping
    (1, 768, 128, 2048, 128, 128, "f32", False),   # e = 2048, generic order
    (1, 512, 256, 2048, 128, 128, "bf16", True),   # e = 2048 mapping
]


@pytest.mark.parametrize("case", WIDE, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}".format(
    *c[:7], "causal" if c[7] else "full"))
def test_layer_with_offsets_matches_oracle(case):
    B, T, d, e, s, C, dtype, causal = case
    inp = make(B, T, d, e, s, C, dtype, seed=B * 4111 + T + C, heads="wide")
    O, ws, cfg, L = run_layer(inp, B, T, d, e, s, C, causal, dtype, stagewise=True)
    ref, im = oracle_layer(inp, C, causal, intermediates=True)
    _stagewise(ws, L, im, B, T, e, s, C, causal, dtype)
    assert_close(O, ref, tol_for(dtype), "O")
    # the offsets are not vacuous: the same layer without them differs by far
    # more than the tolerance
    ref0 = oracle_layer(dict(inp, beta=np.zeros_like(inp["beta"])), C, causal)
    assert np.max(np.abs(ref0 - ref)) > 10 * tol_for(dtype) * np.max(np.abs(ref))


ROPE = [
    # B, T, d, e, s, C, dtype, causal: heads rotated by position (Z tiles, Z in U tiles, s = 256)
    (1, 512, 128, 256, 128, 128, "f32", True),
    (2, 256, 128, 1024, 128, 64, "bf16", True),
    (1, 320, 256, 1024, 256, 64, "bf16", False),
    (1, 1024, 256, 512, 128, 512, "bf16", True),
    (1, 512, 256, 512, 256, 128, "f32", True),     # Z tile with s = 256
    (1, 960, 128, 1536, 128, 64, "bf16", False),   # e = 1536 mapping, ragged last token tile
]


@pytest.mark.parametrize("heads", ["workload", "wide"])
@pytest.mark.parametrize("case", ROPE, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}".format(
    *c[:7], "causal" if c[7] else "full"))
def test_layer_with_rope_matches_oracle(case, heads):
    B, T, d, e, s, C, dtype, causal = case
    inp = make(B, T, d, e, s, C, dtype, seed=B * 613 + T + C, heads=heads)
    O, ws, cfg, L = run_layer(inp, B, T, d, e, s, C, causal, dtype, rope=True, stagewise=True)
    ref, im = oracle_layer(inp, C, causal, intermediates=True, rope=True)
    _stagewise(ws, L, im, B, T, e, s, C, causal, dtype)
    assert_close(O, ref, tol_for(dtype), "O")


@pytest.mark.parametrize("parts", ["local", "global"])
@pytest.mark.parametrize("case", [(2, 512, 256, 512, 128, 128, "bf16", True), (1, 256, 128, 256, 128, 64, "f32", False),
                                  (1, 256, 128, 1024, 256, 128, "bf16", True)],
                         ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}".format(*c[:7], "causal" if c[7] else "full"))
def test_local_only_and_global_only_match_oracle(case, parts):
    """The LocalOnly / GlobalOnly variants: only that term reaches Y."""
    B, T, d, e, s, C, dtype, causal = case
    inp = make(B, T, d, e, s, C, dtype, seed=B * 211 + T + C)
    O, ws, cfg, L = run_layer(inp, B, T, d, e, s, C, causal, dtype, parts=parts)
    ref, im = oracle_layer(inp, C, causal, intermediates=True, parts=parts)
    assert_close(ws_array(ws, L, "Y", (B, T, e), dtype), im["Y"], tol_for(dtype), "Y")
    assert_close(O, ref, tol_for(dtype), "O")


@pytest.mark.parametrize("n", [64, 512, 1024])
def test_rope_relpos_matches_code4_toeplitz(n):
    """The 2n-1 vector from the kernel against the oracle's Toeplitz matrix
    of Code 4's RoPE branch (first row and column)."""
    rng = np.random.default_rng(n)
    a = (0.3 * rng.standard_normal(128)).astype(np.float32)
    b = (0.3 * rng.standard_normal(128)).astype(np.float32)
    w = g.rope_relpos(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), n)
    torch.cuda.synchronize()
    ref = orc.rope_relpos(a, b, n)
    assert_close(w.cpu().numpy().astype(np.float64), ref, 1e-5, "relpos")


def test_tiny_fp32_workload():
    cfg, inp = inputs.workload_inputs("layer_fp32_B1_T256_d128_C64")
    O, *_ = run_layer(inp, cfg["B"], cfg["T"], cfg["d"], cfg["e"], cfg["s"], cfg["C"], cfg["causal"],
                      cfg["dtype"])
    ref = oracle_layer(inp, cfg["C"], cfg["causal"])
    assert_close(O, ref, 1e-4, "O")


@pytest.mark.parametrize("scales", [(1.0, 1.0), (0.05, 0.3)])
def test_equation_scaling_reading(scales):
    qs, ls = scales
    B, T, d, e, s, C = 1, 512, 256, 512, 128, 128
    inp = make(B, T, d, e, s, C, "bf16", seed=5)
    O, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16", qs, ls)
    assert_close(O, oracle_layer(inp, C, True, qs, ls), 2e-2, "O")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_attention_is_glu(dtype):
    """gamma = beta = 0 and relpos = one-hot at C-1: the layer is a GLU."""
    B, T, d, e, s, C = 1, 256, 128, 256, 128, 64
    inp = make(B, T, d, e, s, C, dtype, seed=9)
    inp["gamma"][:] = 0
    inp["beta"][:] = 0
    inp["relpos"][:] = 0
    inp["relpos"][C - 1] = 1.0
    O, *_ = run_layer(inp, B, T, d, e, s, C, True, dtype)
    ref = orc.glu(inp["X"], inp["W_u"], inp["W_v"], inp["W_o"])
    assert_close(O, ref, tol_for(dtype), "O vs GLU")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causal_output_ignores_future_bitwise(dtype):
    B, T, d, e, s, C = 2, 512, 256, 512, 128, 128
    inp = make(B, T, d, e, s, C, dtype, seed=21)
    a, *_ = run_layer(inp, B, T, d, e, s, C, True, dtype)
    for t in (127, 200):
        q = dict(inp)
        q["X"] = inp["X"].copy()
        q["X"][:, t + 1:] = np.random.default_rng(t).standard_normal(q["X"][:, t + 1:].shape)
        if dtype == "bf16":
            q["X"] = inputs.round_bf16(q["X"].astype(np.float32))
        b, *_ = run_layer(q, B, T, d, e, s, C, True, dtype)
        np.testing.assert_array_equal(a[:, :t + 1], b[:, :t + 1])
        assert np.max(np.abs(a[:, t + 1:] - b[:, t + 1:])) > 0


def test_runs_are_bitwise_deterministic():
    B, T, d, e, s, C = 2, 512, 256, 512, 128, 128
    inp = make(B, T, d, e, s, C, "bf16", seed=33)
    a, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16")
    b, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16")
    np.testing.assert_array_equal(a, b)


def test_local_only_and_global_only_components():
    """The quadratic and linear parts, each alone, meet the same tolerance
    (the global gate alone would not see an error in a small part)."""
    B, T, d, e, s, C = 1, 1024, 256, 512, 128, 256
    base = make(B, T, d, e, s, C, "bf16", seed=41)
    loc = {k: v.copy() for k, v in base.items()}
    loc["gamma"][2] = 0
    loc["beta"][2] = 0
    O, *_ = run_layer(loc, B, T, d, e, s, C, True, "bf16")
    assert_close(O, oracle_layer(loc, C, True), 2e-2, "LocalOnly")
    glo = {k: v.copy() for k, v in base.items()}
    glo["gamma"][0] = 0
    glo["beta"][0] = 0
    glo["relpos"] = -np.abs(glo["relpos"]) - 0.01
    O, *_ = run_layer(glo, B, T, d, e, s, C, True, "bf16")
    assert_close(O, oracle_layer(glo, C, True), 2e-2, "GlobalOnly")


def test_batch_rows_independent_on_gpu():
    B, T, d, e, s, C = 3, 256, 128, 256, 128, 64
    inp = make(B, T, d, e, s, C, "bf16", seed=45)
    full, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16")
    one = dict(inp, X=inp["X"][1:2].copy())
    row, *_ = run_layer(one, 1, T, d, e, s, C, True, "bf16")
    np.testing.assert_array_equal(full[1:2], row)


# ------------------------------------------------------------------ full-size workloads

FULL = ["layer_bf16_B8_T1024_d768_C256", "layer_bf16_B4_T4096_d768_C256",
        "layer_bf16_B4_T4096_d768_C256_noncausal", "layer_bf16_B2_T8192_d768_C512",
        "layer_bf16_B2_T8192_d768_C256"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    """The benchmark's launch configuration at full size.  The oracle checks
    batch row 0 (rows are independent: pinned in the oracle tests and checked
    on the GPU above) and, for B <= 2 or B * T <= 8192, every row.  Besides
    the global gate, every chunk is gated relative to its own largest value:
    in a causal layer the linear term grows with the chunk index, so the
    global gate alone cannot see an error confined to early chunks."""
    cfg, inp = inputs.workload_inputs(name)
    B, T, d, e, s, C = (cfg[k] for k in ("B", "T", "d", "e", "s", "C"))
    print(f"{name}: GPU run", flush=True)
    O, *_ = run_layer(inp, B, T, d, e, s, C, cfg["causal"], "bf16")
    assert np.all(np.isfinite(O))
    rows = range(B) if B <= 2 else [0]
    if B > 2 and B * T <= 8192:
        rows = range(B)
    for b in rows:
        one = dict(inp, X=inp["X"][b:b + 1])
        ref = oracle_layer(one, C, cfg["causal"])
        err = assert_close(O[b:b + 1], ref, 2e-2, f"{name} row {b}")
        ce = chunk_errors(O[b:b + 1], ref, C)
        print(f"{name} row {b}: global {err:.2e}, worst per-chunk {ce.max():.2e} (chunk {int(ce.argmax())})",
              flush=True)
        assert ce.max() <= 2e-2, f"{name} row {b} chunk {int(ce.argmax())}: {ce.max():.3e}"


@pytest.mark.parametrize("parts", ["local", "global"])
def test_benchmark_workload_parts(parts):
    """LocalOnly and GlobalOnly at the benchmark shape (B=2, T=8192, d=768,
    C=256): the quadratic part, which the linear term dwarfs in late chunks
    of the full layer, under the gate on its own, and the linear part alone."""
    name = "layer_bf16_B2_T8192_d768_C256"
    cfg, inp = inputs.workload_inputs(name)
    B, T, d, e, s, C = (cfg[k] for k in ("B", "T", "d", "e", "s", "C"))
    print(f"{name} {parts}: GPU run", flush=True)
    O, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16", parts=parts)
    ref = oracle_layer(inp, C, True, parts=parts)
    err = assert_close(O, ref, 2e-2, f"{name} {parts}")
    ce = chunk_errors(O, ref, C)
    print(f"{name} {parts}: global {err:.2e}, worst per-chunk {ce.max():.2e}", flush=True)
    assert ce.max() <= 2e-2, f"chunk {int(ce.argmax())}: {ce.max():.3e}"


# ------------------------------------------------------------------ large sizes

def test_long_sequence():
    """B=1, T=131072 (512 chunks, 128 x the benchmark's chunk count per
    sequence): every token against the oracle, and every chunk under the gate
    relative to its own largest value."""
    B, T, d, e, s, C = 1, 131072, 768, 1536, 128, 256
    inp = make(B, T, d, e, s, C, "bf16", seed=77)
    print("T=131072: GPU run", flush=True)
    O, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16")
    assert np.all(np.isfinite(O))
    print("T=131072: oracle", flush=True)
    ref = oracle_layer(inp, C, True)
    err = assert_close(O, ref, 2e-2, "T=131072")
    ce = chunk_errors(O, ref, C)
    print(f"T=131072: global {err:.2e}, worst per-chunk {ce.max():.2e} (chunk {int(ce.argmax())})", flush=True)
    assert ce.max() <= 2e-2, f"chunk {int(ce.argmax())}: {ce.max():.3e}"


def test_longest_bf16_sequence():
    """T = 2^22 tokens, the longest sequence bf16 takes (the matrix cores'
    buffer copies address up to 255 rows of T-element token runs with 32-bit
    offsets: 255 * 2^23 bytes at the farthest).  No oracle pass over 4M tokens;
    instead properties that hold at any length, compared bitwise between GPU
    runs: LocalOnly, a chunk's output depends on its own tokens only, so the
    first and last chunks equal forwards of those chunks alone; the full
    layer's first two chunks equal a forward of those two chunks (causality).
    The short forwards are checked against the oracle, and every output of the
    long ones is finite."""
    B, T, d, e, s, C = 1, 1 << 22, 128, 256, 128, 256
    inp = make(B, C, d, e, s, C, "bf16", seed=91)  # the weights (and one chunk of X, unused)
    dev = g.device_layer(inp, torch.bfloat16)
    W = [dev[k] for k in ("W_u", "W_v", "W_z", "W_o", "scale", "offset", "relpos")]
    # X ~ N(0, 1) drawn on the device; the oracle takes the same values
    X = inputs.device_normal_bf16((B, T, d), seed=91)

    def forward(t0, n, parts):
        cfg = g.make_config(B, n, d, e, s, C, True, g.GAU_BF16, parts=parts)
        ws = torch.empty(g.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
        O = torch.empty((B, n, d), dtype=torch.bfloat16, device="cuda")
        g.forward(cfg, X[:, t0:t0 + n].contiguous(), *W, O, ws)
        torch.cuda.synchronize()
        del ws
        return O

    def short_ref(t0, n, parts):
        one = dict(inp, X=X[:, t0:t0 + n].float().cpu().numpy().astype(np.float64))
        return oracle_layer(one, C, True, parts=parts)

    print("T=2^22 LocalOnly: GPU run", flush=True)
    O = forward(0, T, "local")
    assert bool(torch.isfinite(O).all())
    for t0 in (0, T - C):
        Oc = forward(t0, C, "local")
        assert torch.equal(O[:, t0:t0 + C], Oc), f"LocalOnly chunk at {t0}"
        assert_close(Oc.float().cpu().numpy().astype(np.float64), short_ref(t0, C, "local"), 2e-2,
                     f"LocalOnly chunk at {t0}")
    del O
    torch.cuda.empty_cache()
    print("T=2^22 full layer: GPU run", flush=True)
    O = forward(0, T, "both")
    assert bool(torch.isfinite(O).all())
    O2 = forward(0, 2 * C, "both")
    assert torch.equal(O[:, :2 * C], O2), "the first two chunks"
    assert_close(O2.float().cpu().numpy().astype(np.float64), short_ref(0, 2 * C, "both"), 2e-2,
                 "the first two chunks")


def test_many_sequences_checked_on_first_and_last_rows():
    """B=64, T=1024: 65536 tokens in 64 independent rows; rows 0 and 63
    against the oracle."""
    B, T, d, e, s, C = 64, 1024, 768, 1536, 128, 256
    inp = make(B, T, d, e, s, C, "bf16", seed=78)
    O, *_ = run_layer(inp, B, T, d, e, s, C, True, "bf16")
    for b in (0, B - 1):
        ref = oracle_layer(dict(inp, X=inp["X"][b:b + 1]), C, True)
        assert_close(O[b:b + 1], ref, 2e-2, f"row {b} of B=64")


def _random_configs(n, seed):
    """n layer configurations drawn from the ABI's valid ranges (sizes kept
    small enough for the oracle): batch, chunk, chunks per sequence, widths,
    storage type, mask, RoPE, ablation and head parameters all vary."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        C = int(rng.choice([64, 128, 256, 512]))
        G = int(rng.integers(1, 5 if C <= 128 else 3))
        out.append(dict(B=int(rng.integers(1, 4)), T=C * G, d=128 * int(rng.integers(1, 5)),
                        e=256 * int(rng.integers(1, 9)), s=int(rng.choice([128, 256])), C=C,
                        dtype=str(rng.choice(["f32", "bf16"])), causal=bool(rng.integers(0, 2)),
                        rope=bool(rng.integers(0, 2)), parts=str(rng.choice(["both", "local", "global"])),
                        heads=str(rng.choice(["workload", "wide"]))))
    return out


RANDOM = _random_configs(16, seed=4242)


@pytest.mark.parametrize("k", range(len(RANDOM)), ids=lambda k: "B{B}_T{T}_d{d}_e{e}_s{s}_C{C}_{dtype}_{causal}_"
                         "rope{rope}_{parts}_{heads}".format(**RANDOM[k]))
def test_random_configurations_match_oracle(k):
    """Seeded random configurations across every option the layer has,
    output against the oracle under the storage type's gate."""
    c = RANDOM[k]
    B, T, d, e, s, C, dtype, causal = (c[x] for x in ("B", "T", "d", "e", "s", "C", "dtype", "causal"))
    inp = make(B, T, d, e, s, C, dtype, seed=9000 + k, heads=c["heads"])
    O, _, _, _ = run_layer(inp, B, T, d, e, s, C, causal, dtype, rope=c["rope"], parts=c["parts"])
    ref = oracle_layer(inp, C, causal, rope=c["rope"], parts=c["parts"])
    assert_close(O, ref, tol_for(dtype), "O")
