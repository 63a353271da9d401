"""GPU parity of the layer's gradients: gau_backward against the float64
oracle's chain rule (oracle.flash_backward, itself pinned against central
differences of the brute-force forward), every gradient element by element."""

import numpy as np
import pytest
import torch

import chunked_linear_attention_amd as g
from chunked_linear_attention_amd import inputs
from oracle import gau_oracle as orc

from _gpu import assert_close, make, tol_for, torch_dtype

pytestmark = pytest.mark.gpu


def _backward(inp, dO, B, T, d, e, s, C, causal, dtype, fill=0, rope=False, parts="both", seg=None):
    tdt = torch_dtype(dtype)
    dev = g.device_layer(inp, tdt)
    cfg = g.make_config(B, T, d, e, s, C, causal, g.GAU_BF16 if dtype == "bf16" else g.GAU_F32, rope=rope,
                        parts=parts)
    ws = torch.full((g.backward_workspace_bytes(cfg),), fill, dtype=torch.uint8, device="cuda")
    dOd = g.device_tensor(dO, tdt)
    like = {"X": (B, T, d), "W_u": (e, d), "W_v": (e, d), "W_z": (s, d), "W_o": (d, e), "scale": (4, s),
            "offset": (4, s), "relpos": (2 * C - 1,)}
    grads = {k: torch.full(like[k], float("nan"), dtype=torch.float32, device="cuda") for k in g.GRAD_NAMES}
    sg = None if seg is None else torch.from_numpy(np.ascontiguousarray(seg, dtype=np.int32)).cuda()
    g.backward(cfg, dev["X"], dev["W_u"], dev["W_v"], dev["W_z"], dev["W_o"], dev["scale"], dev["offset"],
               dev["relpos"], dOd, grads, ws, chunk_segments=sg)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.float64) for k, v in grads.items()}


def _oracle(inp, dO, C, causal, rope=False, parts="both", seg=None):
    r = orc.flash_backward(inp["X"], inp["W_u"], inp["W_v"], inp["W_z"], inp["W_o"], inp["gamma"], inp["beta"],
                           inp["relpos"], C, causal, dO, use_rope=rope, parts=parts, chunk_segments=seg)
    # the library returns weight gradients output-major, like the weights it takes
    return {"X": r["X"], "W_u": r["W_u"].T, "W_v": r["W_v"].T, "W_z": r["W_z"].T, "W_o": r["W_o"].T,
            "scale": r["gamma"], "offset": r["beta"], "relpos": r["relpos"]}


def _compare(got, ref, dtype):
    for k in g.GRAD_NAMES:
        assert np.all(np.isfinite(got[k])), f"d{k} has non-finite entries"
        if not np.any(ref[k]):   # a gradient the layer's dropped term alone would carry
            assert not np.any(got[k]), f"d{k} should be zero"
            continue
        assert_close(got[k], ref[k], tol_for(dtype), f"d{k}")


CASES = [
    # B, T, d, e, s, C, dtype, causal
    (1, 256, 128, 256, 128, 64, "f32", True),
    (1, 256, 128, 256, 128, 64, "f32", False),
    (2, 512, 256, 512, 128, 128, "bf16", True),
    (1, 512, 256, 512, 256, 256, "bf16", False),
    (1, 1024, 256, 512, 128, 512, "bf16", True),    # the largest chunk
    (3, 192, 384, 768, 128, 64, "bf16", True),      # three chunks per sequence, d and e not powers of two
    (1, 320, 128, 1024, 256, 64, "f32", False),
    # gamma ~ N(1, 0.5^2), beta ~ N(0, 0.3^2): the heads' offsets count
    (1, 256, 128, 256, 128, 64, "f32", True, "wide"),
    (2, 512, 256, 512, 128, 128, "bf16", False, "wide"),
    (1, 320, 128, 1024, 256, 64, "bf16", True, "wide"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}{}".format(
    *c[:7], "causal" if c[7] else "full", "_wide" if len(c) > 8 else ""))
def test_backward_matches_oracle(case):
    B, T, d, e, s, C, dtype, causal = case[:8]
    heads = case[8] if len(case) > 8 else "workload"
    print(f"backward case {case}", flush=True)
    inp = make(B, T, d, e, s, C, dtype, seed=B * 131 + T + C, heads=heads)
    dO = inputs.make_output_grad(B, T, d, seed=T + d, dtype=dtype)
    _compare(_backward(inp, dO, B, T, d, e, s, C, causal, dtype), _oracle(inp, dO, C, causal), dtype)


ROPE_CASES = [
    # B, T, d, e, s, C, dtype, causal, heads: the four heads rotated by position
    (1, 256, 128, 256, 128, 64, "f32", True, "wide"),
    (2, 512, 256, 512, 128, 128, "bf16", False, "wide"),
    (1, 512, 256, 512, 256, 256, "f32", True, "wide"),     # s = 256
    (1, 960, 128, 1536, 128, 64, "bf16", True, "wide"),    # e >= 1024: heads formed inside the U tiles
]


@pytest.mark.parametrize("case", ROPE_CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}_rope".format(
    *c[:7], "causal" if c[7] else "full"))
def test_backward_with_rope_matches_oracle(case):
    B, T, d, e, s, C, dtype, causal, heads = case
    print(f"backward rope case {case}", flush=True)
    inp = make(B, T, d, e, s, C, dtype, seed=B * 97 + T + C, heads=heads)
    dO = inputs.make_output_grad(B, T, d, seed=T + 3 * d, dtype=dtype)
    _compare(_backward(inp, dO, B, T, d, e, s, C, causal, dtype, rope=True), _oracle(inp, dO, C, causal, rope=True),
             dtype)


def test_backward_with_rope_at_benchmark_shape():
    """B=2, T=8192 (angles up to 8191 rad), d=768, e=1536, bf16, causal, RoPE."""
    B, T, d, e, s, C = 2, 8192, 768, 1536, 128, 256
    print("backward rope benchmark shape", flush=True)
    inp = make(B, T, d, e, s, C, "bf16", seed=2025, heads="wide")
    dO = inputs.make_output_grad(B, T, d, seed=2025, dtype="bf16")
    _compare(_backward(inp, dO, B, T, d, e, s, C, True, "bf16", rope=True), _oracle(inp, dO, C, True, rope=True),
             "bf16")


PARTS_CASES = [
    # B, T, d, e, s, C, dtype, causal
    (1, 256, 128, 256, 128, 64, "f32", True),
    (2, 512, 256, 512, 128, 128, "bf16", False),
    (1, 960, 128, 1536, 128, 64, "bf16", True),
]


@pytest.mark.parametrize("parts", ["local", "global"])
@pytest.mark.parametrize("case", PARTS_CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}".format(
    *c[:7], "causal" if c[7] else "full"))
def test_backward_of_one_part_matches_oracle(case, parts):
    """LocalOnly / GlobalOnly: the kept term's gradients, and exact zeros for
    the parameters only the dropped term uses."""
    B, T, d, e, s, C, dtype, causal = case
    print(f"backward {parts} case {case}", flush=True)
    inp = make(B, T, d, e, s, C, dtype, seed=B * 61 + T + C, heads="wide")
    dO = inputs.make_output_grad(B, T, d, seed=T + 5 * d, dtype=dtype)
    _compare(_backward(inp, dO, B, T, d, e, s, C, causal, dtype, parts=parts),
             _oracle(inp, dO, C, causal, parts=parts), dtype)


SEG_CASES = [
    # B, T, d, e, s, C, dtype, causal, longest segment (chunks)
    (1, 512, 128, 256, 128, 64, "f32", True, 3),
    (2, 512, 128, 256, 128, 64, "f32", False, 3),
    (2, 1024, 256, 512, 128, 128, "bf16", True, 2),
    (1, 960, 128, 1536, 128, 64, "bf16", False, 4),
]


def _runs(rng, B, G, max_run):
    """Per-row chunk ids: runs of 1..max_run chunks, ids increasing."""
    seg = np.zeros((B, G), np.int32)
    for b in range(B):
        g0, sid = 0, 0
        while g0 < G:
            n = int(rng.integers(1, max_run + 1))
            seg[b, g0:g0 + n] = sid
            g0, sid = g0 + n, sid + 1
    return seg


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}_seg{}".format(
    *c[:7], "causal" if c[7] else "full", c[8]))
def test_backward_with_segments_matches_oracle(case):
    """gau_backward_segmented: packed sequences, every gradient."""
    B, T, d, e, s, C, dtype, causal, max_run = case
    print(f"backward segments case {case}", flush=True)
    seg = _runs(np.random.default_rng(T + C + max_run), B, T // C, max_run)
    inp = make(B, T, d, e, s, C, dtype, seed=B * 53 + T + C, heads="wide")
    dO = inputs.make_output_grad(B, T, d, seed=T + 7 * d, dtype=dtype)
    _compare(_backward(inp, dO, B, T, d, e, s, C, causal, dtype, seg=seg), _oracle(inp, dO, C, causal, seg=seg),
             dtype)


def test_backward_with_segments_at_benchmark_shape():
    """B=2, T=8192 packed with documents of 1..8 chunks, bf16, causal."""
    B, T, d, e, s, C = 2, 8192, 768, 1536, 128, 256
    print("backward segments benchmark shape", flush=True)
    seg = _runs(np.random.default_rng(11), B, T // C, 8)
    inp = make(B, T, d, e, s, C, "bf16", seed=2026)
    dO = inputs.make_output_grad(B, T, d, seed=2026, dtype="bf16")
    _compare(_backward(inp, dO, B, T, d, e, s, C, True, "bf16", seg=seg), _oracle(inp, dO, C, True, seg=seg), "bf16")


@pytest.mark.parametrize("B,T,causal", [(4, 4096, False), (8, 1024, True)], ids=["B4_T4096_full", "B8_T1024_causal"])
def test_backward_at_other_full_shapes(B, T, causal):
    """The layer's other full-size shapes (d=768, e=1536, s=128, C=256, bf16):
    B=4 T=4096 non-causal, B=8 T=1024 causal; every gradient."""
    d, e, s, C = 768, 1536, 128, 256
    print(f"backward full shape B{B} T{T} causal={causal}", flush=True)
    inp = make(B, T, d, e, s, C, "bf16", seed=3000 + B, heads="wide")
    dO = inputs.make_output_grad(B, T, d, seed=3000 + T, dtype="bf16")
    _compare(_backward(inp, dO, B, T, d, e, s, C, causal, "bf16"), _oracle(inp, dO, C, causal), "bf16")


def test_backward_at_benchmark_shape():
    """B=2, T=8192, d=768, e=1536, s=128, C=256, bf16, causal: every gradient."""
    B, T, d, e, s, C = 2, 8192, 768, 1536, 128, 256
    print("backward benchmark shape", flush=True)
    inp = make(B, T, d, e, s, C, "bf16", seed=2024)
    dO = inputs.make_output_grad(B, T, d, seed=2024, dtype="bf16")
    _compare(_backward(inp, dO, B, T, d, e, s, C, True, "bf16"), _oracle(inp, dO, C, True), "bf16")


@pytest.mark.parametrize("shape", [(2, 256, 128, 256, 128, 64), (1, 1024, 256, 1536, 128, 256)],
                         ids=["C64", "C256"])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_backward_is_reproducible_and_ignores_workspace_contents(causal, shape):
    """Bitwise equal gradients from a zeroed and from a NaN-filled workspace
    (at C = 256 the causal score tiles above the diagonal are never written:
    nothing may read them unmasked)."""
    B, T, d, e, s, C = shape
    inp = make(B, T, d, e, s, C, "bf16", seed=77)
    dO = inputs.make_output_grad(B, T, d, seed=77, dtype="bf16")
    a = _backward(inp, dO, B, T, d, e, s, C, causal, "bf16", fill=0)
    b = _backward(inp, dO, B, T, d, e, s, C, causal, "bf16", fill=0xFF)
    for k in g.GRAD_NAMES:
        assert np.array_equal(a[k], b[k]), k


def test_backward_without_tokens_zeroes_the_parameter_gradients():
    d, e, s, C = 128, 256, 128, 64
    cfg = g.make_config(0, 256, d, e, s, C, True, g.GAU_BF16)
    grads = {k: torch.full(sh, 5.0, device="cuda") for k, sh in
             {"X": (0, 256, d), "W_u": (e, d), "W_v": (e, d), "W_z": (s, d), "W_o": (d, e), "scale": (4, s),
              "offset": (4, s), "relpos": (2 * C - 1,)}.items()}
    emp = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device="cuda")
    f32 = lambda *sh: torch.zeros(sh, device="cuda")
    g.backward(cfg, emp(0, 256, d), emp(e, d), emp(e, d), emp(s, d), emp(d, e), f32(4, s), f32(4, s),
               f32(2 * C - 1), emp(0, 256, d), grads, torch.empty(1, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    for k in g.GRAD_NAMES[1:]:
        assert torch.count_nonzero(grads[k]).item() == 0, k


def _random_backward_configs(n, seed):
    """n configurations drawn from the valid ranges (sizes kept small enough
    for the oracle's chain rule): every option of the layer varies."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(n):
        C = int(rng.choice([64, 128, 256]))
        out.append(dict(B=int(rng.integers(1, 3)), T=C * int(rng.integers(1, 4)), d=128 * int(rng.integers(1, 3)),
                        e=256 * int(rng.integers(1, 7)), s=int(rng.choice([128, 256])), C=C,
                        dtype=str(rng.choice(["f32", "bf16"])), causal=bool(rng.integers(0, 2)),
                        rope=bool(rng.integers(0, 2)), parts=str(rng.choice(["both", "local", "global"])),
                        heads=str(rng.choice(["workload", "wide"]))))
    return out


RANDOM = _random_backward_configs(10, seed=5151)


@pytest.mark.parametrize("k", range(len(RANDOM)), ids=lambda k: "B{B}_T{T}_d{d}_e{e}_s{s}_C{C}_{dtype}_{causal}_"
                         "rope{rope}_{parts}_{heads}".format(**RANDOM[k]))
def test_random_configurations_backward_matches_oracle(k):
    """Seeded random configurations: every gradient against the oracle's."""
    c = RANDOM[k]
    B, T, d, e, s, C, dtype, causal = (c[x] for x in ("B", "T", "d", "e", "s", "C", "dtype", "causal"))
    inp = make(B, T, d, e, s, C, dtype, seed=9500 + k, heads=c["heads"])
    dO = inputs.make_output_grad(B, T, d, seed=9500 + k, dtype=dtype)
    got = _backward(inp, dO, B, T, d, e, s, C, causal, dtype, rope=c["rope"], parts=c["parts"])
    _compare(got, _oracle(inp, dO, C, causal, rope=c["rope"], parts=c["parts"]), dtype)
