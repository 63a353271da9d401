"""The library's kernel sources on the CPU emulation (tests/emu): every access
in bounds, and the results of the emulated kernels equal to the oracle's.

The emulation compiles the same .hip sources for the host, so these tests
check the kernels' addressing, barriers, copy waits and MFMA operand layouts
without a GPU.  They do not replace the GPU parity tests: the compiler's
device code and the hardware are not exercised.
"""

import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "emu"))

emu_build = pytest.importorskip("emu_build", reason="tests/emu is not present")

from chunked_linear_attention_amd import inputs  # noqa: E402
from chunked_linear_attention_amd._lib import GauConfig, GauWsLayout  # noqa: E402
from oracle import gau_oracle as orc  # noqa: E402

pytestmark = pytest.mark.skipif(not emu_build.available(), reason="host clang++ of ROCm not found")


@pytest.fixture(scope="module")
def emu():
    emu_build.build()
    lib = ctypes.CDLL(emu_build.LIB)
    P = ctypes.c_void_p
    lib.gau_workspace_bytes.restype = ctypes.c_size_t
    lib.gau_workspace_bytes.argtypes = [ctypes.POINTER(GauConfig)]
    lib.gau_workspace_layout.argtypes = [ctypes.POINTER(GauConfig), ctypes.POINTER(GauWsLayout)]
    lib.gau_forward.argtypes = [ctypes.POINTER(GauConfig)] + [P] * 9 + [P, ctypes.c_size_t, P]
    lib.gau_forward.restype = ctypes.c_int
    lib.gau_forward_stages.argtypes = [ctypes.POINTER(GauConfig), ctypes.c_int, ctypes.c_int] + [P] * 9 + \
        [P, ctypes.c_size_t, P]
    lib.gau_forward_stages.restype = ctypes.c_int
    lib.emu_set_mode.argtypes = [ctypes.c_int, ctypes.c_int]
    return lib


def _bounds(which):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([emu_build.BOUNDS, which], capture_output=True, text=True, env=env, timeout=900)
    assert r.returncode == 0 and "all launches in bounds" in r.stderr, r.stderr[-4000:]


def test_every_launch_in_bounds_at_test_shapes(emu):
    """All kernels at the shapes the parity tests use (ragged tiles, every C
    and s, fp32 and bf16, causal and not): each operand in its own exact-size
    buffer under AddressSanitizer."""
    _bounds("small")


def test_every_launch_in_bounds_at_benchmark_shape(emu):
    """The same at B=2, T=8192, d=768, e=1536, s=128, C=256."""
    _bounds("headline")


CASES = [
    # B, T, d, e, s, C, dtype, causal
    (1, 256, 128, 256, 128, 64, "f32", True),
    (1, 256, 128, 256, 128, 64, "f32", False),
    (1, 320, 128, 256, 128, 64, "bf16", True),
    (2, 256, 256, 512, 128, 128, "bf16", True),
    (1, 512, 128, 256, 256, 256, "bf16", False),
    (1, 512, 128, 256, 128, 512, "bf16", True),
    (1, 256, 128, 1024, 128, 64, "f32", True),      # Z formed inside the U tiles (s = 128)
    (1, 256, 128, 1024, 256, 128, "bf16", False),   # Z formed inside the U tiles (s = 256)
    (1, 1024, 128, 1536, 128, 256, "bf16", True),   # e = 1536: tiles spread over the XCDs by column halves
    (1, 512, 128, 2048, 128, 128, "bf16", True),    # e = 2048: column quarters per XCD
    (1, 256, 128, 256, 128, 64, "f32", True, True),   # heads rotated by position (RoPE)
    (1, 256, 128, 1024, 256, 128, "bf16", True, True),
    (1, 256, 128, 256, 128, 64, "f32", True, False, "local"),     # LocalOnly / GlobalOnly variants
    (1, 256, 128, 1024, 256, 128, "bf16", False, False, "global"),
    # gamma ~ N(1, 0.5^2), beta ~ N(0, 0.3^2): the offsets count (Z tiles and Z in U tiles, s = 128 and 256)
    (1, 256, 128, 256, 128, 64, "f32", True, False, "both", "wide"),
    (1, 256, 128, 256, 256, 128, "bf16", False, False, "both", "wide"),
    (1, 256, 128, 1024, 128, 64, "bf16", True, False, "both", "wide"),
    (1, 256, 128, 1024, 256, 128, "f32", False, True, "both", "wide"),
    (1, 320, 128, 256, 256, 64, "bf16", True, True, "both", "wide"),   # Z tile with s = 256, rotated, ragged
]


def _host(a, bf):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return inputs.bf16_bits(a) if bf else a


@pytest.mark.parametrize("late", [0, 1], ids=["dma_at_issue", "dma_at_wait"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}{}{}{}".format(
    *c[:7], "causal" if c[7] else "full", "_rope" if len(c) > 8 and c[8] else "",
    "_" + c[9] if len(c) > 9 else "", "_wide" if len(c) > 10 else ""))
def test_emulated_kernels_match_oracle(emu, case, late):
    B, T, d, e, s, C, dtype, causal = case[:8]
    rope = len(case) > 8 and case[8]
    parts = case[9] if len(case) > 9 else "both"
    heads = case[10] if len(case) > 10 else "workload"
    bf = dtype == "bf16"
    emu.emu_set_mode(1, late)
    inp = inputs.make_layer_inputs(B=B, T=T, d=d, e=e, s=s, C=C, seed=B * 31 + T + C, dtype=dtype, heads=heads)
    cfg = GauConfig(B, T, d, e, s, C, 1 if causal else 0, 1 if bf else 0, 1.0 / C, 1.0 / C, 1 if rope else 0,
                    {"both": 0, "local": 1, "global": 2}[parts])
    X = _host(inp["X"], bf)
    W = {k: _host(np.ascontiguousarray(inp[k].T), bf) for k in ("W_u", "W_v", "W_z", "W_o")}
    sc, of, rp = (np.ascontiguousarray(inp[k], np.float32) for k in ("gamma", "beta", "relpos"))
    O = np.zeros((B, T, d), np.uint16 if bf else np.float32)
    wsb = emu.gau_workspace_bytes(ctypes.byref(cfg))
    raw = np.zeros(wsb + 256, np.uint8)
    ws = raw[(-raw.ctypes.data) % 256:][:wsb]
    ptr = lambda a: ctypes.c_void_p(a.ctypes.data)
    # the forward in two ranges, so that U and S can be read before the
    # attention stage gates U into Y in place and the scan turns S into P
    args = (ptr(X), ptr(W["W_u"]), ptr(W["W_v"]), ptr(W["W_z"]), ptr(W["W_o"]), ptr(sc), ptr(of), ptr(rp), ptr(O),
            ptr(ws), wsb, None)
    assert emu.gau_forward_stages(ctypes.byref(cfg), 0, 2, *args) == 0
    early = ws.copy()
    assert emu.gau_forward_stages(ctypes.byref(cfg), 3, 5, *args) == 0
    L = GauWsLayout()
    assert emu.gau_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)) == 0
    ref, im = orc.flash_forward(inp["X"], inp["W_u"], inp["W_v"], inp["W_z"], inp["W_o"], inp["gamma"],
                                inp["beta"], inp["relpos"], C, causal, return_intermediates=True, use_rope=rope,
                                parts=parts)
    conv = inputs.bf16_bits_to_f32 if bf else (lambda a: a)
    eb = 2 if bf else 4

    def region(name, shape):
        n = int(np.prod(shape))
        o = getattr(L, name)
        src = early if name in ("U", "S") else ws
        return conv(src[o:o + eb * n].view(np.uint16 if bf else np.float32).reshape(shape)).astype(np.float64)

    tol = 2e-2 if bf else 1e-4
    G = T // C
    checks = {
        "U": (region("U", (B, T, e)), im["U"]),
        "Vt": (region("Vt", (B, e, T)), im["V"].transpose(0, 2, 1)),
        "Q_quad": (region("Q_quad", (B, T, s)), im["Q_quad"]),
        "K_quad": (region("K_quad", (B, T, s)), im["K_quad"]),
        "Q_lin": (region("Q_lin", (B, T, s)), im["Q_lin"]),
        "K_lin_t": (region("K_lin_t", (B, s, T)), im["K_lin"].transpose(0, 2, 1)),
        "S": (region("S", (B, G, e, s)), im["S"].transpose(0, 1, 3, 2)),
        "Y": (region("Y", (B, T, e)), im["Y"]),
        "O": (conv(O).astype(np.float64), ref),
    }
    if parts == "local":
        del checks["S"]  # the state stages queue nothing
    for name, (got, want) in checks.items():
        assert np.all(np.isfinite(got)), name
        err = np.max(np.abs(got - want)) / np.max(np.abs(want))
        assert err <= tol, f"{name}: {err:.3e} > {tol}"


SEG_CASES = [
    # B, T, d, e, s, C, dtype, causal, per-row chunk ids
    (1, 512, 128, 256, 128, 64, "f32", True, [[0, 0, 0, 1, 1, 2, 2, 2]]),
    (2, 512, 128, 256, 128, 128, "bf16", False, [[5, 5, 6, 6], [1, 2, 2, 1]]),
    (1, 1024, 128, 1024, 128, 128, "bf16", True, [[0, 1, 1, 1, 0, 0, 3, 3]]),
    (2, 256, 128, 256, 256, 64, "f32", False, [[0, 0, 0, 0], [0, 1, 2, 3]]),
]


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}".format(
    *c[:7], "causal" if c[7] else "full"))
def test_emulated_segmented_layer_matches_oracle(emu, case):
    """gau_forward_segmented on the emulation (copies landing at their waits)
    against the oracle's segment-masked layer: the output and the averaged
    per-chunk states it leaves in the S region."""
    B, T, d, e, s, C, dtype, causal, seg = case
    bf = dtype == "bf16"
    emu.emu_set_mode(1, 1)
    P = ctypes.c_void_p
    emu.gau_forward_segmented.argtypes = [ctypes.POINTER(GauConfig), P] + [P] * 9 + [P, ctypes.c_size_t, P]
    emu.gau_forward_segmented.restype = ctypes.c_int
    inp = inputs.make_layer_inputs(B=B, T=T, d=d, e=e, s=s, C=C, seed=B * 53 + T + C, dtype=dtype, heads="wide")
    cfg = GauConfig(B, T, d, e, s, C, 1 if causal else 0, 1 if bf else 0, 1.0 / C, 1.0 / C, 0, 0)
    X = _host(inp["X"], bf)
    W = {k: _host(np.ascontiguousarray(inp[k].T), bf) for k in ("W_u", "W_v", "W_z", "W_o")}
    sc, of, rp = (np.ascontiguousarray(inp[k], np.float32) for k in ("gamma", "beta", "relpos"))
    segr = np.zeros(len(seg) * len(seg[0]) + 4, np.int32)
    sega = segr[(-segr.ctypes.data) % 16 // 4:][:B * (T // C)].reshape(B, T // C)
    sega[:] = np.array(seg, np.int32)
    O = np.zeros((B, T, d), np.uint16 if bf else np.float32)
    wsb = emu.gau_workspace_bytes(ctypes.byref(cfg))
    raw = np.full(wsb + 256, 0xFF, np.uint8)
    ws = raw[(-raw.ctypes.data) % 256:][:wsb]
    ptr = lambda a: P(a.ctypes.data)
    assert emu.gau_forward_segmented(ctypes.byref(cfg), ptr(sega), ptr(X), ptr(W["W_u"]), ptr(W["W_v"]),
                                     ptr(W["W_z"]), ptr(W["W_o"]), ptr(sc), ptr(of), ptr(rp), ptr(O), ptr(ws),
                                     wsb, None) == 0
    L = GauWsLayout()
    assert emu.gau_workspace_layout(ctypes.byref(cfg), ctypes.byref(L)) == 0
    ref, im = orc.flash_forward(inp["X"], inp["W_u"], inp["W_v"], inp["W_z"], inp["W_o"], inp["gamma"],
                                inp["beta"], inp["relpos"], C, causal, return_intermediates=True,
                                chunk_segments=np.array(seg))
    conv = inputs.bf16_bits_to_f32 if bf else (lambda a: a)
    eb = 2 if bf else 4
    G = T // C
    n = B * G * e * s
    Pg = conv(ws[L.S:L.S + eb * n].view(np.uint16 if bf else np.float32).reshape(B, G, e, s)).astype(np.float64)
    tol = 2e-2 if bf else 1e-4
    for name, got, want in (("P", Pg, im["P"].transpose(0, 1, 3, 2)), ("O", conv(O).astype(np.float64), ref)):
        assert np.all(np.isfinite(got)), name
        err = np.max(np.abs(got - want)) / np.max(np.abs(want))
        assert err <= tol, f"{name}: {err:.3e} > {tol}"


@pytest.mark.parametrize("dtype,B,heads", [("f32", 2, "workload"), ("bf16", 2, "workload"), ("bf16", 18, "workload"),
                                           ("f32", 2, "wide"), ("bf16", 18, "wide")])
def test_emulated_decoding_matches_the_causal_layer(emu, dtype, B, heads):
    """gau_decode_step on the emulation for 66 tokens (one chunk end, C = 64)
    against the oracle's causal layer; B = 18 takes the MFMA products (from B = 9 on);
    "wide": gamma ~ N(1, 0.5^2), beta ~ N(0, 0.3^2)."""
    T, d, e, s, C = 128, 128, 256, 128, 64
    steps = 66
    bf = dtype == "bf16"
    emu.emu_set_mode(1, 1)
    P = ctypes.c_void_p
    emu.gau_decode_workspace_bytes.restype = ctypes.c_size_t
    emu.gau_decode_workspace_bytes.argtypes = [ctypes.POINTER(GauConfig)]
    emu.gau_decode_reset.argtypes = [ctypes.POINTER(GauConfig), P, ctypes.c_size_t, P]
    emu.gau_decode_step.argtypes = [ctypes.POINTER(GauConfig), ctypes.c_int64] + [P] * 10 + [ctypes.c_size_t, P]
    inp = inputs.make_layer_inputs(B=B, T=T, d=d, e=e, s=s, C=C, seed=41, dtype=dtype, heads=heads)
    cfg = GauConfig(B, T, d, e, s, C, 1, 1 if bf else 0, 1.0 / C, 1.0 / C, 1)
    W = {k: _host(np.ascontiguousarray(inp[k].T), bf) for k in ("W_u", "W_v", "W_z", "W_o")}
    sc, of, rp = (np.ascontiguousarray(inp[k], np.float32) for k in ("gamma", "beta", "relpos"))
    wsb = emu.gau_decode_workspace_bytes(ctypes.byref(cfg))
    raw = np.full(wsb + 256, 0xFF, np.uint8)
    ws = raw[(-raw.ctypes.data) % 256:][:wsb]
    ptr = lambda a: P(a.ctypes.data)
    assert emu.gau_decode_reset(ctypes.byref(cfg), ptr(ws), wsb, None) == 0
    conv = inputs.bf16_bits_to_f32 if bf else (lambda a: a)
    got = np.zeros((B, steps, d))
    for t in range(steps):
        x = _host(np.ascontiguousarray(inp["X"][:, t]), bf)
        o = np.zeros((B, d), np.uint16 if bf else np.float32)
        assert emu.gau_decode_step(ctypes.byref(cfg), t, ptr(x), ptr(W["W_u"]), ptr(W["W_v"]), ptr(W["W_z"]),
                                   ptr(W["W_o"]), ptr(sc), ptr(of), ptr(rp), ptr(o), ptr(ws), wsb, None) == 0
        got[:, t] = conv(o)
    ref = orc.flash_forward(inp["X"], inp["W_u"], inp["W_v"], inp["W_z"], inp["W_o"], inp["gamma"], inp["beta"],
                            inp["relpos"], C, True, use_rope=True)[:, :steps]
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert err <= (2e-2 if bf else 1e-4), err


BWD_CASES = [
    # B, T, d, e, s, C, dtype, causal
    (1, 256, 128, 256, 128, 64, "f32", True),
    (1, 256, 128, 256, 128, 64, "f32", False),
    (2, 256, 128, 256, 256, 128, "bf16", True),
    (1, 320, 128, 512, 128, 64, "bf16", False),
    (1, 1024, 1024, 1024, 128, 256, "bf16", True),   # 128 x 128 tiles (weight gradients, dV, dX)
    (1, 256, 128, 256, 128, 64, "f32", True, "wide"),  # gamma ~ N(1, 0.5^2), beta ~ N(0, 0.3^2)
    (1, 256, 128, 256, 128, 64, "f32", True, "wide", True),    # RoPE
    (2, 256, 128, 256, 256, 128, "bf16", False, "wide", True),  # RoPE, s = 256
    (1, 256, 128, 256, 128, 64, "f32", True, "wide", False, "local"),   # LocalOnly
    (1, 256, 128, 256, 128, 64, "bf16", False, "wide", False, "global"),  # GlobalOnly
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}_T{}_d{}_e{}_s{}_C{}_{}_{}{}{}".format(
    *c[:7], "causal" if c[7] else "full", "_wide" if len(c) > 8 else "", "_rope" if len(c) > 9 and c[9] else "")
    + ("_" + c[10] if len(c) > 10 else ""))
def test_emulated_backward_matches_oracle(emu, case):
    """gau_backward on the emulation: every gradient against the oracle's."""
    _emulated_backward(emu, case)


@pytest.mark.parametrize("causal", [True, False])
def test_emulated_segmented_backward_matches_oracle(emu, causal):
    """gau_backward_segmented on the emulation (packed runs of 1..3 chunks)."""
    seg = np.array([[0, 0, 0, 1, 2, 2], [4, 5, 5, 5, 6, 6]], np.int32)
    _emulated_backward(emu, (2, 384, 128, 256, 128, 64, "f32", causal, "wide"), seg=seg)


def _emulated_backward(emu, case, seg=None):
    B, T, d, e, s, C, dtype, causal = case[:8]
    heads = case[8] if len(case) > 8 else "workload"
    rope = len(case) > 9 and case[9]
    parts = case[10] if len(case) > 10 else "both"
    bf = dtype == "bf16"
    emu.emu_set_mode(1, 1)
    P = ctypes.c_void_p
    emu.gau_backward_workspace_bytes.restype = ctypes.c_size_t
    emu.gau_backward_workspace_bytes.argtypes = [ctypes.POINTER(GauConfig)]
    emu.gau_backward.argtypes = [ctypes.POINTER(GauConfig)] + [P] * 18 + [ctypes.c_size_t, P]
    emu.gau_backward.restype = ctypes.c_int
    inp = inputs.make_layer_inputs(B=B, T=T, d=d, e=e, s=s, C=C, seed=B * 17 + T + C, dtype=dtype, heads=heads)
    dO = inputs.make_output_grad(B, T, d, seed=T + C, dtype=dtype)
    cfg = GauConfig(B, T, d, e, s, C, 1 if causal else 0, 1 if bf else 0, 1.0 / C, 1.0 / C, 1 if rope else 0,
                    {"both": 0, "local": 1, "global": 2}[parts])
    X, dOh = _host(inp["X"], bf), _host(dO, bf)
    W = {k: _host(np.ascontiguousarray(inp[k].T), bf) for k in ("W_u", "W_v", "W_z", "W_o")}
    sc, of, rp = (np.ascontiguousarray(inp[k], np.float32) for k in ("gamma", "beta", "relpos"))
    out = {"X": np.zeros((B, T, d), np.float32), "W_u": np.zeros((e, d), np.float32),
           "W_v": np.zeros((e, d), np.float32), "W_z": np.zeros((s, d), np.float32),
           "W_o": np.zeros((d, e), np.float32), "gamma": np.zeros((4, s), np.float32),
           "beta": np.zeros((4, s), np.float32), "relpos": np.zeros(2 * C - 1, np.float32)}
    wsb = emu.gau_backward_workspace_bytes(ctypes.byref(cfg))
    assert wsb > 0
    raw = np.full(wsb + 256, 0xFF, np.uint8)
    ws = raw[(-raw.ctypes.data) % 256:][:wsb]
    ptr = lambda a: P(a.ctypes.data)
    args = (ptr(X), ptr(W["W_u"]), ptr(W["W_v"]), ptr(W["W_z"]), ptr(W["W_o"]), ptr(sc), ptr(of), ptr(rp), ptr(dOh),
            *[ptr(out[k]) for k in out], ptr(ws), wsb, None)
    if seg is None:
        st = emu.gau_backward(ctypes.byref(cfg), *args)
    else:
        emu.gau_backward_segmented.argtypes = [ctypes.POINTER(GauConfig)] + [P] * 19 + [ctypes.c_size_t, P]
        emu.gau_backward_segmented.restype = ctypes.c_int
        segr = np.zeros(seg.size + 4, np.int32)
        sega = segr[(-segr.ctypes.data) % 16 // 4:][:seg.size]
        sega[:] = seg.ravel()
        st = emu.gau_backward_segmented(ctypes.byref(cfg), ptr(sega), *args)
    assert st == 0
    ref = orc.flash_backward(inp["X"], inp["W_u"], inp["W_v"], inp["W_z"], inp["W_o"], inp["gamma"], inp["beta"],
                             inp["relpos"], C, causal, dO, use_rope=rope, parts=parts, chunk_segments=seg)
    tol = 2e-2 if bf else 1e-4
    for k, got in out.items():
        want = ref[k] if k != "W_o" else ref[k].T     # weights come back output-major
        want = want.T if k in ("W_u", "W_v", "W_z") else want
        assert np.all(np.isfinite(got)), k
        if not np.any(want):   # carried by the dropped term alone
            assert not np.any(got), k
            continue
        err = np.max(np.abs(got - want)) / np.max(np.abs(want))
        assert err <= tol, f"d{k}: {err:.3e} > {tol}"
