"""Pins for the CPU oracle: brute force, closed forms, invariants and the
hand-worked Code 4 fixture.  CPU only."""

import math
import os

import numpy as np
import pytest

from oracle import gau_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _tiny(B, T, d, e, s, C, seed, beta_scale=0.3, w_scale=0.5):
    rng = np.random.default_rng(seed)
    return dict(
        X=rng.standard_normal((B, T, d)),
        W_u=rng.standard_normal((d, e)) / np.sqrt(d),
        W_v=rng.standard_normal((d, e)) / np.sqrt(d),
        W_z=rng.standard_normal((d, s)) / np.sqrt(d),
        W_o=rng.standard_normal((e, d)) / np.sqrt(e),
        gamma=1.0 + 0.5 * rng.standard_normal((4, s)),
        beta=beta_scale * rng.standard_normal((4, s)),
        relpos=w_scale * rng.standard_normal(2 * C - 1),
    )


def _run(fn, p, C, causal, **kw):
    return fn(p["X"], p["W_u"], p["W_v"], p["W_z"], p["W_o"], p["gamma"], p["beta"],
              p["relpos"], C, causal, **kw)


# ---------------------------------------------------------------- Code 4

def _read_golden_toeplitz():
    mats, cur, n = {}, None, None
    with open(os.path.join(GOLDEN, "toeplitz_code4.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("n="):
                n = int(line[2:])
                cur = mats.setdefault(n, [])
            else:
                cur.append([int(v) for v in line.split()])
    return {k: np.array(v) for k, v in mats.items()}


def test_toeplitz_matches_hand_worked_code4():
    for n, idx in _read_golden_toeplitz().items():
        w = np.arange(2 * n - 1, dtype=np.float64) * 10.0 + 1.0   # distinct entries
        np.testing.assert_array_equal(orc.toeplitz_bias(w, n), w[idx])


def _code4_steps(w, n):
    """Code 4's n < 512 branch carried out with numpy array operations."""
    t = np.pad(w, (0, n))                 # pad(w, [[0, n]])
    t = np.tile(t, n)                     # tile(t, [n])
    t = t[:-n]                            # t[..., :-n]
    t = t.reshape(n, 3 * n - 2)           # reshape(t, [n, 3n-2])
    r = (2 * n - 1) // 2
    return t[:, r:t.shape[1] - r]         # t[..., r:-r]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 7, 64, 256])
def test_toeplitz_matches_code4_steps(n):
    w = np.random.default_rng(n).standard_normal(2 * n - 1)
    np.testing.assert_array_equal(orc.toeplitz_bias(w, n), _code4_steps(w, n))


# ---------------------------------------------------------------- elementwise

def test_silu_fixture_values():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "silu_values.txt"))
            if l.strip() and not l.startswith("#")]
    for x, y in rows:
        assert orc.silu(float(x)) == pytest.approx(float(y), rel=1e-15, abs=1e-300)


def test_silu_odd_part_identity():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(orc.silu(x) - orc.silu(-x), x, rtol=0, atol=1e-13)
    assert orc.silu(40.0) == pytest.approx(40.0, rel=1e-15)


def test_relu_squared_and_mask():
    np.testing.assert_array_equal(orc.relu_squared(np.array([-2.0, 0.0, 3.0])), [0.0, 0.0, 9.0])
    m = orc.causal_mask(3)
    np.testing.assert_array_equal(m, [[1, 0, 0], [1, 1, 0], [1, 1, 1]])


def test_rms_norm_closed_form():
    x = np.array([[3.0, 4.0]])
    np.testing.assert_allclose(orc.rms_norm(x, eps=0.0), x / math.sqrt(12.5), rtol=1e-15)
    y = orc.rms_norm(np.random.default_rng(0).standard_normal((5, 64)), eps=0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, rtol=1e-13)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("B,T,C", [(2, 12, 4), (1, 8, 1), (1, 8, 8), (1, 9, 3), (2, 10, 5)])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("scales", [(None, None), (1.0, 1.0), (0.7, 1.9)])
def test_chunked_equals_bruteforce(B, T, C, causal, scales):
    p = _tiny(B, T, d=5, e=6, s=4, C=C, seed=B * 100 + T * 10 + C)
    qs, ls = scales
    got = _run(orc.flash_forward, p, C, causal, quad_scale=qs, lin_scale=ls)
    ref = _run(orc.flash_forward_bruteforce, p, C, causal, quad_scale=qs, lin_scale=ls)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_bruteforce_sees_clipping_and_bias():
    """The random tiny cases must exercise relu's clipping and the bias
    direction, or the brute-force comparison would not pin them."""
    p = _tiny(1, 12, 5, 6, 4, 4, seed=3)
    _, im = _run(orc.flash_forward, p, 4, True, return_intermediates=True)
    Qq = im["Q_quad"].reshape(1, 3, 4, 4)
    Kq = im["K_quad"].reshape(1, 3, 4, 4)
    sc = (Qq @ Kq.swapaxes(-1, -2)) / 4 + orc.toeplitz_bias(p["relpos"], 4)
    low = sc[..., np.tril_indices(4)[0], np.tril_indices(4)[1]]
    assert (low < 0).any() and (low > 0).any()
    # a flipped bias index (w[C-1+i-j]) gives a different answer
    flipped = dict(p, relpos=p["relpos"][::-1].copy())
    a = _run(orc.flash_forward, p, 4, True)
    b = _run(orc.flash_forward, flipped, 4, True)
    assert np.max(np.abs(a - b)) > 1e-6


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [True, False])
def test_identity_attention_reduces_to_glu(causal):
    """gamma = beta = 0 for all heads and w = one-hot at C-1 make
    relu^2(bias) the identity and the linear term zero, so the GAU is a GLU
    (blog, "Gated Attention": A = I reduces the GAU to the GLU)."""
    C = 4
    p = _tiny(2, 12, 5, 6, 4, C, seed=7)
    p["gamma"][:] = 0.0
    p["beta"][:] = 0.0
    p["relpos"][:] = 0.0
    p["relpos"][C - 1] = 1.0
    got = _run(orc.flash_forward, p, C, causal, quad_scale=0.3, lin_scale=0.9)
    ref = orc.glu(p["X"], p["W_u"], p["W_v"], p["W_o"])
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-14)


def test_full_chunk_causal_has_no_linear_term():
    """C = T: one chunk, so the exclusive prefix is zero and FLASH is the
    quadratic GAU (papercache C.3: chunk size equal to the context length)."""
    p = _tiny(2, 8, 5, 6, 4, 8, seed=11)
    O, im = _run(orc.flash_forward, p, 8, True, return_intermediates=True)
    assert np.all(im["P"] == 0.0) and np.all(im["lin"] == 0.0)
    # quadratic GAU over the whole sequence, from the GAU equation directly
    U, V, _ = orc.projections(p["X"], p["W_u"], p["W_v"], p["W_z"])
    A = im["kernel"][:, 0]
    np.testing.assert_allclose(O, (U * (A @ V)) @ p["W_o"], rtol=1e-13, atol=1e-14)


def test_unit_chunks_match_token_recurrence():
    """C = 1: the linear part is token-level causal linear attention through
    the running cache M_t (papercache 3.1 and C.3)."""
    T = 9
    p = _tiny(1, T, 5, 6, 4, 1, seed=13)
    _, im = _run(orc.flash_forward, p, 1, True, quad_scale=0.8, lin_scale=0.6,
                 return_intermediates=True)
    ref_lin = orc.linear_attention_recurrence(im["Q_lin"][0], im["K_lin"][0], im["V"][0], 0.6)
    np.testing.assert_allclose(im["lin"][0], ref_lin, rtol=1e-12, atol=1e-13)
    diag = np.sum(im["Q_quad"][0] * im["K_quad"][0], axis=-1) * 0.8 + p["relpos"][0]
    np.testing.assert_allclose(im["quad"][0], (np.maximum(diag, 0) ** 2)[:, None] * im["V"][0],
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("C", [1, 2, 4, 8])
def test_noncausal_linear_term_is_full_linear_attention(C):
    """Eq. 7 equals linear attention on the full matrices, whatever C is
    (blog, "Mixed Chunking")."""
    p = _tiny(2, 8, 5, 6, 4, C, seed=17)
    _, im = _run(orc.flash_forward, p, C, False, lin_scale=0.25, return_intermediates=True)
    full = im["Q_lin"] @ (im["K_lin"].swapaxes(-1, -2) @ im["V"]) * 0.25
    np.testing.assert_allclose(im["lin"], full, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("t", [0, 3, 4, 7, 10])
def test_causal_output_ignores_future_tokens_bitwise(t):
    p = _tiny(2, 12, 5, 6, 4, 4, seed=19)
    a = _run(orc.flash_forward, p, 4, True)
    q = dict(p)
    q["X"] = p["X"].copy()
    q["X"][:, t + 1:] += np.random.default_rng(t).standard_normal(q["X"][:, t + 1:].shape)
    b = _run(orc.flash_forward, q, 4, True)
    np.testing.assert_array_equal(a[:, :t + 1], b[:, :t + 1])
    if t + 1 < 12:
        assert np.max(np.abs(a[:, t + 1:] - b[:, t + 1:])) > 0


def test_noncausal_output_sees_future_tokens():
    p = _tiny(1, 12, 5, 6, 4, 4, seed=23)
    a = _run(orc.flash_forward, p, 4, False)
    q = dict(p)
    q["X"] = p["X"].copy()
    q["X"][:, 11] += 1.0
    b = _run(orc.flash_forward, q, 4, False)
    assert np.max(np.abs(a[:, 0] - b[:, 0])) > 0


def test_batch_rows_are_independent():
    p = _tiny(3, 8, 5, 6, 4, 4, seed=29)
    full = _run(orc.flash_forward, p, 4, True)
    for b in range(3):
        q = dict(p, X=p["X"][b:b + 1])
        np.testing.assert_allclose(_run(orc.flash_forward, q, 4, True)[0], full[b],
                                   rtol=1e-13, atol=1e-14)


def test_scale_placement():
    """quad_scale multiplies Q K^T inside relu^2: with a zero bias the local
    term scales with its square; lin_scale multiplies the linear term once."""
    p = _tiny(1, 8, 5, 6, 4, 4, seed=31)
    p["relpos"][:] = 0.0
    _, a = _run(orc.flash_forward, p, 4, True, quad_scale=1.0, lin_scale=1.0,
                return_intermediates=True)
    _, b = _run(orc.flash_forward, p, 4, True, quad_scale=3.0, lin_scale=5.0,
                return_intermediates=True)
    np.testing.assert_allclose(b["quad"], 9.0 * a["quad"], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(b["lin"], 5.0 * a["lin"], rtol=1e-13, atol=1e-14)
    assert np.max(np.abs(a["quad"])) > 0 and np.max(np.abs(a["lin"])) > 0


def test_local_only_and_global_only_isolation():
    """LocalOnly / GlobalOnly ablations (wikillm, "Ablation variants"): zero
    Q_lin removes the global part; zero Q_quad with a non-positive bias
    removes the local part."""
    C = 4
    p = _tiny(1, 12, 5, 6, 4, C, seed=37)
    loc = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    loc["gamma"][2] = 0.0
    loc["beta"][2] = 0.0
    O, im = _run(orc.flash_forward, loc, C, True, return_intermediates=True)
    assert np.all(im["lin"] == 0.0)
    np.testing.assert_allclose(O, (im["U"] * im["quad"]) @ p["W_o"], rtol=1e-13, atol=1e-14)
    glo = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    glo["gamma"][0] = 0.0
    glo["beta"][0] = 0.0
    glo["relpos"] = -np.abs(glo["relpos"])
    O, im = _run(orc.flash_forward, glo, C, True, return_intermediates=True)
    assert np.all(im["quad"] == 0.0)
    np.testing.assert_allclose(O, (im["U"] * im["lin"]) @ p["W_o"], rtol=1e-13, atol=1e-14)


def test_exclusive_prefix_order():
    """P_0 = 0 and P_g - P_{g-1} = S_{g-1} (eq. 8 sums h = 1..g-1)."""
    p = _tiny(1, 16, 5, 6, 4, 4, seed=41)
    _, im = _run(orc.flash_forward, p, 4, True, return_intermediates=True)
    P, S = im["P"], im["S"]
    assert np.all(P[:, 0] == 0)
    np.testing.assert_allclose(P[:, 1:] - P[:, :-1], S[:, :-1], rtol=1e-12, atol=1e-14)


def test_stack_first_layer_matches_single_layer():
    C = 4
    layers = [{k: v for k, v in _tiny(1, 8, 6, 8, 4, C, seed=50 + l).items() if k != "X"}
              for l in range(2)]
    X = np.random.default_rng(5).standard_normal((1, 8, 6))
    out1 = orc.flash_stack_forward(X, layers[:1], C, True)
    L = layers[0]
    ref = X + orc.flash_forward(orc.rms_norm(X), L["W_u"], L["W_v"], L["W_z"], L["W_o"],
                                L["gamma"], L["beta"], L["relpos"], C, True)
    np.testing.assert_allclose(out1, ref, rtol=1e-14, atol=1e-14)
    out2 = orc.flash_stack_forward(X, layers, C, True)
    L = layers[1]
    ref2 = out1 + orc.flash_forward(orc.rms_norm(out1), L["W_u"], L["W_v"], L["W_z"], L["W_o"],
                                    L["gamma"], L["beta"], L["relpos"], C, True)
    np.testing.assert_allclose(out2, ref2, rtol=1e-13, atol=1e-13)


def _stack_layers(n, C, d=6, e=8, s=4, seed=60):
    return [{k: v for k, v in _tiny(1, 8, d, e, s, C, seed=seed + l).items() if k != "X"} for l in range(n)]


def test_stack_with_zero_output_weights_is_the_identity():
    """W_o = 0 in every layer: each block adds exactly zero, so the stack
    returns its input bit for bit (a dropped shortcut, or a norm applied to
    the residual stream itself, would not)."""
    C = 4
    layers = _stack_layers(3, C)
    for L in layers:
        L["W_o"] = np.zeros_like(L["W_o"])
    X = 3.0 * np.random.default_rng(6).standard_normal((2, 8, 6))
    np.testing.assert_array_equal(orc.flash_stack_forward(X, layers, C, True), X)


@pytest.mark.parametrize("c", [0.5, 7.0])
def test_stack_layer_sees_a_scale_free_input(c):
    """Pre-norm: one block adds f(norm(x)) to x, and the RMS norm removes a
    positive scale, so stack(cX) - cX equals stack(X) - X up to the norm's
    eps (a post-norm, or a residual taken after the norm, would scale).  X
    has mean square ~100, so eps = 1e-6 moves the normalised rows by ~1e-8."""
    C = 4
    layers = _stack_layers(1, C)
    X = 10.0 * np.random.default_rng(7).standard_normal((1, 8, 6))
    a = orc.flash_stack_forward(X, layers, C, True) - X
    b = orc.flash_stack_forward(c * X, layers, C, True) - c * X
    np.testing.assert_allclose(b, a, rtol=1e-5, atol=1e-7 * np.max(np.abs(a)))
    assert np.max(np.abs(a)) > 1e-2


def test_stack_is_causal_bitwise():
    """A causal stack with a per-token norm: outputs before position t do not
    depend on tokens after t, bit for bit, through every layer."""
    C = 4
    layers = _stack_layers(3, C)
    X = np.random.default_rng(8).standard_normal((1, 8, 6))
    a = orc.flash_stack_forward(X, layers, C, True)
    Y = X.copy()
    Y[:, 5:] = np.random.default_rng(9).standard_normal(Y[:, 5:].shape)
    b = orc.flash_stack_forward(Y, layers, C, True)
    np.testing.assert_array_equal(a[:, :5], b[:, :5])
    assert np.max(np.abs(a[:, 5:] - b[:, 5:])) > 0


# ---------------------------------------------------------------- RoPE

def test_rope_frequencies_match_the_printed_sinusoid_helper():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "rope_frequencies_s8.txt"))
            if l.strip() and not l.startswith("#")]
    want = np.array([float(v) for _, v in rows])
    np.testing.assert_allclose(orc.rope_frequencies(8), want, rtol=1e-14)


def test_rope_position_zero_is_identity_and_norms_are_kept():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 9, 16))
    np.testing.assert_array_equal(orc.rope(x[:, :1], [0.0]), x[:, :1])
    y = orc.rope(x, np.arange(9) * 37.0)
    half = 8
    np.testing.assert_allclose(y[..., :half] ** 2 + y[..., half:] ** 2,
                               x[..., :half] ** 2 + x[..., half:] ** 2, rtol=1e-12)


def test_rope_basis_vector_turns_by_position_times_frequency():
    """e_i at position p becomes cos(p theta_i) e_i + sin(p theta_i) e_{i+s/2}
    (the pair (i, i+s/2) is one plane; theta from the golden fixture)."""
    s, theta = 8, [1.0, 0.1, 0.01, 0.001]
    for i in range(4):
        for p in (1.0, 5.0, 123.0):
            x = np.zeros((1, s))
            x[0, i] = 1.0
            y = orc.rope(x, [p])[0]
            want = np.zeros(s)
            want[i] = math.cos(p * theta[i])
            want[i + 4] = math.sin(p * theta[i])
            np.testing.assert_allclose(y, want, atol=1e-13)


def test_rope_scores_depend_on_the_offset_only():
    """rope(q, m) . rope(k, n) is a function of n - m (shift both by any D)."""
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal((2, 6, 32))
    m = rng.integers(0, 5000, 6).astype(float)
    n = rng.integers(0, 5000, 6).astype(float)
    base = np.sum(orc.rope(q, m) * orc.rope(k, n), axis=-1)
    for D in (1.0, 250.0, 4097.0):
        shifted = np.sum(orc.rope(q, m + D) * orc.rope(k, n + D), axis=-1)
        np.testing.assert_allclose(shifted, base, rtol=1e-9, atol=1e-9)


def test_rope_rotations_compose():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 12))
    a = rng.uniform(0, 900, 5)
    b = rng.uniform(0, 900, 5)
    np.testing.assert_allclose(orc.rope(orc.rope(x, a), b), orc.rope(x, a + b), atol=1e-10)


@pytest.mark.parametrize("B,T,C", [(2, 12, 4), (1, 9, 3)])
@pytest.mark.parametrize("causal", [True, False])
def test_chunked_with_rope_equals_bruteforce(B, T, C, causal):
    """The four heads rotated by their position in the whole sequence (the
    brute force rotates each token's head vectors pair by pair itself)."""
    p = _tiny(B, T, d=5, e=6, s=4, C=C, seed=B * 31 + T)
    got = _run(orc.flash_forward, p, C, causal, use_rope=True)
    ref = _run(orc.flash_forward_bruteforce, p, C, causal, use_rope=True)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    plain = _run(orc.flash_forward, p, C, causal)
    assert np.max(np.abs(got - plain)) > 1e-3  # the rotation changes the result


def test_rope_toeplitz_is_toeplitz_with_closed_form_diagonals():
    """Code 4's n >= 512 branch depends only on the key minus query offset;
    for a = e_0 and b = e_0 or e_{half} the diagonals are cos(d) and -sin(d)
    (theta_0 = 1)."""
    rng = np.random.default_rng(10)
    a, b = rng.standard_normal((2, 16))
    t = orc.rope_toeplitz(a, b, 12)
    for dd in range(-11, 12):
        diag = np.diagonal(t, offset=dd)
        np.testing.assert_allclose(diag, diag[0], rtol=1e-10, atol=1e-10)
    w = orc.rope_relpos(a, b, 12)
    i, j = np.meshgrid(np.arange(12), np.arange(12), indexing="ij")
    np.testing.assert_allclose(w[12 - 1 + j - i], t, atol=1e-12)
    e0 = np.zeros(16); e0[0] = 1.0
    eh = np.zeros(16); eh[8] = 1.0
    d = np.arange(-11, 12)
    np.testing.assert_allclose(orc.rope_relpos(e0, e0, 12), np.cos(d), atol=1e-12)
    np.testing.assert_allclose(orc.rope_relpos(e0, eh, 12), -np.sin(d), atol=1e-12)


# ---------------------------------------------------------------- decoding

@pytest.mark.parametrize("B,T,C", [(2, 12, 4), (1, 9, 3), (1, 8, 8), (2, 10, 1)])
@pytest.mark.parametrize("use_rope", [False, True])
def test_token_by_token_decoding_equals_the_causal_layer(B, T, C, use_rope):
    """The constant-state recurrence reproduces the parallel chunked form
    (and so the brute-force T x T operator) token for token."""
    p = _tiny(B, T, d=5, e=6, s=4, C=C, seed=B * 53 + T * 7 + C)
    got = orc.flash_decode(p["X"], p["W_u"], p["W_v"], p["W_z"], p["W_o"], p["gamma"], p["beta"],
                           p["relpos"], C, use_rope=use_rope)
    ref = _run(orc.flash_forward, p, C, True, use_rope=use_rope)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_decoding_a_ragged_prefix_matches_the_layer_prefix():
    """Decoding the first 7 tokens (not a multiple of C) gives the first 7
    outputs of the full causal layer."""
    p = _tiny(1, 12, d=5, e=6, s=4, C=4, seed=77)
    full = _run(orc.flash_forward, p, 4, True)
    got = orc.flash_decode(p["X"][:, :7], p["W_u"], p["W_v"], p["W_z"], p["W_o"], p["gamma"], p["beta"],
                           p["relpos"], 4)
    np.testing.assert_allclose(got, full[:, :7], rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_parts_local_and_global_match_the_ablation_by_weights(causal):
    """parts="local" equals the layer whose Q_lin head is zero, and
    parts="global" the layer whose Q_quad head is zero with a negative bias
    (relu clips every score): the ablations expressed through the inputs."""
    C = 4
    p = _tiny(2, 12, 5, 6, 4, C, seed=38)
    loc = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    loc["gamma"][2] = 0.0
    loc["beta"][2] = 0.0
    np.testing.assert_allclose(_run(orc.flash_forward, p, C, causal, parts="local"),
                               _run(orc.flash_forward_bruteforce, loc, C, causal), rtol=1e-11, atol=1e-12)
    glo = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    glo["gamma"][0] = 0.0
    glo["beta"][0] = 0.0
    glo["relpos"] = -np.abs(glo["relpos"]) - 0.1
    np.testing.assert_allclose(_run(orc.flash_forward, p, C, causal, parts="global"),
                               _run(orc.flash_forward_bruteforce, glo, C, causal), rtol=1e-11, atol=1e-12)
    full = _run(orc.flash_forward, p, C, causal)
    both = _run(orc.flash_forward, p, C, causal, parts="local") + _run(orc.flash_forward, p, C, causal, parts="global")
    np.testing.assert_allclose(both, full, rtol=1e-11, atol=1e-12)   # the output is linear in (quad + lin)


# ---------------------------------------------------------------- gradients

def test_silu_grad_matches_central_differences():
    x = np.linspace(-12, 12, 97)
    h = 1e-5
    fd = (orc.silu(x + h) - orc.silu(x - h)) / (2 * h)
    np.testing.assert_allclose(orc.silu_grad(x), fd, rtol=1e-8, atol=1e-10)


@pytest.mark.parametrize("B,T,C,rope", [(2, 8, 4, False), (1, 9, 3, False), (2, 8, 4, True)])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_matches_central_differences(B, T, C, rope, causal):
    """Every gradient of <dO, O> against central differences of the
    brute-force forward (not the chunked one), entry by entry; with RoPE the
    brute force rotates each head vector by its own position."""
    p = _tiny(B, T, d=4, e=5, s=4, C=C, seed=B * 17 + T + C)
    dO = np.random.default_rng(5).standard_normal((B, T, 4))
    g = orc.flash_backward(p["X"], p["W_u"], p["W_v"], p["W_z"], p["W_o"], p["gamma"], p["beta"],
                           p["relpos"], C, causal, dO, quad_scale=0.6, lin_scale=0.8, use_rope=rope)
    h = 1e-6

    def f(q):
        return float(np.sum(dO * _run(orc.flash_forward_bruteforce, q, C, causal, quad_scale=0.6, lin_scale=0.8,
                                      use_rope=rope)))

    names = {"X": "X", "W_u": "W_u", "W_v": "W_v", "W_z": "W_z", "W_o": "W_o", "gamma": "gamma",
             "beta": "beta", "relpos": "relpos"}
    for k, pk in names.items():
        fd = np.zeros_like(p[pk])
        for idx in np.ndindex(p[pk].shape):
            up = {a: (b.copy() if isinstance(b, np.ndarray) else b) for a, b in p.items()}
            dn = {a: (b.copy() if isinstance(b, np.ndarray) else b) for a, b in p.items()}
            up[pk][idx] += h
            dn[pk][idx] -= h
            fd[idx] = (f(up) - f(dn)) / (2 * h)
        np.testing.assert_allclose(g[k], fd, rtol=1e-5, atol=1e-6, err_msg=k)


@pytest.mark.parametrize("parts", ["local", "global"])
@pytest.mark.parametrize("causal", [True, False])
def test_backward_of_one_part_matches_central_differences(parts, causal):
    """LocalOnly / GlobalOnly: every gradient against central differences of
    the chunked forward with that part alone (pinned above by the weight
    ablations it equals)."""
    B, T, C = 2, 8, 4
    p = _tiny(B, T, d=4, e=5, s=4, C=C, seed=41)
    dO = np.random.default_rng(6).standard_normal((B, T, 4))
    g = orc.flash_backward(p["X"], p["W_u"], p["W_v"], p["W_z"], p["W_o"], p["gamma"], p["beta"],
                           p["relpos"], C, causal, dO, quad_scale=0.6, lin_scale=0.8, parts=parts)
    h = 1e-6

    def f(q):
        return float(np.sum(dO * _run(orc.flash_forward, q, C, causal, quad_scale=0.6, lin_scale=0.8, parts=parts)))

    for k in ("X", "W_u", "W_v", "W_z", "W_o", "gamma", "beta", "relpos"):
        fd = np.zeros_like(p[k])
        for idx in np.ndindex(p[k].shape):
            up = {a: (b.copy() if isinstance(b, np.ndarray) else b) for a, b in p.items()}
            dn = {a: (b.copy() if isinstance(b, np.ndarray) else b) for a, b in p.items()}
            up[k][idx] += h
            dn[k][idx] -= h
            fd[idx] = (f(up) - f(dn)) / (2 * h)
        np.testing.assert_allclose(g[k], fd, rtol=1e-5, atol=1e-6, err_msg=k)
    # what only feeds the dropped part gets nothing
    if parts == "local":
        assert np.all(g["gamma"][2:] == 0) and np.all(g["beta"][2:] == 0)
    else:
        assert np.all(g["gamma"][:2] == 0) and np.all(g["relpos"] == 0)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_with_segments_matches_central_differences(causal):
    """Packed sequences: every gradient against central differences of the
    brute-force forward with the same chunk segments."""
    B, T, C = 2, 12, 2
    seg = [[0, 0, 1, 1, 1, 5], [3, 4, 4, 4, 4, 4]]
    p = _tiny(B, T, d=4, e=5, s=4, C=C, seed=43)
    dO = np.random.default_rng(7).standard_normal((B, T, 4))
    g = orc.flash_backward(p["X"], p["W_u"], p["W_v"], p["W_z"], p["W_o"], p["gamma"], p["beta"],
                           p["relpos"], C, causal, dO, quad_scale=0.6, lin_scale=0.8, chunk_segments=seg)
    h = 1e-6

    def f(q):
        return float(np.sum(dO * _run(orc.flash_forward_bruteforce, q, C, causal, quad_scale=0.6, lin_scale=0.8,
                                      chunk_segments=seg)))

    for k in ("X", "W_u", "W_v", "W_z", "W_o", "gamma", "beta", "relpos"):
        fd = np.zeros_like(p[k])
        for idx in np.ndindex(p[k].shape):
            up = {a: (b.copy() if isinstance(b, np.ndarray) else b) for a, b in p.items()}
            dn = {a: (b.copy() if isinstance(b, np.ndarray) else b) for a, b in p.items()}
            up[k][idx] += h
            dn[k][idx] -= h
            fd[idx] = (f(up) - f(dn)) / (2 * h)
        np.testing.assert_allclose(g[k], fd, rtol=1e-5, atol=1e-6, err_msg=k)


# ---------------------------------------------------------------- segment masks

SEGMENTS = [
    # B, T, C, causal, per-row chunk ids
    (1, 24, 4, True, [[0, 0, 1, 1, 1, 2]]),
    (2, 24, 4, False, [[3, 3, 3, 8, 8, 8], [1, 2, 3, 4, 5, 6]]),
    (1, 16, 2, True, [[0, 1, 0, 0, 2, 2, 2, 2]]),   # an id that comes back starts a new segment
    (2, 12, 3, True, [[7, 7, 7, 7], [0, 1, 1, 1]]),
    (1, 12, 4, False, [[0, 0, 0]]),
]


@pytest.mark.parametrize("case", SEGMENTS, ids=lambda c: f"B{c[0]}_T{c[1]}_C{c[2]}_{'causal' if c[3] else 'full'}")
def test_segmented_chunked_equals_bruteforce(case):
    B, T, C, causal, seg = case
    p = _tiny(B, T, 5, 6, 4, C, seed=T + C + B)
    seg = np.array(seg)
    got = _run(orc.flash_forward, p, C, causal, chunk_segments=seg)
    ref = _run(orc.flash_forward_bruteforce, p, C, causal, chunk_segments=seg)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    # the segments matter: the unsegmented layer differs
    assert np.max(np.abs(_run(orc.flash_forward, p, C, causal) - ref)) > 1e-3 * np.max(np.abs(ref))


@pytest.mark.parametrize("causal", [True, False])
def test_one_segment_averages_the_visible_summaries(causal):
    """One segment per row: the linear term of chunk g is the plain layer's
    with its summaries divided by the number of visible chunks (g when
    causal, G otherwise), i.e. the plain layer with lin_scale / n, chunk by
    chunk; chunk 0 of a causal row sees nothing (divide_no_nan) and equals
    the plain layer's chunk 0."""
    B, T, C = 2, 20, 4
    G = T // C
    p = _tiny(B, T, 5, 6, 4, C, seed=71)
    seg = np.zeros((B, G), dtype=int)
    got = _run(orc.flash_forward, p, C, causal, chunk_segments=seg)
    for g in range(G):
        n = g if causal else G
        ls = (1.0 / C) / n if n > 0 else 1.0 / C
        ref = _run(orc.flash_forward, p, C, causal, lin_scale=ls)
        np.testing.assert_allclose(got[:, g * C:(g + 1) * C], ref[:, g * C:(g + 1) * C], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("causal", [True, False])
def test_packed_sequences_equal_separate_runs(causal):
    """Two sequences packed into one row, each a segment starting on a chunk
    boundary: the packed output is the two rows run on their own, each as one
    segment (the local part never crosses a chunk, and the mask keeps the
    linear part inside each segment)."""
    C, T1, T2 = 4, 12, 8
    p = _tiny(1, T1 + T2, 5, 6, 4, C, seed=72)
    seg = np.array([[4] * (T1 // C) + [9] * (T2 // C)])
    packed = _run(orc.flash_forward, p, C, causal, chunk_segments=seg)
    for lo, hi in ((0, T1), (T1, T1 + T2)):
        q = dict(p, X=p["X"][:, lo:hi])
        alone = _run(orc.flash_forward, q, C, causal, chunk_segments=np.zeros((1, (hi - lo) // C), int))
        np.testing.assert_allclose(packed[:, lo:hi], alone, rtol=1e-11, atol=1e-13)


def test_segment_ids_matter_only_through_runs():
    """Relabelling the ids, run for run, changes nothing (bitwise)."""
    C, T = 4, 24
    p = _tiny(1, T, 5, 6, 4, C, seed=73)
    a = _run(orc.flash_forward, p, C, True, chunk_segments=np.array([[0, 0, 1, 1, 1, 2]]))
    b = _run(orc.flash_forward, p, C, True, chunk_segments=np.array([[-5, -5, 40, 40, 40, 7]]))
    np.testing.assert_array_equal(a, b)


def test_segment_mask_rows():
    """The mask's rows: each sums to 1 or is all zero (divide_no_nan); the
    first chunk of a causal segment sees nothing."""
    M = orc.segment_chunk_mask(np.array([[0, 0, 1, 1, 1, 0]]), True)[0]
    np.testing.assert_array_equal(M.sum(axis=1), [0, 1, 0, 1, 1, 0])
    assert M[4, 2] == M[4, 3] == 0.5 and M[3, 2] == 1.0 and M[1, 0] == 1.0
    N = orc.segment_chunk_mask(np.array([[0, 0, 1]]), False)[0]
    np.testing.assert_array_equal(N, [[0.5, 0.5, 0], [0.5, 0.5, 0], [0, 0, 1]])
