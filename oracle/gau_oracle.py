"""CPU oracle for the FLASH gated attention unit with mixed chunk attention.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain float64 statement of
what the layer computes.  Only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
library: no kernels, headers, helpers or constants, and it imports nothing from
the package.

Sources ("Transformer Quality in Linear Time", Hua, Dai, Liu, Le, and two
summaries of it; Su Jianlin's blog post "FLASH: Possibly the Most Interesting
Efficient Transformer Design in Recent Times"):

* GAU output O = (U * (A V)) W_o with U, V = SiLU(X W_u), SiLU(X W_v):
  blog, "Gated Attention" (GLU and GAU equations); paper summary (wikillm),
  "Method", eq. 1-3.
* Z = SiLU(X W_z) and the four per-dimension scale+offset heads:
  blog, "Weak Attention" (the relu^2 attention equation); wikillm, "Method",
  "Mixed chunk attention"; papercache, section 3.2 "Preparation".
* Intra-chunk attention relu^2(Q K^T + b) V with a causal lower-triangular mask:
  blog, "Mixed Chunking" (the V_quad equation); wikillm, "Method" step 1 and the
  FLASH block pseudocode (Code 8 rewrite).
* Inter-chunk linear attention, a plain sum over all chunks (non-causal, eq. 7)
  or over strictly earlier chunks (causal, eq. 8): wikillm, "Method" steps 2-3;
  blog, "Mixed Chunking".
* O_g = [U_g * (V_quad_g + V_lin_g)] W_o: wikillm, "Method" step 4; blog,
  "Mixed Chunking" (final equation).
* Relative-position bias as a Toeplitz matrix of a 2n-1 vector:
  papercache, appendix D, Code 4 (the n < 512 branch); for n >= 512 the same
  listing builds it from two RoPE-rotated vectors (einsum of the rotated
  rows), which ``rope_toeplitz`` carries out.
* Rotary position embedding on the four heads, positions counted over the
  whole sequence: wikillm, FLASH block pseudocode (the Code 8 rewrite) and
  "Paper vs code"; Su's post credits the paper's use of RoPE.

Readings where the pages are silent or disagree (each is also listed in the
design notes):

* Scaling.  The equations put no factor on Q K^T or on the chunk summaries; the
  listing divides Q K^T by C and K_lin^T V by C.  Both are parameters here:
  ``quad_scale`` multiplies Q K^T before the bias is added (inside relu^2), and
  ``lin_scale`` multiplies each chunk summary K_lin^T V.  The listing's reading
  is quad_scale = lin_scale = 1/C.
* Bias index: b[i, j] = w[C - 1 + j - i] (key position minus query position),
  obtained by carrying out Code 4's pad / tile / slice / reshape / slice steps.
* The causal mask keeps j <= i (diagonal included) and is applied after relu^2.
* SiLU on U, V and Z.  No dense-layer biases.  RoPE is
  optional (off in the layer's plain form, which has no RoPE argument).
* RoPE itself is not printed on the pages.  ``rope`` rotates the pairs
  (x_i, x_{i+s/2}) by t * theta_i with theta_i = 10000^(-i/(s/2)): the
  frequency schedule and the [first half | second half] layout of the
  sinusoid helper the pages do print (papercache, appendix D, other
  pseudocode, _get_scaledsin).  parity unpinned for this convention choice:
  the pins fix the rotation's defining properties, not which pairing the
  authors' hidden helper used.
* Non-causal: every chunk (its own included) feeds the linear term.
* Segment masks for packed sequences (optional ``chunk_segments``).  The
  listing's Code 7 builds a chunk-level mask and divides each of its rows by
  the row's sum (divide_no_nan: an all-zero row stays zero); Code 8 applies it
  to the chunk summaries only, so the linear term becomes the average of the
  visible summaries; the local part has no segment mask (wikillm, "Paper vs
  code" and "Pitfalls", segment masks).  Code 7 itself is not on the pages.
  Reading taken here: one segment id per chunk (documents packed along the
  sequence start on chunk boundaries); a segment is a maximal run of
  consecutive chunks with equal ids; chunk h is visible from chunk g when both
  lie in one segment and, causal, h < g (non-causal: every chunk of the
  segment, g included).  Without ``chunk_segments`` the layer is the plain
  sum of equations 7 and 8.  parity unpinned for the reading itself (which
  chunks Code 7 counts as visible is not printed); its arithmetic is pinned.

parity pinned: every function here is checked in tests/test_oracle.py against
brute force, closed forms or invariants that do not reuse its code.
"""

import numpy as np


# --------------------------------------------------------------------------
# elementwise pieces
# --------------------------------------------------------------------------

def silu(x):
    """SiLU / Swish, x * sigmoid(x), in float64.

    Blog, "Gated Attention": the paper applies Swish (SiLU) to both U and V;
    wikillm, "Paper vs code" (Activation): Code 6 and Code 8 apply SiLU to U, V
    and Z.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def scale_offset(z, gamma, beta):
    """Per-dimension affine head Z * gamma + beta (like LayerNorm's gamma, beta).

    Blog, "Weak Attention" (Q and K are simple affine transforms of Z);
    papercache section 2 (per-dimension scale and offset).
    """
    return np.asarray(z, np.float64) * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def relu_squared(x):
    """relu(x)**2, the attention activation (blog, "Weak Attention"; eq. 5)."""
    r = np.maximum(np.asarray(x, np.float64), 0.0)
    return r * r


def toeplitz_bias(w, n):
    """n x n relative-position bias built from a learned 2n-1 vector.

    papercache, appendix D, Code 4 (n < 512 branch).  Carrying out that
    listing's steps (pad by n zeros, tile n times, drop the last n, reshape to
    n x (3n-2), keep the middle n columns) gives b[i, j] = w[n - 1 + j - i].
    """
    w = np.asarray(w, dtype=np.float64)
    if w.shape != (2 * n - 1,):
        raise ValueError("relative-position vector must have length 2n-1")
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return w[n - 1 + j - i]


def causal_mask(n):
    """Lower-triangular 0/1 mask, diagonal included (wikillm, Code 8 rewrite)."""
    return np.tril(np.ones((n, n), dtype=np.float64))


# --------------------------------------------------------------------------
# the layer, chunked form (the steps in the order of the FLASH block)
# --------------------------------------------------------------------------

def _as64(a):
    return np.asarray(a, dtype=np.float64)


def projections(X, W_u, W_v, W_z):
    """U, V, Z = SiLU(X W_u), SiLU(X W_v), SiLU(X W_z).

    One dense layer of width 2e+s followed by SiLU, split into U, V and the
    shared base Z (wikillm, FLASH block pseudocode; blog, "Gated Attention").
    Weights are in the pages' orientation: W_u, W_v are d x e, W_z is d x s.
    """
    X = _as64(X)
    H = X @ np.concatenate([_as64(W_u), _as64(W_v), _as64(W_z)], axis=1)
    e = np.shape(W_u)[1]
    return silu(H[..., :e]), silu(H[..., e:2 * e]), silu(H[..., 2 * e:])


def rope_frequencies(s):
    """theta_i = 10000^(-i / (s/2)), i = 0 .. s/2-1 (the inverse frequencies
    of the pages' sinusoid helper, papercache appendix D, _get_scaledsin)."""
    half = s // 2
    return 10000.0 ** (-(np.arange(half, dtype=np.float64) / half))


def rope(x, positions):
    """Rotary position embedding over the last axis of x (..., T, s):
    the pair (x_i, x_{i+s/2}) at position p is rotated by the angle
    p * theta_i:  (x_i cos - x_{i+s/2} sin, x_{i+s/2} cos + x_i sin)."""
    x = _as64(x)
    s = x.shape[-1]
    half = s // 2
    ang = _as64(positions)[:, None] * rope_frequencies(s)[None, :]   # (T, s/2)
    c, sn = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * sn, hi * c + lo * sn], axis=-1)


def rope_toeplitz(a, b, n):
    """The n >= 512 branch of Code 4 (papercache, appendix D): tile the
    vectors a and b over n positions, rotate each row by its position, and
    take t[m, k] = rope(a)_m . rope(b)_k."""
    a = np.tile(_as64(a)[None, :], (n, 1))
    b = np.tile(_as64(b)[None, :], (n, 1))
    pos = np.arange(n)
    return rope(a, pos) @ rope(b, pos).T


def rope_relpos(a, b, n):
    """The 2n-1 vector w of that Toeplitz matrix, t[i, j] = w[n-1 + j - i]
    (read off its first row and first column)."""
    t = rope_toeplitz(a, b, n)
    return np.concatenate([t[::-1, 0][:-1], t[0, :]])


def segment_chunk_mask(chunk_segments, causal):
    """The row-normalised chunk mask M[b, g, h] of Code 7 as described on the
    wikillm page ("Paper vs code", segment masks): 1 where chunk h is visible
    from chunk g, each row divided by its sum (divide_no_nan: rows with no
    visible chunk stay 0).  A segment is a maximal run of consecutive chunks
    with equal ids; visible = same segment and, when causal, h < g."""
    seg = np.asarray(chunk_segments)
    B, G = seg.shape
    run = np.zeros((B, G), dtype=np.int64)          # run index of each chunk
    run[:, 1:] = np.cumsum(seg[:, 1:] != seg[:, :-1], axis=1)
    same = run[:, :, None] == run[:, None, :]
    if causal:
        same = same & (np.arange(G)[None, :, None] > np.arange(G)[None, None, :])
    M = same.astype(np.float64)
    n = M.sum(axis=-1, keepdims=True)
    return np.divide(M, n, out=np.zeros_like(M), where=n > 0)


def heads(Z, gamma, beta):
    """The four heads Q_quad, K_quad, Q_lin, K_lin from Z.

    gamma, beta have shape (4, s) in that order (wikillm, "Mixed chunk
    attention": four heads are derived from Z; papercache 3.2 "Preparation").
    """
    gamma = _as64(gamma)
    beta = _as64(beta)
    return tuple(scale_offset(Z, gamma[h], beta[h]) for h in range(4))


def flash_forward(X, W_u, W_v, W_z, W_o, gamma, beta, relpos, C, causal,
                  quad_scale=None, lin_scale=None, return_intermediates=False, use_rope=False,
                  parts="both", chunk_segments=None):
    """Forward pass of one FLASH layer (GAU with mixed chunk attention).

    X: (B, T, d).  W_u, W_v: (d, e).  W_z: (d, s).  W_o: (e, d).
    gamma, beta: (4, s).  relpos: (2C-1,).  T must be a multiple of C.
    quad_scale / lin_scale default to 1/C (the listing's reading).
    use_rope rotates the four heads by their position in the sequence (0 ..
    T-1, not restarted per chunk: wikillm, FLASH block pseudocode).
    parts = "local" keeps only the quadratic in-chunk term and "global" only
    the linear cross-chunk term (the LocalOnly / GlobalOnly ablation
    variants: wikillm, "Ablation variants"; Su's post reports both fall well
    short of the full model).
    chunk_segments (B, G) ints: packed sequences; the linear term of chunk g
    becomes the average of the summaries of the chunks visible from it
    (segment_chunk_mask), the local part is unchanged.

    Steps, in the order of the FLASH block (wikillm pseudocode; blog "Mixed
    Chunking"; papercache 3.2):
      1. U, V, Z from one SiLU projection; four scale+offset heads from Z.
      2. Split the sequence into G = T / C non-overlapping chunks.
      3. Per chunk: kernel = relu^2(Q_quad K_quad^T * quad_scale + bias),
         lower-triangular masked when causal; quad = kernel @ V.
      4. Per chunk summary S_g = lin_scale * K_lin_g^T V_g  (s x e).
      5. Causal: P_g = sum_{h<g} S_h (exclusive prefix, eq. 8); otherwise
         P_g = sum over all h (eq. 7).
      6. lin = Q_lin_g P_g;  out = U * (quad + lin);  O = out @ W_o.
    """
    X = _as64(X)
    B, T, d = X.shape
    if T % C != 0:
        raise ValueError("T must be a multiple of C")
    G = T // C
    if quad_scale is None:
        quad_scale = 1.0 / C
    if lin_scale is None:
        lin_scale = 1.0 / C

    U, V, Z = projections(X, W_u, W_v, W_z)
    e = U.shape[-1]
    s = Z.shape[-1]
    Qq, Kq, Ql, Kl = heads(Z, gamma, beta)
    if use_rope:
        pos = np.arange(T)
        Qq, Kq, Ql, Kl = (rope(h, pos) for h in (Qq, Kq, Ql, Kl))

    def chunks(a):
        return a.reshape(B, G, C, a.shape[-1])

    Ug, Vg, Qqg, Kqg, Qlg, Klg = map(chunks, (U, V, Qq, Kq, Ql, Kl))

    # step 3: local squared-ReLU attention inside each chunk
    scores = (Qqg @ Kqg.swapaxes(-1, -2)) * quad_scale + toeplitz_bias(relpos, C)
    kernel = relu_squared(scores)
    if causal:
        kernel = kernel * causal_mask(C)
    quad = kernel @ Vg

    # step 4: one s x e summary per chunk
    S = (Klg.swapaxes(-1, -2) @ Vg) * lin_scale

    # step 5: chunk-level sum, exclusive prefix when causal; with segments,
    # the row-normalised chunk mask applied to the summaries
    if chunk_segments is not None:
        if np.shape(chunk_segments) != (B, G):
            raise ValueError("chunk_segments must have shape (B, T / C)")
        M = segment_chunk_mask(chunk_segments, causal)
        P = np.einsum("bgh,bhse->bgse", M, S)
    elif causal:
        incl = np.cumsum(S, axis=1)
        P = np.concatenate([np.zeros_like(S[:, :1]), incl[:, :-1]], axis=1)
    else:
        P = np.broadcast_to(S.sum(axis=1, keepdims=True), S.shape)

    # step 6: linear term, gate, output projection
    lin = Qlg @ P
    if parts == "local":
        lin = np.zeros_like(lin)
    elif parts == "global":
        quad = np.zeros_like(quad)
    elif parts != "both":
        raise ValueError("parts must be 'both', 'local' or 'global'")
    Y = Ug * (quad + lin)
    O = (Y.reshape(B, T, e)) @ _as64(W_o)
    if not return_intermediates:
        return O
    flat = lambda a: a.reshape(B, T, a.shape[-1])
    return O, {
        "U": U, "V": V, "Z": Z, "Q_quad": Qq, "K_quad": Kq, "Q_lin": Ql, "K_lin": Kl,
        "quad": flat(quad), "S": S, "P": np.array(P), "lin": flat(lin), "Y": flat(Y),
        "kernel": kernel,
    }


# --------------------------------------------------------------------------
# the same layer as one T x T operator, built token by token (tiny T only)
# --------------------------------------------------------------------------

def flash_forward_bruteforce(X, W_u, W_v, W_z, W_o, gamma, beta, relpos, C, causal,
                             quad_scale=None, lin_scale=None, use_rope=False, chunk_segments=None):
    """The layer as O = (U * (A V)) W_o with the full T x T matrix A.

    A per-token double loop builds A[t, tau] (blog, "Gated Attention" GAU
    equation; "Mixed Chunking" notes that the chunked global part is exactly
    linear attention on the full matrices):
      * same chunk (and tau <= t when causal):
          relu^2(q_quad_t . k_quad_tau * quad_scale + w[C-1 + (tau mod C) - (t mod C)])
      * plus q_lin_t . k_lin_tau * lin_scale when chunk(tau) < chunk(t)
        (causal), or for every tau (non-causal, own chunk included).
    With use_rope, each head vector of token t is rotated pair by pair,
    (h_i, h_{i+s/2}) by the angle t * 10000^(-i/(s/2)), written out here.
    With chunk_segments, the linear entry is kept only when chunk(tau) is in
    the same segment (run of equal consecutive ids) as chunk(t), and divided
    by the number of chunks visible from chunk(t), counted here by a loop.
    Every product is written out per token; nothing is shared with
    ``flash_forward`` beyond the SiLU definition.  Pure Python loops: keep
    T small.
    """
    X = _as64(X)
    B, T, d = X.shape
    if T % C != 0:
        raise ValueError("T must be a multiple of C")
    if quad_scale is None:
        quad_scale = 1.0 / C
    if lin_scale is None:
        lin_scale = 1.0 / C
    W_u, W_v, W_z, W_o = map(_as64, (W_u, W_v, W_z, W_o))
    gamma, beta, w = _as64(gamma), _as64(beta), _as64(relpos)
    e = W_u.shape[1]
    out = np.zeros((B, T, d))
    for b in range(B):
        u = np.zeros((T, e)); v = np.zeros((T, e))
        qq = [None] * T; kq = [None] * T; ql = [None] * T; kl = [None] * T
        for t in range(T):
            x = X[b, t]
            u[t] = silu(x @ W_u)
            v[t] = silu(x @ W_v)
            z = silu(x @ W_z)
            qq[t] = z * gamma[0] + beta[0]
            kq[t] = z * gamma[1] + beta[1]
            ql[t] = z * gamma[2] + beta[2]
            kl[t] = z * gamma[3] + beta[3]
            if use_rope:
                for hv in (qq[t], kq[t], ql[t], kl[t]):
                    half = hv.shape[0] // 2
                    for i in range(half):
                        ang = t * 10000.0 ** (-i / half)
                        x0, x1 = hv[i], hv[i + half]
                        hv[i] = x0 * np.cos(ang) - x1 * np.sin(ang)
                        hv[i + half] = x1 * np.cos(ang) + x0 * np.sin(ang)
        G = T // C
        if chunk_segments is not None:
            ids = [int(x) for x in np.asarray(chunk_segments)[b]]
            first = [0] * G                      # first chunk of each chunk's segment
            for g in range(1, G):
                first[g] = first[g - 1] if ids[g] == ids[g - 1] else g
            last = [G - 1] * G                   # last chunk of each chunk's segment
            for g in range(G - 2, -1, -1):
                last[g] = last[g + 1] if ids[g] == ids[g + 1] else g

        def visible(g, h):
            if chunk_segments is not None and not (first[g] <= h <= last[g]):
                return False
            return h < g if causal else True

        nvis = [sum(1 for h in range(G) if visible(g, h)) for g in range(G)]
        A = np.zeros((T, T))
        for t in range(T):
            for tau in range(T):
                a = 0.0
                same = (t // C) == (tau // C)
                if same and (tau <= t or not causal):
                    sc = float(np.dot(qq[t], kq[tau])) * quad_scale + w[C - 1 + (tau % C) - (t % C)]
                    a += max(sc, 0.0) ** 2
                if visible(t // C, tau // C):
                    lin = float(np.dot(ql[t], kl[tau])) * lin_scale
                    a += lin / nvis[t // C] if chunk_segments is not None else lin
                A[t, tau] = a
        out[b] = (u * (A @ v)) @ W_o
    return out


# --------------------------------------------------------------------------
# gradients of the layer (the chain rule through the steps of flash_forward)
# --------------------------------------------------------------------------

def silu_grad(h):
    """d SiLU(h) / dh = sigma(h) (1 + h (1 - sigma(h)))."""
    sg = 1.0 / (1.0 + np.exp(-_as64(h)))
    return sg * (1.0 + h * (1.0 - sg))


def flash_backward(X, W_u, W_v, W_z, W_o, gamma, beta, relpos, C, causal, dO,
                   quad_scale=None, lin_scale=None, use_rope=False, parts="both", chunk_segments=None):
    """Gradients of <dO, O> for O = flash_forward(...): a dict with X, W_u,
    W_v, W_z, W_o (pages' orientation), gamma, beta, relpos.  parts as in
    flash_forward: "local" drops the linear term (and everything that only
    feeds it gets a zero gradient), "global" the quadratic one.  The steps of
    flash_forward taken backwards, each product's derivative written out:
      O = Y W_o; Y = U * Wq (Wq = quad + lin); lin_g = Ql_g P_g;
      P = exclusive (or full) sum of S_h = ls Kl_h^T V_h;
      quad_g = A_g V_g with A_g = relu(Sc_g)^2 * mask, Sc_g = qs Qq Kq^T + Bias;
      heads h_k = Z gamma_k + beta_k (rotated by rope at their positions when
      use_rope); U, V, Z = SiLU(X W).
    A rotation's transpose is the rotation by the opposite angle, so the
    gradients of the rotated heads go back through rope at the negated
    positions.  With chunk_segments the summaries reach P through the
    row-normalised chunk mask M (P_g = sum_h M[g, h] S_h), so dS_h =
    sum_g M[g, h] dP_g.
    """
    X = _as64(X)
    B, T, d = X.shape
    G = T // C
    if quad_scale is None:
        quad_scale = 1.0 / C
    if lin_scale is None:
        lin_scale = 1.0 / C
    W_u, W_v, W_z, W_o = map(_as64, (W_u, W_v, W_z, W_o))
    gamma, beta, dO = _as64(gamma), _as64(beta), _as64(dO)
    Hu, Hv, Hz = X @ W_u, X @ W_v, X @ W_z
    U, V, Z = silu(Hu), silu(Hv), silu(Hz)
    e, s = U.shape[-1], Z.shape[-1]
    Qq, Kq, Ql, Kl = heads(Z, gamma, beta)
    pos = np.arange(T)
    if use_rope:
        Qq, Kq, Ql, Kl = (rope(h, pos) for h in (Qq, Kq, Ql, Kl))
    ch = lambda a: a.reshape(B, G, C, a.shape[-1])
    Vg, Qqg, Kqg, Qlg, Klg = map(ch, (V, Qq, Kq, Ql, Kl))
    mask = causal_mask(C) if causal else np.ones((C, C))
    Sc = (Qqg @ Kqg.swapaxes(-1, -2)) * quad_scale + toeplitz_bias(relpos, C)
    A = relu_squared(Sc) * mask
    S = (Klg.swapaxes(-1, -2) @ Vg) * lin_scale
    if chunk_segments is not None:
        if np.shape(chunk_segments) != (B, G):
            raise ValueError("chunk_segments must have shape (B, T / C)")
        Mseg = segment_chunk_mask(chunk_segments, causal)
        P = np.einsum("bgh,bhse->bgse", Mseg, S)
    elif causal:
        incl = np.cumsum(S, axis=1)
        P = np.concatenate([np.zeros_like(S[:, :1]), incl[:, :-1]], axis=1)
    else:
        P = np.broadcast_to(S.sum(axis=1, keepdims=True), S.shape)
    if parts not in ("both", "local", "global"):
        raise ValueError("parts must be 'both', 'local' or 'global'")
    keep_quad, keep_lin = parts != "global", parts != "local"
    Wq = ((A @ Vg) * keep_quad + (Qlg @ P) * keep_lin).reshape(B, T, e)
    Y = U * Wq
    # backwards
    dY = dO @ W_o.T
    dW_o = Y.reshape(-1, e).T @ dO.reshape(-1, d)
    dU = dY * Wq
    dWq = ch(dY * U)
    dWq_quad, dWq_lin = dWq * keep_quad, dWq * keep_lin   # the parts that reach O
    dA = dWq_quad @ Vg.swapaxes(-1, -2)
    dV = A.swapaxes(-1, -2) @ dWq_quad
    dQl = dWq_lin @ P.swapaxes(-1, -2)
    dP = Qlg.swapaxes(-1, -2) @ dWq_lin
    if chunk_segments is not None:   # S_h feeds P_g with weight M[g, h]
        dS = np.einsum("bgh,bgse->bhse", Mseg, dP)
    elif causal:   # S_h feeds P_g for every g > h
        rev = np.cumsum(dP[:, ::-1], axis=1)[:, ::-1]
        dS = np.concatenate([rev[:, 1:], np.zeros_like(dP[:, :1])], axis=1)
    else:
        dS = np.broadcast_to(dP.sum(axis=1, keepdims=True), dP.shape)
    dKl = lin_scale * (Vg @ dS.swapaxes(-1, -2))
    dV = dV + lin_scale * (Klg @ dS)
    dSc = dA * 2.0 * np.maximum(Sc, 0.0) * mask
    dQq = quad_scale * (dSc @ Kqg)
    dKq = quad_scale * (dSc.swapaxes(-1, -2) @ Qqg)
    i, j = np.meshgrid(np.arange(C), np.arange(C), indexing="ij")
    drel = np.zeros(2 * C - 1)
    np.add.at(drel, (C - 1 + j - i).ravel(), dSc.sum(axis=(0, 1)).ravel())
    flat = lambda a: a.reshape(B, T, a.shape[-1])
    dh = [flat(x) for x in (dQq, dKq, dQl, dKl)]
    if use_rope:
        dh = [rope(x, -pos) for x in dh]
    dZ = sum(dh[k] * gamma[k] for k in range(4))
    dgamma = np.stack([(dh[k] * Z).sum(axis=(0, 1)) for k in range(4)])
    dbeta = np.stack([dh[k].sum(axis=(0, 1)) for k in range(4)])
    dHu, dHv, dHz = dU * silu_grad(Hu), flat(dV) * silu_grad(Hv), dZ * silu_grad(Hz)
    dX = dHu @ W_u.T + dHv @ W_v.T + dHz @ W_z.T
    Xf = X.reshape(-1, d)
    return {"X": dX, "W_u": Xf.T @ dHu.reshape(-1, e), "W_v": Xf.T @ dHv.reshape(-1, e),
            "W_z": Xf.T @ dHz.reshape(-1, s), "W_o": dW_o, "gamma": dgamma, "beta": dbeta, "relpos": drel}


# --------------------------------------------------------------------------
# incremental (token-by-token) causal decoding
# --------------------------------------------------------------------------

def flash_decode(X, W_u, W_v, W_z, W_o, gamma, beta, relpos, C, quad_scale=None, lin_scale=None,
                 use_rope=False):
    """Causal decoding one token at a time with a constant-size state.

    The chunk-level recurrence of the causal layer (wikillm, "Method" steps
    2-4; Su's post, "Mixed Chunking": the decoder's linear part as a
    cumulative sum over chunks; papercache 3.1, the incremental form of linear
    attention): the state is P, the sum of the summaries K_lin^T V of the
    chunks already completed (s x e), plus the current chunk's keys and
    values.  Token t at slot j = t mod C of its chunk:
      quad = sum over the chunk's slots tau <= j of
             relu^2(q_quad . k_quad_tau * quad_scale + w[C-1 + tau - j]) v_tau
      lin  = q_lin P;   o_t = (u * (quad + lin)) W_o
    and when j = C-1 the chunk's summary lin_scale * sum_tau k_lin_tau v_tau^T
    is added to P.  X may have any length T (no multiple of C needed).
    """
    X = _as64(X)
    B, T, d = X.shape
    if quad_scale is None:
        quad_scale = 1.0 / C
    if lin_scale is None:
        lin_scale = 1.0 / C
    W_u, W_v, W_z, W_o = map(_as64, (W_u, W_v, W_z, W_o))
    gamma, beta, w = _as64(gamma), _as64(beta), _as64(relpos)
    e, s = W_u.shape[1], W_z.shape[1]
    out = np.zeros((B, T, d))
    for b in range(B):
        P = np.zeros((s, e))
        kq_c, v_c, kl_c = [], [], []
        for t in range(T):
            x = X[b, t]
            u = silu(x @ W_u)
            v = silu(x @ W_v)
            z = silu(x @ W_z)
            qq, kq, ql, kl = (z * gamma[h] + beta[h] for h in range(4))
            if use_rope:
                qq, kq, ql, kl = (rope(h[None, :], [t])[0] for h in (qq, kq, ql, kl))
            j = t % C
            if j == 0:
                kq_c, v_c, kl_c = [], [], []
            kq_c.append(kq)
            v_c.append(v)
            kl_c.append(kl)
            quad = np.zeros(e)
            for tau in range(j + 1):
                sc = float(qq @ kq_c[tau]) * quad_scale + w[C - 1 + tau - j]
                quad += max(sc, 0.0) ** 2 * v_c[tau]
            lin = ql @ P
            out[b, t] = (u * (quad + lin)) @ W_o
            if j == C - 1:
                P = P + lin_scale * sum(np.outer(kl_c[tau], v_c[tau]) for tau in range(C))
    return out


# --------------------------------------------------------------------------
# references used by the invariant tests and by the stack configuration
# --------------------------------------------------------------------------

def glu(X, W_u, W_v, W_o):
    """GLU feed-forward O = (SiLU(X W_u) * SiLU(X W_v)) W_o.

    Blog, "Gated Attention" (GLU equation); the GAU reduces to it when A = I.
    """
    X = _as64(X)
    return (silu(X @ _as64(W_u)) * silu(X @ _as64(W_v))) @ _as64(W_o)


def linear_attention_recurrence(Q, K, V, scale):
    """Causal token-level linear attention through the running cache
    M_t = M_{t-1} + k_t v_t^T, output q_t M_{t-1} (strictly earlier tokens).

    papercache 3.1 (linear attention, the incremental form M_t).  Used to pin
    the chunked form at C = 1, where every chunk is one token.
    Q, K: (T, s); V: (T, e).
    """
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    T, s = Q.shape
    e = V.shape[1]
    M = np.zeros((s, e))
    out = np.zeros((T, e))
    for t in range(T):
        out[t] = Q[t] @ M
        M = M + scale * np.outer(K[t], V[t])
    return out


def rms_norm(x, eps=1e-6):
    """Pre-norm for the layer stack: x / sqrt(mean(x^2) + eps) over the last axis.

    The listings put a norm before each block and add the shortcut after it
    (wikillm, gau_block / flash_block pseudocode); the norm's body (Code 5) is
    missing from the pages, so this is ScaleNorm with its gain fixed at sqrt(d),
    which is an RMS norm.
    """
    x = _as64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def flash_stack_forward(X, layers, C, causal, quad_scale=None, lin_scale=None):
    """A stack of FLASH layers with pre-norm and residual adds:
    x <- x + flash_forward(rms_norm(x), layer weights).

    ``layers`` is a list of dicts with keys W_u, W_v, W_z, W_o, gamma, beta,
    relpos (pages' orientation, as for flash_forward).
    """
    x = _as64(X).copy()
    for L in layers:
        x = x + flash_forward(rms_norm(x), L["W_u"], L["W_v"], L["W_z"], L["W_o"],
                              L["gamma"], L["beta"], L["relpos"], C, causal,
                              quad_scale, lin_scale)
    return x
