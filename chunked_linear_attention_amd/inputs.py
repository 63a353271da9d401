"""Seeded synthetic inputs for the FLASH layer, shared by the tests, the
benchmark and the smoke check.

This module draws random numbers and rounds them; it holds none of the layer's
arithmetic.  It imports only numpy, so the CPU oracle and the HIP path can be
fed identical tensors without either importing the other.

Distributions (one seeded PCG64 stream per layer, drawn in this order):
  X ~ N(0, 1)                 (B, T, d)
  W_u, W_v ~ N(0, 1/d)        (d, e)
  W_z ~ N(0, 1/d)             (d, s)
  W_o ~ N(0, 1/e)             (e, d)
  gamma ~ N(1, 0.02^2)        (4, s)   scales of Q_quad, K_quad, Q_lin, K_lin
  beta = 0                    (4, s)   offsets
  relpos ~ N(0, 0.02^2)       (2C-1,)  relative-position bias vector
All are drawn in float32.  For bf16 workloads X and the four weight matrices
are rounded to bf16 (round to nearest, ties to even); gamma, beta and relpos
stay float32, which is the precision the library takes them in.

With heads="wide" (parity tests only) gamma and beta are redrawn after the
rest, from a stream of their own (seed + 104729), as
  gamma ~ N(1, 0.5^2), beta ~ N(0, 0.3^2)
so that every offset moves the output and a mix-up of two heads' scales is
far outside the bf16 tolerance; the other tensors keep their values.
"""

import numpy as np

# Workloads: a single layer (or a stack) with its shapes, precision and seed.
WORKLOADS = {
    "layer_fp32_B1_T256_d128_C64": dict(B=1, T=256, d=128, e=256, s=128, C=64,
                                        dtype="f32", causal=True, seed=1000),
    "layer_bf16_B8_T1024_d768_C256": dict(B=8, T=1024, d=768, e=1536, s=128, C=256,
                                          dtype="bf16", causal=True, seed=1001),
    "layer_bf16_B4_T4096_d768_C256": dict(B=4, T=4096, d=768, e=1536, s=128, C=256,
                                          dtype="bf16", causal=True, seed=1002),
    "layer_bf16_B4_T4096_d768_C256_noncausal": dict(B=4, T=4096, d=768, e=1536, s=128,
                                                    C=256, dtype="bf16", causal=False,
                                                    seed=1002),
    "layer_bf16_B2_T8192_d768_C512": dict(B=2, T=8192, d=768, e=1536, s=128, C=512,
                                          dtype="bf16", causal=True, seed=1003),
    "layer_bf16_B2_T8192_d768_C256": dict(B=2, T=8192, d=768, e=1536, s=128, C=256,
                                          dtype="bf16", causal=True, seed=1003),
    "layer_bf16_B2_T8192_d768_C256_rope": dict(B=2, T=8192, d=768, e=1536, s=128, C=256,
                                               dtype="bf16", causal=True, seed=1003, rope=True),
    # the same number of tokens as one long sequence and as many short ones
    # (cost linear in T: the two take the same time per token)
    "layer_bf16_B1_T131072_d768_C256": dict(B=1, T=131072, d=768, e=1536, s=128, C=256,
                                            dtype="bf16", causal=True, seed=1004),
    "layer_bf16_B16_T8192_d768_C256": dict(B=16, T=8192, d=768, e=1536, s=128, C=256,
                                           dtype="bf16", causal=True, seed=1004),
    "stack24_bf16_B2_T8192_d1024_C256": dict(B=2, T=8192, d=1024, e=2048, s=128, C=256,
                                             dtype="bf16", causal=True, layers=24,
                                             weight_seed=2000, x_seed=2100),
}

# The configuration the headline throughput is quoted on.
HEADLINE = "layer_bf16_B2_T8192_d768_C256"


def bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.

    Finite inputs only (the generators never produce inf or NaN).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    """uint16 bf16 bit patterns -> the float32 values they denote (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def round_bf16(x):
    """float32 values rounded to the nearest bf16 value, returned as float32."""
    return bf16_bits_to_f32(bf16_bits(x))


def _draw_weights(rng, d, e, s, C):
    W_u = rng.standard_normal((d, e), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    W_v = rng.standard_normal((d, e), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    W_z = rng.standard_normal((d, s), dtype=np.float32) * np.float32(1.0 / np.sqrt(d))
    W_o = rng.standard_normal((e, d), dtype=np.float32) * np.float32(1.0 / np.sqrt(e))
    gamma = np.float32(1.0) + np.float32(0.02) * rng.standard_normal((4, s), dtype=np.float32)
    beta = np.zeros((4, s), dtype=np.float32)
    relpos = np.float32(0.02) * rng.standard_normal((2 * C - 1,), dtype=np.float32)
    return dict(W_u=W_u, W_v=W_v, W_z=W_z, W_o=W_o, gamma=gamma, beta=beta, relpos=relpos)


def wide_heads(s, seed):
    """gamma ~ N(1, 0.5^2) and beta ~ N(0, 0.3^2), both (4, s) float32, from a
    stream of their own (seed + 104729)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    gamma = np.float32(1.0) + np.float32(0.5) * rng.standard_normal((4, s), dtype=np.float32)
    beta = np.float32(0.3) * rng.standard_normal((4, s), dtype=np.float32)
    return gamma, beta


def make_layer_inputs(B, T, d, e, s, C, seed, dtype="bf16", heads="workload", **_ignored):
    """All inputs of one layer as float32 numpy arrays in the pages' orientation
    (W_u is d x e, etc.).  For dtype "bf16" the matrices hold bf16-exact values.
    heads="wide" replaces gamma and beta by wide_heads(s, seed).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = rng.standard_normal((B, T, d), dtype=np.float32)
    out = dict(X=X)
    out.update(_draw_weights(rng, d, e, s, C))
    if heads == "wide":
        out["gamma"], out["beta"] = wide_heads(s, seed)
    elif heads != "workload":
        raise ValueError("heads must be 'workload' or 'wide'")
    if dtype == "bf16":
        for k in ("X", "W_u", "W_v", "W_z", "W_o"):
            out[k] = round_bf16(out[k])
    elif dtype != "f32":
        raise ValueError("dtype must be 'bf16' or 'f32'")
    return out


def device_normal_bf16(shape, seed):
    """X ~ N(0, 1) of `shape` drawn on the GPU by torch's seeded generator and
    rounded to bf16 (to nearest even), for sequences too long to draw on the
    host in a test's time (2^29 host draws take minutes).  Callers that check
    against the oracle hand it these same values."""
    import torch

    gen = torch.Generator(device="cuda").manual_seed(seed)
    return torch.randn(tuple(shape), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def make_output_grad(B, T, d, seed, dtype="bf16"):
    """A seeded upstream gradient dL/dO [B, T, d] (standard normal, bf16-exact
    for dtype "bf16"), float32."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    g = rng.standard_normal((B, T, d), dtype=np.float32)
    return round_bf16(g) if dtype == "bf16" else g


def make_stack_inputs(B, T, d, e, s, C, layers, weight_seed, x_seed, dtype="bf16", heads="workload",
                      **_ignored):
    """Inputs of a layer stack: X (float32, the residual stream) and a list of
    per-layer weight dicts, layer l drawn from seed weight_seed + l (with
    heads="wide", its gamma and beta from wide_heads(s, weight_seed + l))."""
    rng = np.random.Generator(np.random.PCG64(x_seed))
    X = rng.standard_normal((B, T, d), dtype=np.float32)
    Ls = []
    for l in range(layers):
        w = _draw_weights(np.random.Generator(np.random.PCG64(weight_seed + l)), d, e, s, C)
        if heads == "wide":
            w["gamma"], w["beta"] = wide_heads(s, weight_seed + l)
        elif heads != "workload":
            raise ValueError("heads must be 'workload' or 'wide'")
        if dtype == "bf16":
            for k in ("W_u", "W_v", "W_z", "W_o"):
                w[k] = round_bf16(w[k])
        Ls.append(w)
    return X, Ls


def workload_inputs(name, **overrides):
    """Inputs for a named workload; keyword overrides replace shape entries
    (used by tests to take a smaller slice of the same recipe)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(overrides)
    return cfg, make_layer_inputs(**cfg)
