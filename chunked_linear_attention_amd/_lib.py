"""ctypes binding of libgau (include/gau.h).  Argument marshalling only: every
step of the layer runs in the HIP kernels behind these calls.

The functions take torch tensors for device memory and the current HIP stream
of PyTorch; they check dtype/device/contiguity, pass raw pointers, and raise on
a non-OK status.  There is no fallback: without the built library (see
chunked_linear_attention_amd.build) importing this module's loader fails.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgau.so")

GAU_F32 = 0
GAU_BF16 = 1

STAGE_PROJ, STAGE_SCORES, STAGE_STATE, STAGE_SCAN, STAGE_ATTN, STAGE_OUT = range(6)

STATUS = {
    0: "GAU_OK", 1: "GAU_ERR_NULL", 2: "GAU_ERR_SHAPE", 3: "GAU_ERR_ALIGN",
    4: "GAU_ERR_DTYPE", 5: "GAU_ERR_WORKSPACE", 6: "GAU_ERR_HIP",
}

# Every symbol include/gau.h and include/gau_probe.h declare.
EXPORTS = (
    "gau_workspace_bytes", "gau_workspace_layout", "gau_forward", "gau_forward_stages",
    "gau_stack_workspace_bytes", "gau_stack_forward", "gau_decode_workspace_bytes", "gau_decode_reset",
    "gau_decode_step", "gau_rope_relpos", "gau_backward_workspace_bytes", "gau_backward", "gau_status_string",
    "gau_probe_mfma", "gau_forward_noalloc", "gau_forward_segmented", "gau_backward_segmented",
)

# include/gau.h: the size of gau_forward_noalloc's device scratch array
NOALLOC_SCRATCH_BYTES = 64 << 20


class GauConfig(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("d", ctypes.c_int64),
                ("e", ctypes.c_int64), ("s", ctypes.c_int64), ("C", ctypes.c_int64),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("quad_scale", ctypes.c_float), ("lin_scale", ctypes.c_float), ("rope", ctypes.c_int32),
                ("ablation", ctypes.c_int32)]

# gau_config.ablation values
GAU_FULL, GAU_LOCAL_ONLY, GAU_GLOBAL_ONLY = 0, 1, 2
_PARTS = {"both": GAU_FULL, "local": GAU_LOCAL_ONLY, "global": GAU_GLOBAL_ONLY}


class GauWsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("U", "Vt", "Q_quad", "K_quad", "Q_lin", "K_lin_t", "S", "P", "A", "Y", "total")]


class GauError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


_lib = None


def load():
    """Load libgau.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m chunked_linear_attention_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    cfgp = ctypes.POINTER(GauConfig)
    lib.gau_workspace_bytes.argtypes = [cfgp]
    lib.gau_workspace_bytes.restype = ctypes.c_size_t
    lib.gau_workspace_layout.argtypes = [cfgp, ctypes.POINTER(GauWsLayout)]
    lib.gau_workspace_layout.restype = ctypes.c_int
    layer = [P] * 5 + [P] * 3 + [P, P, ctypes.c_size_t, P]
    lib.gau_forward.argtypes = [cfgp] + layer
    lib.gau_forward.restype = ctypes.c_int
    lib.gau_forward_stages.argtypes = [cfgp, ctypes.c_int, ctypes.c_int] + layer
    lib.gau_forward_stages.restype = ctypes.c_int
    lib.gau_forward_noalloc.argtypes = [cfgp] + [P] * 5 + [P] * 3 + [P, P]
    lib.gau_forward_noalloc.restype = ctypes.c_int
    lib.gau_forward_segmented.argtypes = [cfgp, P] + layer
    lib.gau_forward_segmented.restype = ctypes.c_int
    lib.gau_stack_workspace_bytes.argtypes = [cfgp]
    lib.gau_stack_workspace_bytes.restype = ctypes.c_size_t
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.gau_stack_forward.argtypes = [cfgp, ctypes.c_int, P] + [PP] * 7 + [P, ctypes.c_size_t, P]
    lib.gau_stack_forward.restype = ctypes.c_int
    lib.gau_decode_workspace_bytes.argtypes = [cfgp]
    lib.gau_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.gau_decode_reset.argtypes = [cfgp, P, ctypes.c_size_t, P]
    lib.gau_decode_reset.restype = ctypes.c_int
    lib.gau_decode_step.argtypes = [cfgp, ctypes.c_int64] + layer
    lib.gau_decode_step.restype = ctypes.c_int
    lib.gau_rope_relpos.argtypes = [P, P, ctypes.c_int64, ctypes.c_int64, P, P]
    lib.gau_rope_relpos.restype = ctypes.c_int
    lib.gau_backward_workspace_bytes.argtypes = [cfgp]
    lib.gau_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.gau_backward.argtypes = [cfgp] + [P] * 18 + [ctypes.c_size_t, P]
    lib.gau_backward.restype = ctypes.c_int
    lib.gau_backward_segmented.argtypes = [cfgp] + [P] * 19 + [ctypes.c_size_t, P]
    lib.gau_backward_segmented.restype = ctypes.c_int
    lib.gau_status_string.argtypes = [ctypes.c_int]
    lib.gau_status_string.restype = ctypes.c_char_p
    lib.gau_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, P, P]
    lib.gau_probe_mfma.restype = ctypes.c_int
    _lib = lib
    return lib


def make_config(B, T, d, e, s, C, causal, dtype, quad_scale=None, lin_scale=None, rope=False, parts="both"):
    """gau_config; quad_scale / lin_scale default to 1/C (the listing's reading);
    rope rotates the four heads by position; parts "local" / "global" keeps
    only that term (the LocalOnly / GlobalOnly variants)."""
    return GauConfig(B, T, d, e, s, C, 1 if causal else 0, dtype,
                     (1.0 / C) if quad_scale is None else float(quad_scale),
                     (1.0 / C) if lin_scale is None else float(lin_scale), 1 if rope else 0, _PARTS[parts])


def workspace_bytes(cfg):
    return load().gau_workspace_bytes(ctypes.byref(cfg))


def stack_workspace_bytes(cfg):
    return load().gau_stack_workspace_bytes(ctypes.byref(cfg))


def workspace_layout(cfg):
    L = GauWsLayout()
    st = load().gau_workspace_layout(ctypes.byref(cfg), ctypes.byref(L))
    if st != 0:
        raise GauError(st, "gau_workspace_layout")
    return {n: getattr(L, n) for n, _ in GauWsLayout._fields_}


def status_string(status):
    return load().gau_status_string(status).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(t, name, dtype=None, numel=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _torch_dtype(cfg):
    import torch
    return torch.bfloat16 if cfg.dtype == GAU_BF16 else torch.float32


def _check_layer(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O, T=None):
    import torch
    dt = _torch_dtype(cfg)
    B, d, e, s, C = cfg.B, cfg.d, cfg.e, cfg.s, cfg.C
    T = cfg.T if T is None else T
    _check(X, "X", dt, B * T * d)
    _check(W_u, "W_u", dt, e * d)
    _check(W_v, "W_v", dt, e * d)
    _check(W_z, "W_z", dt, s * d)
    _check(W_o, "W_o", dt, d * e)
    _check(scale, "scale", torch.float32, 4 * s)
    _check(offset, "offset", torch.float32, 4 * s)
    _check(relpos, "relpos", torch.float32, 2 * C - 1)
    _check(O, "O", dt, B * T * d)


def forward_stages(cfg, first, last, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O, workspace,
                   stream=None):
    """gau_forward_stages on torch tensors (weights output-major, see gau.h)."""
    _check_layer(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O)
    _check(workspace, "workspace")
    st = load().gau_forward_stages(
        ctypes.byref(cfg), first, last, _ptr(X), _ptr(W_u), _ptr(W_v), _ptr(W_z), _ptr(W_o),
        _ptr(scale), _ptr(offset), _ptr(relpos), _ptr(O), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_forward_stages")


def forward(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O, workspace, stream=None):
    """gau_forward on torch tensors (weights output-major, see gau.h)."""
    _check_layer(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O)
    _check(workspace, "workspace")
    st = load().gau_forward(
        ctypes.byref(cfg), _ptr(X), _ptr(W_u), _ptr(W_v), _ptr(W_z), _ptr(W_o),
        _ptr(scale), _ptr(offset), _ptr(relpos), _ptr(O), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_forward")


def forward_segmented(cfg, chunk_segments, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O, workspace,
                      stream=None):
    """gau_forward_segmented: the layer over packed sequences; chunk_segments
    is an int32 device tensor [B, T / C] of per-chunk segment ids."""
    import torch
    _check_layer(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O)
    _check(chunk_segments, "chunk_segments", torch.int32, cfg.B * (cfg.T // cfg.C))
    _check(workspace, "workspace")
    st = load().gau_forward_segmented(
        ctypes.byref(cfg), _ptr(chunk_segments), _ptr(X), _ptr(W_u), _ptr(W_v), _ptr(W_z), _ptr(W_o),
        _ptr(scale), _ptr(offset), _ptr(relpos), _ptr(O), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_forward_segmented")


def forward_noalloc(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O, stream=None):
    """gau_forward_noalloc: gau_forward with the workspace in the library's
    device scratch array (no allocation; gau_workspace_bytes(cfg) must not
    exceed NOALLOC_SCRATCH_BYTES)."""
    _check_layer(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, O)
    st = load().gau_forward_noalloc(
        ctypes.byref(cfg), _ptr(X), _ptr(W_u), _ptr(W_v), _ptr(W_z), _ptr(W_o),
        _ptr(scale), _ptr(offset), _ptr(relpos), _ptr(O), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_forward_noalloc")


def stack_forward(cfg, X, layers, workspace, stream=None):
    """gau_stack_forward: X (fp32 [B, T, d]) is updated in place.  ``layers`` is
    a list of dicts of device tensors W_u, W_v, W_z, W_o (output-major), scale,
    offset, relpos."""
    import torch
    _check(X, "X", torch.float32, cfg.B * cfg.T * cfg.d)
    _check(workspace, "workspace")
    n = len(layers)
    arrs = {}
    for k in ("W_u", "W_v", "W_z", "W_o", "scale", "offset", "relpos"):
        for i, L in enumerate(layers):
            _check(L[k], f"layers[{i}].{k}")
        arrs[k] = (ctypes.c_void_p * max(n, 1))(*[L[k].data_ptr() for L in layers])
    for L in layers:
        _check_layer(cfg, None, L["W_u"], L["W_v"], L["W_z"], L["W_o"], L["scale"], L["offset"],
                     L["relpos"], None)
    cast = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
    st = load().gau_stack_forward(
        ctypes.byref(cfg), n, _ptr(X), *[cast(arrs[k]) for k in
                                        ("W_u", "W_v", "W_z", "W_o", "scale", "offset", "relpos")],
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_stack_forward")


def probe_mfma(blocks, iters, out, stream=None):
    """gau_probe_mfma (measurement aid, gau_probe.h): queues the register-only
    MFMA probe; returns its FLOPs per launch.  `out` is a device fp32 tensor."""
    import torch
    _check(out, "out", torch.float32, 1)
    st = load().gau_probe_mfma(int(blocks), int(iters), _ptr(out), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_probe_mfma")
    return float(blocks) * 4 * iters * 16 * 32768


def rope_relpos(a, b, n, out=None, stream=None):
    """gau_rope_relpos: the 2n-1 bias vector of Code 4's RoPE branch from the
    fp32 device vectors a and b (same length)."""
    import torch
    _check(a, "a", torch.float32)
    _check(b, "b", torch.float32, a.numel())
    if out is None:
        out = torch.empty(2 * n - 1, dtype=torch.float32, device=a.device)
    _check(out, "out", torch.float32, 2 * n - 1)
    st = load().gau_rope_relpos(_ptr(a), _ptr(b), n, a.numel(), _ptr(out), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_rope_relpos")
    return out


def decode_workspace_bytes(cfg):
    return load().gau_decode_workspace_bytes(ctypes.byref(cfg))


def decode_reset(cfg, workspace, stream=None):
    """gau_decode_reset: clear the decoding state (before position 0)."""
    _check(workspace, "workspace")
    st = load().gau_decode_reset(ctypes.byref(cfg), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    if st != 0:
        raise GauError(st, "gau_decode_reset")


def decode_step(cfg, t, x, W_u, W_v, W_z, W_o, scale, offset, relpos, o, workspace, stream=None):
    """gau_decode_step: o [B, d] = the causal layer's outputs at position t for
    the tokens x [B, d], advancing the state in ``workspace``."""
    _check_layer(cfg, x, W_u, W_v, W_z, W_o, scale, offset, relpos, o, T=1)
    _check(workspace, "workspace")
    st = load().gau_decode_step(
        ctypes.byref(cfg), int(t), _ptr(x), _ptr(W_u), _ptr(W_v), _ptr(W_z), _ptr(W_o), _ptr(scale), _ptr(offset),
        _ptr(relpos), _ptr(o), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if st != 0:
        raise GauError(st, "gau_decode_step")


def backward_workspace_bytes(cfg):
    return load().gau_backward_workspace_bytes(ctypes.byref(cfg))


# gradient names, in the order gau_backward takes its outputs
GRAD_NAMES = ("X", "W_u", "W_v", "W_z", "W_o", "scale", "offset", "relpos")


def backward(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, dO, grads, workspace, stream=None,
             chunk_segments=None):
    """gau_backward on torch tensors: fills ``grads`` (a dict of fp32 device
    tensors named as GRAD_NAMES; the weight gradients output-major like the
    weights) with the gradients of <dO, O>.  With chunk_segments (an int32
    device tensor [B, T / C]) gau_backward_segmented, the backward of
    gau_forward_segmented."""
    import torch
    _check_layer(cfg, X, W_u, W_v, W_z, W_o, scale, offset, relpos, dO)
    B, T, d, e, s, C = cfg.B, cfg.T, cfg.d, cfg.e, cfg.s, cfg.C
    sizes = {"X": B * T * d, "W_u": e * d, "W_v": e * d, "W_z": s * d, "W_o": d * e, "scale": 4 * s,
             "offset": 4 * s, "relpos": 2 * C - 1}
    for k in GRAD_NAMES:
        _check(grads[k], "d" + k, torch.float32, sizes[k])
    _check(workspace, "workspace")
    tail = (_ptr(X), _ptr(W_u), _ptr(W_v), _ptr(W_z), _ptr(W_o), _ptr(scale), _ptr(offset), _ptr(relpos),
            _ptr(dO), *[_ptr(grads[k]) for k in GRAD_NAMES], _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if chunk_segments is None:
        st = load().gau_backward(ctypes.byref(cfg), *tail)
        name = "gau_backward"
    else:
        _check(chunk_segments, "chunk_segments", torch.int32, B * (T // C))
        st = load().gau_backward_segmented(ctypes.byref(cfg), _ptr(chunk_segments), *tail)
        name = "gau_backward_segmented"
    if st != 0:
        raise GauError(st, name)
