"""Host-side checks of libgau's C ABI: the library loads, exports every symbol
include/gau.h declares, and rejects bad arguments before touching a GPU.
CPU only: no call here launches a kernel."""

import ctypes
import os
import re

import pytest

import chunked_linear_attention_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    inc = os.path.join(ROOT, "include")
    txt = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gau_[a-z_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported():
    lib = g.load()
    decl = _declared()
    assert decl, "no declarations found"
    assert set(decl) == set(g.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def _cfg(**kw):
    base = dict(B=2, T=512, d=256, e=512, s=128, C=128, causal=True, dtype=g.GAU_BF16)
    base.update(kw)
    return g.make_config(**base)


def test_workspace_layout_sizes():
    cfg = _cfg()
    L = g.workspace_layout(cfg)
    M, e, s, B, G = 2 * 512, 512, 128, 2, 4
    assert L["Vt"] - L["U"] >= M * e * 2
    assert L["Y"] == L["U"]                             # the gate is applied in place
    assert L["P"] == L["S"]                             # causal: the scan runs in place
    assert L["A"] - L["S"] >= B * G * e * s * 2
    assert L["total"] - L["A"] >= B * G * 128 * 128 * 2
    assert L["total"] == g.workspace_bytes(cfg)
    for k, v in L.items():
        assert v % 256 == 0, k
    nc = g.workspace_layout(_cfg(causal=False))
    assert nc["Y"] == nc["U"]
    assert nc["A"] - nc["S"] >= B * G * e * s * 2       # S kept: the totals overwrite nothing
    assert nc["P"] - nc["A"] >= B * G * 128 * 128 * 2
    assert nc["total"] - nc["P"] >= B * 1 * e * s * 2   # one total per sequence
    assert nc["total"] > L["total"]
    f32 = g.workspace_layout(_cfg(dtype=g.GAU_F32))
    assert f32["total"] > L["total"]


@pytest.mark.parametrize("bad", [dict(T=500), dict(C=32), dict(C=96), dict(d=200), dict(e=384),
                                 dict(s=64), dict(s=192), dict(B=-1),
                                 # B * e * s = 2^33: the chunk scan's lanes would reach 2^31
                                 dict(B=8192, T=128, C=128, d=128, e=8192, s=128)])
def test_bad_shapes_rejected(bad):
    cfg = _cfg(**bad)
    assert g.workspace_bytes(cfg) == 0
    with pytest.raises(g.GauError) as ei:
        g.workspace_layout(cfg)
    assert ei.value.status == 2


def test_bad_rope_flag_rejected():
    cfg = _cfg()
    cfg.rope = 2
    assert g.workspace_bytes(cfg) == 0
    cfg.rope = 1
    assert g.workspace_bytes(cfg) == g.workspace_bytes(_cfg())


def test_bad_ablation_rejected():
    cfg = _cfg()
    cfg.ablation = 3
    assert g.workspace_bytes(cfg) == 0
    for a in (g.GAU_LOCAL_ONLY, g.GAU_GLOBAL_ONLY):
        cfg.ablation = a
        assert g.workspace_bytes(cfg) == g.workspace_bytes(_cfg())


def test_rope_relpos_argument_checks_without_gpu():
    lib = g.load()
    P = ctypes.c_void_p
    a, b, w = P(4096), P(8192), P(12288)
    assert lib.gau_rope_relpos(None, b, 64, 128, w, None) == 1
    assert lib.gau_rope_relpos(a, b, 64, 128, None, None) == 1
    assert lib.gau_rope_relpos(a, b, 0, 128, w, None) == 2
    assert lib.gau_rope_relpos(a, b, 64, 127, w, None) == 2
    assert lib.gau_rope_relpos(P(4100), b, 64, 128, w, None) == 3


def test_decode_argument_checks_without_gpu():
    lib = g.load()
    cfg = _cfg()
    ws = g.decode_workspace_bytes(cfg)
    assert ws > 0 and g.decode_workspace_bytes(_cfg(causal=False)) == 0
    good = [ctypes.c_void_p(4096 * (i + 1)) for i in range(10)]
    call = lambda c, t, ptrs, n: lib.gau_decode_step(ctypes.byref(c), t, *ptrs, ctypes.c_size_t(n), None)
    assert call(_cfg(causal=False), 0, good, ws) == 2       # decoding is causal only
    assert call(cfg, -1, good, ws) == 2
    assert call(cfg, cfg.T, good, ws) == 2                  # positions 0 .. T-1
    assert call(cfg, 0, good, ws - 1) == 5
    assert call(cfg, 0, [None] + good[1:], ws) == 1
    bad = list(good)
    bad[8] = ctypes.c_void_p(4096 * 9 + 4)
    assert call(cfg, 0, bad, ws) == 3                       # misaligned o
    assert call(_cfg(B=0), 0, [None] * 10, 0) == 0          # nothing to decode
    P = ctypes.c_void_p
    assert lib.gau_decode_reset(ctypes.byref(_cfg(causal=False)), P(4096), ctypes.c_size_t(ws), None) == 2
    assert lib.gau_decode_reset(ctypes.byref(cfg), P(4096), ctypes.c_size_t(ws - 1), None) == 5
    assert lib.gau_decode_reset(ctypes.byref(cfg), None, ctypes.c_size_t(ws), None) == 1


def test_backward_argument_checks_without_gpu():
    lib = g.load()
    cfg = _cfg()
    ws = g.backward_workspace_bytes(cfg)
    assert ws > g.workspace_bytes(cfg)                      # the forward's regions come first
    assert g.backward_workspace_bytes(_cfg(rope=True)) == ws  # the rotated and partial layers: same workspace
    assert g.backward_workspace_bytes(_cfg(parts="local")) == ws
    assert g.backward_workspace_bytes(_cfg(T=500)) == 0
    good = [ctypes.c_void_p(4096 * (i + 1)) for i in range(18)]
    call = lambda c, ptrs, n: lib.gau_backward(ctypes.byref(c), *ptrs, ctypes.c_size_t(n), None)
    assert call(cfg, good, ws - 1) == 5
    assert call(cfg, [None] + good[1:], ws) == 1            # NULL X
    assert call(cfg, good[:8] + [None] + good[9:], ws) == 1  # NULL dO
    assert call(cfg, good[:17] + [None], ws) == 1           # NULL workspace
    bad = list(good)
    bad[12] = ctypes.c_void_p(4096 * 13 + 4)
    assert call(cfg, bad, ws) == 3                          # misaligned dW_z
    # the segment-masked backward: the same checks plus its segment ids
    seg = lambda c, sg, ptrs, n: lib.gau_backward_segmented(ctypes.byref(c), sg, *ptrs, ctypes.c_size_t(n), None)
    assert seg(cfg, None, good, ws) == 1                    # NULL chunk_segments
    assert seg(cfg, ctypes.c_void_p(4096 * 40 + 4), good, ws) == 3  # misaligned chunk_segments
    assert seg(cfg, ctypes.c_void_p(4096 * 40), good, ws - 1) == 5
    assert seg(cfg, ctypes.c_void_p(4096 * 40), [None] + good[1:], ws) == 1
    grow = g.backward_workspace_bytes(_cfg(T=1024))
    assert grow > ws                                        # grows with the tokens
    assert g.backward_workspace_bytes(_cfg(dtype=g.GAU_F32)) > ws


def test_bad_dtype_rejected():
    cfg = _cfg()
    cfg.dtype = 7
    with pytest.raises(g.GauError) as ei:
        g.workspace_layout(cfg)
    assert ei.value.status == 4


def _call_forward(cfg, ptrs, ws_bytes):
    lib = g.load()
    return lib.gau_forward(ctypes.byref(cfg), *[ctypes.c_void_p(p) if p else None for p in ptrs],
                           ctypes.c_size_t(ws_bytes), None)


def test_forward_argument_checks_without_gpu():
    cfg = _cfg()
    good = [4096 * (i + 1) for i in range(10)]       # fake, aligned, never dereferenced
    ws = g.workspace_bytes(cfg)
    assert _call_forward(cfg, [None] + good[1:], ws) == 1           # NULL X
    assert _call_forward(cfg, good[:8] + [None, good[9]], ws) == 1  # NULL O
    bad = list(good)
    bad[3] += 8
    assert _call_forward(cfg, bad, ws) == 3                         # misaligned W_z
    assert _call_forward(cfg, good, ws - 1) == 5                    # workspace too small
    assert _call_forward(_cfg(T=500), good, ws) == 2
    empty = _cfg(B=0)
    assert _call_forward(empty, [None] * 10, 0) == 0                # B*T == 0: nothing to do


def test_stage_range_checks():
    lib = g.load()
    cfg = _cfg()
    good = [ctypes.c_void_p(4096 * (i + 1)) for i in range(10)]
    ws = ctypes.c_size_t(g.workspace_bytes(cfg))
    for first, last in [(-1, 5), (0, 6), (3, 2)]:
        assert lib.gau_forward_stages(ctypes.byref(cfg), first, last, *good, ws, None) == 2


def test_stack_argument_checks():
    lib = g.load()
    cfg = _cfg()
    arr = (ctypes.c_void_p * 1)(4096)
    pp = ctypes.cast(arr, ctypes.POINTER(ctypes.c_void_p))
    ws = g.stack_workspace_bytes(cfg)
    assert ws > g.workspace_bytes(cfg)
    assert lib.gau_stack_forward(ctypes.byref(cfg), 1, None, *[pp] * 7, ctypes.c_void_p(4096),
                                 ctypes.c_size_t(ws), None) == 1
    assert lib.gau_stack_forward(ctypes.byref(cfg), 1, ctypes.c_void_p(4096), *[pp] * 7,
                                 ctypes.c_void_p(4096), ctypes.c_size_t(ws - 1), None) == 5
    assert lib.gau_stack_forward(ctypes.byref(cfg), 0, None, *[pp] * 7, None, 0, None) == 0


def test_longest_bf16_sequence():
    """bf16 takes T up to 2^22 tokens per sequence (the matrix cores' 32-bit
    tile offsets over T-element rows); fp32, copied with 64-bit addresses,
    takes longer ones."""
    ok = _cfg(B=1, T=1 << 22, C=256, d=128, e=256, s=128)
    assert g.workspace_bytes(ok) > 0
    bad = _cfg(B=1, T=(1 << 22) + 256, C=256, d=128, e=256, s=128)
    assert g.workspace_bytes(bad) == 0
    with pytest.raises(g.GauError) as ei:
        g.workspace_layout(bad)
    assert ei.value.status == 2
    assert g.workspace_bytes(_cfg(B=1, T=(1 << 22) + 256, C=256, d=128, e=256, s=128, dtype=g.GAU_F32)) > 0


def test_largest_scan_grid_accepted():
    """Just under the bound: B * e * s = 2^33 - 2^22 (the scan's lanes stay
    below 2^31) is a valid shape."""
    cfg = _cfg(B=8191, T=128, C=128, d=128, e=8192, s=128)
    assert g.workspace_bytes(cfg) > 0


def test_noalloc_forward_argument_checks_without_gpu():
    """gau_forward_noalloc rejects NULL pointers and configurations whose
    workspace exceeds its 64 MiB scratch before anything touches a GPU."""
    lib = g.load()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: rejected first
    cfg = _cfg()
    assert lib.gau_forward_noalloc(ctypes.byref(cfg), *([None] * 8), None, None) == 1      # GAU_ERR_NULL
    big = _cfg(B=1, T=8192, d=768, e=1536, s=128, C=256)
    assert g.workspace_bytes(big) > g.NOALLOC_SCRATCH_BYTES
    assert lib.gau_forward_noalloc(ctypes.byref(big), *([fake] * 8), fake, None) == 5       # GAU_ERR_WORKSPACE
    assert lib.gau_forward_noalloc(ctypes.byref(_cfg(T=500)), *([fake] * 8), fake, None) == 2
    empty = _cfg(B=0)
    assert lib.gau_forward_noalloc(ctypes.byref(empty), *([None] * 8), None, None) == 0     # no tokens: no-op


def test_status_strings():
    for code in range(7):
        assert g.status_string(code)
    assert g.status_string(99) == "unknown status"


def test_mfma_probe_rejects_bad_arguments():
    """The measurement probe checks its arguments before any launch."""
    lib = g.load()
    assert lib.gau_probe_mfma(0, 10, None, None) == 2            # GAU_ERR_SHAPE
    assert lib.gau_probe_mfma(16, 0, None, None) == 2
    assert lib.gau_probe_mfma(16, (1 << 20) + 1, None, None) == 2
    assert lib.gau_probe_mfma(1 << 12, (1 << 10) + 1, None, None) == 2   # blocks * iters > 2^22
    assert lib.gau_probe_mfma(1 << 20, 1 << 20, None, None) == 2
    assert lib.gau_probe_mfma(16, 10, None, None) == 1           # GAU_ERR_NULL
    assert lib.gau_probe_mfma(16, 10, ctypes.c_void_p(8), None) == 3  # GAU_ERR_ALIGN
