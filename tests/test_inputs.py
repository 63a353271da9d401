"""Host-side checks of the seeded input generator (CPU only)."""

import numpy as np
import torch

from chunked_linear_attention_amd import inputs


def test_bf16_rounding_ties_to_even():
    one = 1.0
    ulp = 2.0 ** -7                      # bf16 spacing just above 1.0
    x = np.array([one, one + ulp / 2, one + 3 * ulp / 2, one + ulp / 2 + 2 ** -20,
                  -one - ulp / 2, 0.0, 65504.0, 3.0e38], dtype=np.float32)
    bits = inputs.bf16_bits(x)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80             # tie, even mantissa kept
    assert bits[2] == 0x3F82             # tie, rounds up to the even neighbour
    assert bits[3] == 0x3F81             # above the tie
    assert bits[4] == 0xBF80
    assert bits[5] == 0x0000


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7.0
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(inputs.bf16_bits(x), ref)
    np.testing.assert_array_equal(inputs.round_bf16(x),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_shaped():
    cfg, a = inputs.workload_inputs("layer_fp32_B1_T256_d128_C64")
    _, b = inputs.workload_inputs("layer_fp32_B1_T256_d128_C64")
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert a["X"].shape == (1, 256, 128) and a["W_u"].shape == (128, 256)
    assert a["W_z"].shape == (128, 128) and a["W_o"].shape == (256, 128)
    assert a["gamma"].shape == (4, 128) and a["relpos"].shape == (127,)
    assert np.all(a["beta"] == 0)
    assert abs(float(a["gamma"].mean()) - 1.0) < 0.01


def test_bf16_workload_values_are_bf16_exact():
    _, a = inputs.workload_inputs("layer_bf16_B8_T1024_d768_C256", B=1, T=256)
    for k in ("X", "W_u", "W_v", "W_z", "W_o"):
        np.testing.assert_array_equal(inputs.round_bf16(a[k]), a[k])
    assert a["relpos"].dtype == np.float32


def test_wide_heads_change_only_gamma_and_beta():
    kw = dict(B=1, T=128, d=128, e=256, s=128, C=64, seed=7, dtype="bf16")
    a = inputs.make_layer_inputs(**kw)
    b = inputs.make_layer_inputs(heads="wide", **kw)
    for k in ("X", "W_u", "W_v", "W_z", "W_o", "relpos"):
        np.testing.assert_array_equal(a[k], b[k])
    assert b["beta"].shape == (4, 128) and b["gamma"].shape == (4, 128)
    assert 0.2 < float(b["beta"].std()) < 0.4 and abs(float(b["beta"].mean())) < 0.05
    assert 0.4 < float(b["gamma"].std()) < 0.6 and abs(float(b["gamma"].mean()) - 1.0) < 0.1
    # every head has its own scales and offsets
    for h in range(4):
        for k in range(h):
            assert np.max(np.abs(b["gamma"][h] - b["gamma"][k])) > 0.5
            assert np.max(np.abs(b["beta"][h] - b["beta"][k])) > 0.3
