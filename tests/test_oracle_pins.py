"""The oracle pinned to facts that do not come from itself (CPU only)."""
import numpy as np
import pytest

import oracle as O
import oracle_pins as P


@pytest.mark.parametrize("pin", [
    P.pin_lut_closed_form, P.pin_lut_vs_torch, P.pin_roundtrip, P.pin_worked_ties,
    P.pin_encode_vs_torch, P.pin_bf16, P.pin_grids, P.pin_scale_direction,
    P.pin_quant_invariants, P.pin_brute_force, P.pin_per_tensor, P.pin_sampled_rows, P.pin_int_partials, P.pin_special_cases,
    P.pin_cross_arm, P.pin_upcast, P.pin_dense_brute_force, P.pin_silu_glu,
    P.pin_abs_bounds, P.pin_within_bound, P.pin_cross_arm_metrics, P.pin_exp_correctly_rounded,
], ids=lambda f: f.__name__)
def test_pin(pin):
    ok, detail = pin(O)
    assert ok, detail


def test_quant_act_tail_group_uses_valid_channels_only():
    # K = 200: the second group has 72 channels; its amax ignores the (absent) rest.
    x = np.zeros((1, 200), np.float32)
    x[0, 150] = 3.0
    x[0, 10] = 100.0
    q, s = O.quant_act(x)
    assert s.shape == (1, 2)
    assert s[0, 1] == np.float32(3.0) / np.float32(448.0)
    assert q[0, 150] == 0x7E and q[0, 10] == 0x7E


def test_quant_act_saturates_after_division():
    # amax/448 rounded down makes amax/s exceed 448 slightly; the clamp keeps 0x7E.
    found = 0
    for a in np.linspace(1.0, 2.0, 4001, dtype=np.float32):
        s = np.float32(a) / np.float32(448)
        if np.float32(a) / s > np.float32(448):
            found += 1
            q, _ = O.quant_act(np.array([[a, -a]], np.float32))
            assert q[0, 0] == 0x7E and q[0, 1] == 0xFE
    assert found > 0


def test_nan_weight_code_propagates_in_both_arms():
    codes = np.full((2, 128), 0x38, np.uint8)
    codes[1, 5] = 0x7F
    scale = np.ones((1, 1), np.float32)
    x = np.ones((1, 128), np.float32)
    y = O.linear_w8a16(x, [(codes, scale)])
    assert np.isfinite(y[0, 0]) and np.isnan(y[0, 1])
    xq, xs = O.quant_act(x)
    y8 = O.linear_w8a8(xq, xs, [(codes, scale)])
    assert np.isfinite(y8[0, 0]) and np.isnan(y8[0, 1])


def test_within_bound_bf16_term():
    y_ref = np.array([1.0 + 2 ** -8], np.float64)
    y_bf16 = O.bf16_bits_to_f32(O.round_output(y_ref, "bf16"))
    ok, _ = O.within_bound(y_bf16, y_ref, np.zeros(1), bf16_out=True)
    assert ok
    ok, _ = O.within_bound(y_bf16, y_ref, np.zeros(1), bf16_out=False)
    assert not ok
