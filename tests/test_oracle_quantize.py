"""Pins of the oracle's tensor encoder (``oracle.quantize``).

The pages print no worked example, so the examples below are derived by hand from the format
definitions (the derivation is written next to each), and the rest are invariants that the pages'
description of block scaling implies (ai.info summary, "Methodology in Plain English" and "Main
Findings": the largest value in a 16-element block fixes its E4M3 scale, so an outlier degrades
only the 15 other elements of its block).
"""

import numpy as np
import pytest

import oracle
from workloads import random_matrix


def _codes(packed):
    return oracle.unpack_codes(packed)


# ------------------------------------------------------------------------------------------------
# hand-derived examples
# ------------------------------------------------------------------------------------------------


def test_worked_example_ties_and_packing():
    # g = 1, block [12, 5, -10, 1.5, 0.5, 3.5, 7, 0 x 9]:
    #   gs6 = fl(1/6); s = fl(12 * gs6) = 2.0 -> scale byte 0x40; r = 1/2.0 = 0.5
    #   y = [6, 2.5, 5, 0.75, 0.25, 1.75, 3.5, 0...]: every value after the first is a tie
    #   2.5 -> 2 (idx 4), 5 -> 4 (idx 6, negative: 0xE), 0.75 -> 1 (idx 2), 0.25 -> 0, 1.75 -> 2
    #   (idx 4), 3.5 -> 4 (idx 6); 6 -> idx 7
    #   codes [7, 4, E, 2, 0, 4, 6, 0...] -> bytes (low nibble first) [0x47, 0x2E, 0x40, 0x06, 0...]
    x = np.array([[12, 5, -10, 1.5, 0.5, 3.5, 7] + [0] * 9], np.float32)
    c, s, g = oracle.quantize(x, 1.0)
    assert s.tolist() == [[0x40]]
    assert c.tolist() == [[0x47, 0x2E, 0x40, 0x06, 0, 0, 0, 0]]
    # decoded: code value * 2.0 -> [12, 4, -8, 2, 0, 4, 8, 0...]; each error is half a grid step
    assert oracle.dequantize(c, s, g)[0, :7].tolist() == [12, 4, -8, 2, 0, 4, 8]


def test_worked_example_non_representable_scale():
    # g = 1, block [1.0, -0.3, 0 x 14]: s = fl(1 * fl(1/6)) = 0.16666667 -> nearest E4M3 is
    # 0.171875 = 1.375 * 2^-3 (code 0x23); r = fl(1/0.171875) = 5.818182
    # y0 = 5.818 -> 6 (idx 7); y1 = fl(0.3f * r) = 1.7454547 < 1.75 -> 1.5 (idx 3), negative: 0xB
    x = np.array([[1.0, -0.3] + [0] * 14], np.float32)
    c, s, g = oracle.quantize(x, 1.0)
    assert s.tolist() == [[0x23]]
    assert c.tolist() == [[0xB7, 0, 0, 0, 0, 0, 0, 0]]
    d = oracle.dequantize(c, s, g)[0, :2]
    assert d.tolist() == [6 * 0.171875, -1.5 * 0.171875]  # [1.03125, -0.2578125]


def test_worked_example_dynamic_scale_on_constant_tensor():
    # dynamic g = fl(2688 / fl32(0.7)) = 3840; s = fl(0.7f * fl(3840/6)) = fl(0.7f * 640) = 448
    # -> 0x7E; r = 3840/448 = 8.571428; y = fl(0.7f * r) = 6.0 -> idx 7
    x = np.full((3, 32), 0.7, np.float32)
    c, s, g = oracle.quantize(x)
    assert g == np.float32(3840.0)
    assert np.all(s == 0x7E)
    assert np.all(c == 0x77)
    np.testing.assert_allclose(oracle.dequantize(c, s, g), 0.7, rtol=1e-7)


def test_dynamic_global_scale_formula():
    # 2688 = 6 (largest E2M1) * 448 (largest E4M3)
    assert oracle.GLOBAL_SCALE_NUMERATOR == np.float32(2688.0)
    x = np.zeros((2, 16), np.float32)
    x[1, 5] = -3.0
    assert oracle.dynamic_global_scale(x) == np.float32(896.0)
    assert oracle.dynamic_global_scale(np.zeros((4, 16), np.float32)) == np.float32(1.0)
    # with the dynamic scale the tensor's largest block gets the largest scale code
    c, s, g = oracle.quantize(random_matrix(3, 8, 64))
    assert s.max() == 0x7E


def test_zero_and_signed_zero_blocks():
    x = np.zeros((2, 32), np.float32)
    x[1, :16] = -0.0
    c, s, g = oracle.quantize(x, 7.0)
    assert np.all(s == 0)
    codes = _codes(c)
    assert np.all(codes[0] == 0)
    assert np.all(codes[1, :16] == 0x8) and np.all(codes[1, 16:] == 0)
    assert np.all(oracle.dequantize(c, s, g) == 0)


def test_negative_values_that_round_to_zero_keep_the_sign():
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1], x[0, 2] = 6.0, -0.1, 0.1
    c, s, g = oracle.quantize(x, 1.0)  # s = 1.0, r = 1, y = 0.1 -> 0
    assert _codes(c)[0, :3].tolist() == [0x7, 0x8, 0x0]


def test_underflowed_scale_gives_zero_magnitudes():
    # amax * g / 6 <= 2^-10 rounds the scale to 0: every element gets magnitude 0
    x = np.full((1, 16), 1e-4, np.float32)
    x[0, 3] = -2e-4
    c, s, g = oracle.quantize(x, 1.0)
    assert s.tolist() == [[0]]
    assert _codes(c)[0].tolist() == [0] * 3 + [8] + [0] * 12


def test_saturating_scale_with_under_calibrated_global_scale():
    # a static g four times too large: blocks whose amax*g/6 >= 448 saturate to 0x7E and their
    # large elements saturate to code 7 (6.0)
    x = random_matrix(5, 16, 64)
    g_cal = oracle.dynamic_global_scale(x)
    c, s, _ = oracle.quantize(x, g_cal * 4)
    assert np.any(s == 0x7E)
    codes = _codes(c)
    sat = np.repeat(s == 0x7E, 16, axis=1)
    assert np.all(codes[sat].max() <= 0xF)
    assert np.any((codes[sat] & 7) == 7)


# ------------------------------------------------------------------------------------------------
# invariants of block scaling
# ------------------------------------------------------------------------------------------------


def _normal_scale_blocks(s):
    return (s >= 0x08) & (s < 0x7E)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_block_max_gets_the_largest_code(seed):
    # s = amax * g/6 -> sd within half an E4M3 step of s, so y_max = amax * g / sd is in
    # [6/(1+1/16), 6/(1-1/16)] = [5.65, 6.4] > 5: the block's largest element encodes as 6
    x = random_matrix(seed, 64, 256, outlier_cols=4)
    g = np.float32(oracle.dynamic_global_scale(x) / 8)
    c, s, g = oracle.quantize(x, g)
    codes = _codes(c).reshape(64, 16, 16)
    xb = np.abs(x.reshape(64, 16, 16))
    arg = xb.argmax(axis=2)
    top = np.take_along_axis(codes, arg[..., None], axis=2)[..., 0] & 7
    mask = _normal_scale_blocks(s)
    assert mask.sum() > 500
    assert np.all(top[mask] == 7)


def test_block_locality_of_an_outlier():
    # static g: changing one element changes codes and the scale only inside its own block
    x = random_matrix(21, 4, 128)
    g = np.float32(300.0)
    c0, s0, _ = oracle.quantize(x, g)
    y = x.copy()
    y[2, 37] = 80.0  # an outlier in block 2 of row 2
    c1, s1, _ = oracle.quantize(y, g)
    d_scale = np.argwhere(s0 != s1)
    assert d_scale.tolist() == [[2, 2]]
    d_codes = np.argwhere(_codes(c0) != _codes(c1))
    assert np.all(d_codes[:, 0] == 2)
    assert np.all(d_codes[:, 1] // 16 == 2)
    assert len(d_codes) > 1  # the 15 neighbours were degraded too


@pytest.mark.parametrize("k", [-20, -7, -1, 1, 5, 20])
def test_power_of_two_scaling_with_dynamic_scale(k):
    x = random_matrix(31, 8, 96, outlier_cols=2)
    c0, s0, g0 = oracle.quantize(x)
    c1, s1, g1 = oracle.quantize((x * np.float32(2.0 ** k)).astype(np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert g1 == np.float32(g0 * np.float32(2.0 ** -k))


def test_power_of_two_scaling_with_static_scale():
    x = random_matrix(32, 8, 96)
    g = np.float32(123.25)
    c0, s0, _ = oracle.quantize(x, g)
    c1, s1, _ = oracle.quantize((x * np.float32(8.0)).astype(np.float32), g / np.float32(8.0))
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)


def test_sign_symmetry():
    x = random_matrix(41, 16, 64, outlier_cols=3)
    c0, s0, g0 = oracle.quantize(x)
    c1, s1, g1 = oracle.quantize(-x)
    assert g0 == g1 and np.array_equal(s0, s1)
    assert np.array_equal(_codes(c0) ^ 0x8, _codes(c1))


def test_error_bound_half_grid_step_times_scale():
    # for blocks whose unrounded scale is in the E4M3 normal range, |x - dq| <= half the E2M1 grid
    # step at the decoded point, times sd/g (plus a few ulps of the float32 steps)
    x = random_matrix(51, 128, 512, outlier_cols=5)
    g = oracle.dynamic_global_scale(x)
    c, s, g = oracle.quantize(x, g)
    dq = oracle.dequantize(c, s, g)
    codes = _codes(c) & 7
    step = np.array([0.5, 0.5, 0.5, 0.5, 1.0, 1.0, 2.0, 2.0])[codes]  # spacing around the code
    sd = np.repeat(oracle.e4m3_decode(s), 16, axis=1)
    bound = 0.5 * step * sd / np.float64(g) * (1 + 1e-6)
    mask = np.repeat(_normal_scale_blocks(s), 16, axis=1)
    err = np.abs(x.astype(np.float64) - dq)
    assert np.all(err[mask] <= bound[mask])


def test_constant_blocks_identical_codes():
    # a constant block gives 16 identical codes; with a normal-range scale they are all 7 (+-6),
    # and it decodes exactly when c*g/6 is an E4M3 value (here c*g/6 = 2.0)
    x = np.concatenate([np.full((1, 16), 3.0), np.full((1, 16), -0.37)], axis=1).astype(np.float32)
    c, s, g = oracle.quantize(x, 4.0)
    codes = _codes(c)
    assert np.all(codes[0, :16] == 7) and np.all(codes[0, 16:] == 0xF)
    assert oracle.dequantize(c, s, g)[0, 0] == 3.0


def test_quantization_error_plausibility_band():
    # sanity only, not a pin: per-token relative error of N(0,1) rows with a few hot channels is
    # of the order of the 7.5-9.2% the pages report for real activations
    x = random_matrix(61, 256, 1024, outlier_cols=10)
    c, s, g = oracle.quantize(x)
    dq = oracle.dequantize(c, s, g)
    rel = np.linalg.norm(x - dq, axis=1) / np.linalg.norm(x, axis=1)
    assert 0.03 < np.median(rel) < 0.2


def test_shapes_and_empty_inputs():
    c, s, g = oracle.quantize(np.zeros((0, 32), np.float32), 1.0)
    assert c.shape == (0, 16) and s.shape == (0, 2)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 24), np.float32), 1.0)
    with pytest.raises(ValueError):
        oracle.quantize(np.zeros((2, 32), np.float32), 0.0)
