"""Planted mistakes in the oracle must be caught by its pins.

Each case below rewrites one line of the oracle's source (on the CPU, in a throw-away module), swaps
the rewritten functions into the ``oracle`` package and runs the pin tests of the three oracle test
modules.  A case passes when at least one pin fails: a dropped sign, a swapped nibble order, a wrong
tie rule, an inverted scale, a lost subnormal range, an off-by-one segment index, a transposed
operand and a wrong constant are each detected.
"""

import contextlib
import importlib
import inspect
import os
import types

import pytest

import oracle
import oracle.nvfp4_oracle as _mod

from . import test_oracle_codecs as T_codec
from . import test_oracle_gemm as T_gemm
from . import test_oracle_quantize as T_quant

_SRC_PATH = inspect.getsourcefile(_mod)
with open(_SRC_PATH) as _f:
    _SRC = _f.read()

MUTATIONS = {
    "nibble_order_swapped": ("packed = (code[:, 0::2] | (code[:, 1::2] << 4))",
                             "packed = (code[:, 1::2] | (code[:, 0::2] << 4))"),
    "sign_dropped": ("code = (sign << 3) | idx", "code = idx"),
    "ties_away_from_zero": ("idx = np.where(tie, even, idx)", "idx = np.where(tie, jn, idx)"),
    "block_scale_times_six": ("gs6 = np.float32(g / np.float32(6.0))",
                              "gs6 = np.float32(g * np.float32(6.0))"),
    "element_ratio_inverted": ("r = np.where(nz, g / np.where(nz, sd, np.float32(1.0))",
                               "r = np.where(nz, np.where(nz, sd, np.float32(1.0)) / g"),
    "no_e4m3_subnormals": ("return m * 2.0 ** -9  # subnormal", "return 0.0 * m  # subnormal"),
    "dynamic_numerator_448": ("GLOBAL_SCALE_NUMERATOR = np.float32(E2M1_MAX * E4M3_MAX)",
                              "GLOBAL_SCALE_NUMERATOR = np.float32(E4M3_MAX)"),
    "segment_off_by_one": ("denom = ga * np.float64(seg_g[j])",
                           "denom = ga * np.float64(seg_g[(j + 1) % len(seg_g)])"),
    "weight_operand_transposed_blocks": ("W = decode_integers(w_codes, w_scales)\n    M, K = A.shape",
                                         "W = decode_integers(w_codes, w_scales)[:, ::-1]\n    M, K = A.shape"),
    "missing_power_of_two": ("C[:, lo:hi] = S[:, lo:hi].astype(np.float64) * 2.0 ** -20 / denom",
                             "C[:, lo:hi] = S[:, lo:hi].astype(np.float64) * 2.0 ** -18 / denom"),
    "e2m1_subnormal_value": ("return m * 0.5  # subnormal", "return m * 0.75  # subnormal"),
    "block_max_uses_signed_max": ("amax_b = ax.max(axis=2)", "amax_b = xb.max(axis=2)"),
    # the per-element tolerance scale of every GPU parity test
    "abs_bound_loosened_64x": (
        "B[:, lo:hi] = S[:, lo:hi].astype(np.float64) * 2.0 ** -20 / (ga * np.float64(seg_g[j]))",
        "B[:, lo:hi] = S[:, lo:hi].astype(np.float64) * 2.0 ** -14 / (ga * np.float64(seg_g[j]))"),
    "abs_bound_without_abs": ("A = np.abs(decode_integers(a_codes, a_scales))",
                              "A = decode_integers(a_codes, a_scales)"),
    "abs_bound_segment_off_by_one": (
        "/ (ga * np.float64(seg_g[j]))\n    return B",
        "/ (ga * np.float64(seg_g[(j + 1) % len(seg_g)]))\n    return B"),
}


@contextlib.contextmanager
def _mutated(old, new):
    assert _SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = _SRC_PATH
    exec(compile(_SRC.replace(old, new), _SRC_PATH, "exec"), mod.__dict__)
    saved = {}
    for name in oracle.__dict__:
        if not name.startswith("_") and hasattr(mod, name):
            saved[name] = getattr(oracle, name)
            setattr(oracle, name, getattr(mod, name))
    try:
        yield
    finally:
        for name, v in saved.items():
            setattr(oracle, name, v)


def _pins():
    """The oracle's pin tests, called with fixed parameters."""
    return [
        T_codec.test_e2m1_value_set_is_the_ocp_set,
        T_codec.test_e4m3_decode_matches_torch_for_every_code,
        T_codec.test_e4m3_encode_windows_around_every_midpoint,
        T_codec.test_e2m1_windows_around_every_threshold,
        T_codec.test_e2m1_brute_force_on_ties_and_neighbours,
        T_quant.test_worked_example_ties_and_packing,
        T_quant.test_worked_example_non_representable_scale,
        T_quant.test_worked_example_dynamic_scale_on_constant_tensor,
        T_quant.test_dynamic_global_scale_formula,
        T_quant.test_zero_and_signed_zero_blocks,
        T_quant.test_underflowed_scale_gives_zero_magnitudes,
        lambda: T_quant.test_block_max_gets_the_largest_code(1),
        T_quant.test_block_locality_of_an_outlier,
        T_quant.test_sign_symmetry,
        T_quant.test_error_bound_half_grid_step_times_scale,
        lambda: T_gemm.test_brute_force_exact_rationals(32),
        lambda: T_gemm.test_abs_bound_against_exact_rationals(16),
        T_gemm.test_abs_bound_of_a_cancelling_product,
        T_gemm.test_brute_force_hand_built_operands,
        T_gemm.test_one_hot_activation_selects_a_weight_column,
        T_gemm.test_fused_equals_concatenated_per_module_products,
        T_gemm.test_defective_fused_scale_closed_form_at_the_pages_ratios,
    ]


def test_unmutated_oracle_passes_every_pin():
    for pin in _pins():
        pin()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    caught = []
    with _mutated(old, new):
        for pin in _pins():
            try:
                pin()
            except Exception as e:  # AssertionError or a crash: either way the pin fired
                caught.append((getattr(pin, "__name__", "lambda"), type(e).__name__))
    assert caught, f"no pin caught mutation {name}"


# ---- the fake-quantization / statistics / harmonization oracle --------------------------------

import oracle.fake_quant as _fq_mod  # noqa: E402

from . import test_oracle_fake_quant as T_fq  # noqa: E402

_FQ_PATH = inspect.getsourcefile(_fq_mod)
with open(_FQ_PATH) as _f:
    _FQ_SRC = _f.read()

FQ_MUTATIONS = {
    "dequant_multiplies_by_g": ("(q / np.float32(g))", "(q * np.float32(g))"),
    "dominated_tie_counts": ("2.0 * amax * amax > total", "2.0 * amax * amax >= total"),
    "dominated_factor_dropped": ("2.0 * amax * amax > total", "amax * amax > total"),
    "error_sum_of_abs": ("err2 = (d * d).sum(axis=1)", "err2 = np.abs(d).sum(axis=1)"),
    "harmonize_to_the_largest_scale": ("gs = np.float32(seg_g.min())", "gs = np.float32(seg_g.max())"),
    "requantize_keeps_input_scale": ("return quantize(dequantize_f32(codes, scales, g_in), g_out)[:2]",
                                     "return quantize(dequantize_f32(codes, scales, g_in), g_in)[:2]"),
}


@contextlib.contextmanager
def _fq_mutated(old, new):
    assert _FQ_SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle.fake_quant_mutant")
    mod.__file__ = _FQ_PATH
    mod.__package__ = "oracle"
    exec(compile(_FQ_SRC.replace(old, new), _FQ_PATH, "exec"), mod.__dict__)
    saved = {}
    for name, v in list(vars(_fq_mod).items()):
        if not name.startswith("_") and callable(v) and hasattr(mod, name):
            saved[name] = v
            setattr(_fq_mod, name, getattr(mod, name))
    try:
        yield
    finally:
        for name, v in saved.items():
            setattr(_fq_mod, name, v)


def _fq_pins():
    return [getattr(T_fq, n) for n in dir(T_fq) if n.startswith("test_")]


def test_unmutated_fake_quant_oracle_passes_every_pin():
    for pin in _fq_pins():
        pin()


@pytest.mark.parametrize("name", sorted(FQ_MUTATIONS))
def test_planted_fake_quant_mistake_is_caught(name):
    old, new = FQ_MUTATIONS[name]
    caught = []
    with _fq_mutated(old, new):
        for pin in _fq_pins():
            try:
                pin()
            except Exception as e:
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"
