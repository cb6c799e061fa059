"""Pins of the oracle's W4A4 product and of its fused-module forms.

* ``gemm_exact`` (int64 sum, rounded once) against an independent route: float64 dequantisation and
  the library routine ``numpy.matmul`` (agreement to ~1e-12 relative).
* Brute force on tiny shapes: each output element summed as exact rationals straight from the packed
  bytes (``oracle.element_value_exact`` indexes the bytes by hand, a separate decoding from the
  vectorised one), divided by the two global scales, several segments with distinct scales.
* The tolerance scale ``gemm_abs_bound`` (``sum_k |a*w| / (gA gW[seg])``, the quantity every GPU
  parity bound is a multiple of) against the same exact rationals, on operands whose bytes cover
  every E2M1 nibble, zero and subnormal E4M3 scales and both signs, and against a hand-built case
  where the product cancels to zero but the bound does not.
* Closed forms: one-hot activations select one weight row, constant activations give row sums.
* Fused-module invariants (ai.info summary, "Main Findings"): the per-segment fused product equals the
  concatenation of one product per module; the defective fused product (largest global scale applied
  to every segment) equals the correct one times ``gW[j] / max(gW)`` on segment ``j``, which at the
  pages' paired-scale ratios 1.82 and 2.75 is a relative error of 45.05% and 63.64% on the affected
  segment.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import random_matrix

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _operands(seed, M, N, K, segs=None, a_std=1.0, w_std=0.02):
    a = random_matrix(seed, M, K, std=a_std, outlier_cols=max(1, K // 100))
    w = random_matrix(seed + 1, N, K, std=w_std)
    ac, as_, ga = oracle.quantize(a)
    segs = [0, N] if segs is None else segs
    wc, ws, gw = oracle.quantize_segments(w, segs)
    return ac, as_, ga, wc, ws, gw, segs


@pytest.mark.parametrize("M,N,K,segs", [(7, 5, 48, None), (33, 40, 512, [0, 8, 24, 40]),
                                        (64, 256, 512, None)])
def test_exact_vs_float64_matmul(M, N, K, segs):
    ac, as_, ga, wc, ws, gw, segs = _operands(100 + M, M, N, K, segs)
    C = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    D = oracle.gemm_dequant_f64(ac, as_, ga, wc, ws, gw, segs)
    B = oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs)
    assert np.all(np.abs(C - D) <= 1e-12 * B + 1e-300)
    assert np.linalg.norm(C - D) <= 1e-13 * np.linalg.norm(C)


@pytest.mark.parametrize("K", [16, 32])
def test_brute_force_exact_rationals(K):
    M, N = 3, 5
    segs = [0, 2, 5]
    ac, as_, ga, wc, ws, gw, segs = _operands(7 + K, M, N, K, segs)
    C = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    for m in range(M):
        for n in range(N):
            j = 0 if n < 2 else 1
            acc = Fraction(0)
            for k in range(K):
                acc += oracle.element_value_exact(ac, as_, m, k) * oracle.element_value_exact(wc, ws, n, k)
            ref = acc / (Fraction(float(ga)) * Fraction(float(gw[j])))
            assert abs(Fraction(C[m, n]) - ref) <= abs(ref) * Fraction(1, 2 ** 51)


def _raw_operands(seed, M, N, K):
    """Random code and scale bytes: every nibble 0x0..0xF (both signed zeros), scale codes drawn
    from all 127 finite E4M3 codes 0x00..0x7E (zero, the seven subnormals, 448)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    as_ = rng.integers(0, 0x7F, (M, K // 16), dtype=np.uint8)
    ws = rng.integers(0, 0x7F, (N, K // 16), dtype=np.uint8)
    return ac, as_, wc, ws


@pytest.mark.parametrize("K", [16, 48])
def test_abs_bound_against_exact_rationals(K):
    M, N = 3, 4
    segs = [0, 1, 4]
    ac, as_, wc, ws = _raw_operands(60 + K, M, N, K)
    as_[0, 0] = 0x00  # a zero block
    ws[1, -1] = 0x01  # the smallest subnormal scale
    ga, gw = np.float32(3.0), np.array([0.75, 5.0], np.float32)
    B = oracle.gemm_abs_bound(ac, as_, ga, wc, ws, gw, segs)
    C = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    for m in range(M):
        for n in range(N):
            j = 0 if n < 1 else 1
            acc, acc_abs = Fraction(0), Fraction(0)
            for k in range(K):
                p = oracle.element_value_exact(ac, as_, m, k) * oracle.element_value_exact(wc, ws, n, k)
                acc += p
                acc_abs += abs(p)
            den = Fraction(float(ga)) * Fraction(float(gw[j]))
            ref_b, ref_c = acc_abs / den, acc / den
            assert abs(Fraction(B[m, n]) - ref_b) <= ref_b * Fraction(1, 2 ** 51)
            assert abs(Fraction(C[m, n]) - ref_c) <= ref_b * Fraction(1, 2 ** 51)


def test_abs_bound_of_a_cancelling_product():
    # A: one row, all elements +1.0 (code 0x2, scale 0x38 = 1.0).  W: one row whose first 8
    # elements are +1.5 and last 8 are -1.5 (codes 0x3 / 0xB, scale 0x38).  The product cancels to
    # exactly 0 while the bound is 16 * 1.5 / (gA gW) = 24 / (2 * 0.5) = 24.
    K = 16
    a_codes = np.full((1, 8), 0x22, np.uint8)
    w_codes = np.array([[0x33] * 4 + [0xBB] * 4], np.uint8)
    sc = np.full((1, 1), 0x38, np.uint8)
    assert oracle.gemm_exact(a_codes, sc, 2.0, w_codes, sc, [0.5]).tolist() == [[0.0]]
    assert oracle.gemm_abs_bound(a_codes, sc, 2.0, w_codes, sc, [0.5]).tolist() == [[24.0]]


def test_brute_force_hand_built_operands():
    # A row: codes all 0x2 (value 1.0) with scale 0x38 (1.0) -> the decoded row is all ones.
    # W row n: element k has code (k % 8) with scale 0x40 (2.0) -> values 2 * V[k % 8].
    # So C[0, n] = sum_k 2 * V[k % 8] / (gA gW) = 2 * 2 * (0+0.5+1+1.5+2+3+4+6) / (gA gW) for K=16.
    K = 16
    a_codes = np.full((1, K // 2), 0x22, np.uint8)
    a_scales = np.full((1, 1), 0x38, np.uint8)
    w_codes = np.array([[0x10, 0x32, 0x54, 0x76] * 2, [0x98, 0xBA, 0xDC, 0xFE] * 2], np.uint8)
    w_scales = np.full((2, 1), 0x40, np.uint8)
    C = oracle.gemm_exact(a_codes, a_scales, 2.0, w_codes, w_scales, [0.5])
    assert C.tolist() == [[2 * 2 * 18.0, -2 * 2 * 18.0]]


def test_one_hot_activation_selects_a_weight_column():
    K, N = 64, 24
    w = random_matrix(5, N, K)
    wc, ws, gw = oracle.quantize(w)
    a = np.zeros((1, K), np.float32)
    a[0, 37] = 1.0
    ac, as_, ga = oracle.quantize(a)
    C = oracle.gemm_exact(ac, as_, ga, wc, ws, [gw])
    a_val = oracle.dequantize(ac, as_, ga)[0, 37]
    assert a_val == 1.0
    np.testing.assert_array_equal(C[0], oracle.dequantize(wc, ws, gw)[:, 37])


def test_fused_equals_concatenated_per_module_products():
    M, K = 16, 256
    sizes = [64, 64, 128, 8, 8]
    segs = list(np.cumsum([0] + sizes))
    N = segs[-1]
    a = random_matrix(70, M, K, outlier_cols=3)
    w = random_matrix(71, N, K, std=0.02)
    w[segs[3]:segs[4]] *= np.float32(2.75)
    ac, as_, ga = oracle.quantize(a)
    wc, ws, gw = oracle.quantize_segments(w, segs)
    assert len(set(gw.tolist())) == len(sizes)
    fused = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
    parts = []
    for j in range(len(sizes)):
        c, s, g = oracle.quantize(w[segs[j]:segs[j + 1]])
        assert g == gw[j]
        parts.append(oracle.gemm_exact(ac, as_, ga, c, s, [g]))
    assert np.array_equal(fused, np.concatenate(parts, axis=1))


def test_defective_fused_scale_closed_form_at_the_pages_ratios():
    with open(os.path.join(GOLDEN, "fused_scale_ratios.json")) as f:
        golden = json.load(f)
    ratios = [p["scale_ratio"] for p in golden["pairs"]]
    assert ratios == [1.82, 2.75]
    M, K, n = 8, 128, 32
    for ratio in ratios:
        a = random_matrix(80, M, K, outlier_cols=2)
        w = random_matrix(81, 2 * n, K, std=0.02)
        ac, as_, ga = oracle.quantize(a)
        # two calibrated modules whose global scales differ by the pages' ratio
        g0 = np.float32(1000.0)
        g1 = np.float32(g0 * np.float32(ratio))
        segs = [0, n, 2 * n]
        wc, ws, gw = oracle.quantize_segments(w, segs, [g0, g1])
        good = oracle.gemm_exact(ac, as_, ga, wc, ws, gw, segs)
        bad_g = oracle.fused_scale_defect(gw)
        assert bad_g.tolist() == [g1, g1]
        bad = oracle.gemm_exact(ac, as_, ga, wc, ws, bad_g, segs)
        # segment 1 carries the max scale: untouched; segment 0 shrinks by g0/g1
        assert np.array_equal(bad[:, n:], good[:, n:])
        np.testing.assert_allclose(bad[:, :n], good[:, :n] * (float(g0) / float(g1)), rtol=1e-15)
        rel = np.linalg.norm(bad[:, :n] - good[:, :n]) / np.linalg.norm(good[:, :n])
        expected = 1.0 - 1.0 / ratio
        assert abs(rel - expected) < 1e-6
    assert round(1 - 1 / 1.82, 4) == 0.4505 and round(1 - 1 / 2.75, 4) == 0.6364


def test_single_segment_defect_is_harmless():
    # with one module there is nothing to fuse: the defective path equals the correct one
    ac, as_, ga, wc, ws, gw, segs = _operands(90, 4, 16, 64)
    assert np.array_equal(oracle.fused_scale_defect(gw), gw)


def test_bad_segments_rejected():
    ac, as_, ga, wc, ws, gw, segs = _operands(91, 2, 8, 32)
    with pytest.raises(ValueError):
        oracle.gemm_exact(ac, as_, ga, wc, ws, [1.0, 1.0], [0, 4, 4, 8][:3])
    with pytest.raises(ValueError):
        oracle.gemm_exact(ac, as_, ga, wc, ws, [1.0, 1.0], [0, 5, 7])
