"""Pins of the SiLU(g) * u -> NVFP4 oracle (oracle/activation.py).

* SiLU against torch's float64 SiLU (a library routine) and the exact identity
  silu(x) - silu(-x) = x; its closed values at 0 and far out.
* bfloat16 rounding against brute force over all 65536 bfloat16 bit patterns (nearest value, ties
  to the even pattern), against torch's float32 -> bfloat16 cast for inputs that are exactly
  float32 (one rounding either way), on exact midpoints (must go to the even neighbour), through
  the subnormal range and at the overflow edge.
* A worked example of the whole fused step.
"""

import numpy as np
import pytest
import torch

import oracle


def _all_bf16_values():
    bits = np.arange(65536, dtype=np.uint32) << 16
    with np.errstate(invalid="ignore"):
        v = bits.view(np.float32).astype(np.float64)
    keep = np.isfinite(v)
    return v[keep], (bits[keep] >> 16).astype(np.int64)


def _brute_round(x):
    """Nearest finite bfloat16 by exhaustive search; ties to the even bit pattern."""
    vals, pats = _all_bf16_values()
    order = np.argsort(vals, kind="stable")
    vals, pats = vals[order], pats[order]
    # -0.0 and +0.0 both appear: keep +0.0 for the search, fix the sign afterwards
    out = np.empty_like(x)
    for i, xi in enumerate(x):
        d = np.abs(vals - xi)
        best = d.min()
        cand = np.nonzero(d == best)[0]
        cvals, cpats = vals[cand], pats[cand]
        if len(set(cvals)) > 1:  # a true tie between two neighbours: even significand wins
            even = cpats[(cpats & 1) == 0]
            out[i] = vals[cand][np.isin(cpats, even)][0]
        else:
            out[i] = cvals[0]
        if out[i] == 0.0:
            out[i] = np.copysign(0.0, xi)
    return out


def test_silu_matches_library_and_identity():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 3, 20000), rng.uniform(-700, 700, 2000)])
    ours = oracle.silu(x)
    lib = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(ours, lib, rtol=1e-14, atol=1e-300)
    # silu(x) - silu(-x) = x / (1+e^-x) - (-x) / (1+e^x) = x (exact in real arithmetic)
    y = rng.normal(0, 4, 20000)
    assert np.allclose(oracle.silu(y) - oracle.silu(-y), y, rtol=1e-14, atol=1e-14)


def test_silu_closed_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(1000.0) == 1000.0
    assert oracle.silu(-1000.0) == 0.0 and np.signbit(oracle.silu(-1000.0))  # -0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16


def test_round_to_bf16_brute_force():
    rng = np.random.default_rng(6)
    x = np.concatenate([
        rng.normal(0, 1, 3000) * np.exp2(rng.integers(-140, 120, 3000)),
        rng.normal(0, 1, 500),
    ])
    assert np.array_equal(oracle.round_to_bf16(x).astype(np.float64), _brute_round(x))


def test_round_to_bf16_ties_go_to_even():
    vals, pats = _all_bf16_values()
    pos = vals > 0
    v, pt = vals[pos], pats[pos]
    order = np.argsort(v)
    v, pt = v[order], pt[order]
    mids = (v[:-1] + v[1:]) / 2  # exact in binary64: neighbours differ in few bits
    got = oracle.round_to_bf16(mids).astype(np.float64)
    want = np.where((pt[:-1] & 1) == 0, v[:-1], v[1:])
    assert np.array_equal(got, want)
    # one unit of 2^-53 either side of a midpoint decides by proximity
    lo = np.nextafter(mids, -np.inf)
    hi = np.nextafter(mids, np.inf)
    assert np.array_equal(oracle.round_to_bf16(lo).astype(np.float64), v[:-1])
    assert np.array_equal(oracle.round_to_bf16(hi).astype(np.float64), v[1:])


def test_round_to_bf16_matches_torch_for_float32_inputs():
    rng = np.random.default_rng(7)
    x32 = (rng.normal(0, 1, 100000) * np.exp2(rng.integers(-130, 100, 100000))).astype(np.float32)
    lib = torch.from_numpy(x32).to(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.round_to_bf16(x32.astype(np.float64)), lib)


def test_round_to_bf16_edges():
    tiny = 2.0 ** -133  # smallest bfloat16 subnormal
    assert oracle.round_to_bf16(np.array([tiny * 0.5]))[0] == 0.0  # tie -> even (zero)
    assert oracle.round_to_bf16(np.array([tiny * 0.5000001]))[0] == np.float32(tiny)
    assert oracle.round_to_bf16(np.array([tiny * 1.5]))[0] == np.float32(2 * tiny)  # tie -> even
    big = float(np.float32(3.3895314e38))  # largest bfloat16, 0x7F7F
    assert oracle.round_to_bf16(np.array([big]))[0] == np.float32(big)
    assert np.isinf(oracle.round_to_bf16(np.array([2.0 ** 128]))[0])
    assert np.signbit(oracle.round_to_bf16(np.array([-1e-300]))[0])


def test_worked_example():
    # g = 0 gives an exact zero activation of the sign of u (0 * u); g = 2, u = 1.5:
    # silu(2) = 2 / (1 + e^-2) = 1.7615941559557649; * 1.5 = 2.6423912339336475 -> bf16 2.640625
    # (bf16 step at 2 is 2^-6 = 0.015625: 2.6423.. lies between 2.640625 and 2.65625, nearer the first)
    g = np.array([[0.0, 0.0, 2.0] + [0.0] * 13], dtype=np.float32)
    u = np.array([[1.0, -1.0, 1.5] + [1.0] * 13], dtype=np.float32)
    a = oracle.silu_mul_activation(g, u)
    assert a[0, 0] == 0.0 and not np.signbit(a[0, 0])
    assert a[0, 1] == 0.0 and np.signbit(a[0, 1])
    assert a[0, 2] == np.float32(2.640625)
    codes, scales, ga = oracle.silu_mul_quantize(g, u, 1.0)
    # static g = 1: block amax 2.640625 -> s = 2.640625 / 6 = 0.44010416.. -> E4M3 0.4375 (0x2E);
    # r = 1 / 0.4375 = 2.2857..; y = 6.0357.. -> code 7 (6); zeros -> 0x0 and 0x8
    assert scales[0, 0] == 0x2E
    assert codes[0, 0] == 0x80 and codes[0, 1] == 0x07
    assert ga == np.float32(1.0)
