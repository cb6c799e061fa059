"""Pins of the oracle's two element codecs against things other than themselves.

* E4M3 (block scale) encoder and decoder: PyTorch's ``float8_e4m3fn`` cast (a library routine that
  rounds to nearest-even) on every non-negative binary32 pattern below 464 (and, cheaply, every bf16
  pattern, dense windows around every rounding midpoint and random patterns); the saturation rule
  above the largest finite value.
* E2M1 (element) encoder: the closed-form threshold rule
  ``i = [y>0.25]+[y>=0.75]+[y>1.25]+[y>=1.75]+[y>2.5]+[y>=3.5]+[y>5]``, derived by hand from the
  value set {0, 0.5, 1, 1.5, 2, 3, 4, 6} with ties to the even code, on every non-negative binary32
  pattern from +0 to +inf (and, cheaply, every bf16 pattern, dense windows around every threshold
  and random patterns); and an exact rational brute-force argmin on the tie points.

The value sets are the public OCP definitions of the format names the pages use (ai.info summary,
"Methodology in Plain English": 4-bit E2M1 values with an E4M3 scale per 16-element block).
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _f32(bits):
    return np.asarray(bits, dtype=np.uint32).view(np.float32)


def _nonneg_bf16_patterns():
    hi = np.arange(0, 0x7F80 + 1, dtype=np.uint32)  # +0 .. +inf
    return _f32(hi << 16)


def _windows(centres, half=4096):
    out = []
    for c in centres:
        b = int(np.float32(c).view(np.uint32))
        lo = max(b - half, 0)
        out.append(np.arange(lo, b + half + 1, dtype=np.uint32))
    return _f32(np.concatenate(out))


def _random_nonneg_f32(n, seed, below):
    rng = np.random.Generator(np.random.PCG64(seed))
    top = int(np.float32(below).view(np.uint32))
    return _f32(rng.integers(0, top, size=n, dtype=np.uint32))


# ------------------------------------------------------------------------------------------------
# tables
# ------------------------------------------------------------------------------------------------


def test_e2m1_value_set_is_the_ocp_set():
    assert oracle.E2M1_VALUES.tolist() == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(0x7F, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.e4m3_decode(codes), ref)
    # a few landmarks of the format
    assert oracle.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert oracle.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6
    assert oracle.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert oracle.e4m3_decode(np.array([0x40]))[0] == 2.0
    assert oracle.e4m3_decode(np.array([0x23]))[0] == 0.171875


# ------------------------------------------------------------------------------------------------
# E4M3 encoder vs torch's cast
# ------------------------------------------------------------------------------------------------

# torch rounds values in [464, 480) to the NaN code; the oracle saturates everything >= 448 (and the
# tie at 464 resolves to 448 in both), so the library comparison stops below 464.
_TORCH_LIMIT = 464.0


def _torch_e4m3(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _check_e4m3_against_torch(x):
    x = x[x < _TORCH_LIMIT]
    got = oracle.e4m3_encode(x)
    ref = _torch_e4m3(x)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r} got={got[bad[0]]:#x} ref={ref[bad[0]]:#x}"


def test_e4m3_encode_all_bf16_patterns():
    _check_e4m3_against_torch(_nonneg_bf16_patterns())


def test_e4m3_encode_windows_around_every_midpoint():
    v = oracle.E4M3_VALUES
    mids = (v[:-1] + v[1:]) / 2.0
    _check_e4m3_against_torch(_windows(np.concatenate([mids, v]), half=2048))


def test_e4m3_encode_random_patterns():
    _check_e4m3_against_torch(_random_nonneg_f32(2_000_000, 11, _TORCH_LIMIT))
    # tiny values: everything at or below 2^-10 (half the smallest subnormal, a tie to 0) is zero
    tiny = _random_nonneg_f32(200_000, 12, 2.0 ** -10)
    assert np.all(oracle.e4m3_encode(tiny) == 0)
    assert oracle.e4m3_encode(np.array([2.0 ** -10], np.float32))[0] == 0
    assert oracle.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1)).reshape(1))[0] == 1


def _e4m3_chunk(start: int) -> tuple[int, int]:
    """Mismatches of the oracle against torch's cast on patterns [start, start + 2^24), below 464."""
    torch.set_num_threads(1)
    stop = min(start + (1 << 24), _E4M3_STOP)
    x = _f32(np.arange(start, stop, dtype=np.uint32))
    bad = np.nonzero(oracle.e4m3_encode(x) != _torch_e4m3(x))[0]
    return int(bad.size), (int(start + bad[0]) if bad.size else -1)


_E4M3_STOP = int(np.float32(_TORCH_LIMIT).view(np.uint32))


def test_e4m3_encode_every_binary32_pattern_below_464():
    # exhaustive from +0 up to the library's limit: every pattern (about 1.14e9), the subnormal
    # scales and the 448 saturation included, in 2^24-pattern chunks over the host's cores
    import multiprocessing as mp
    import os

    starts = list(range(0, _E4M3_STOP, 1 << 24))
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    # fresh interpreters: torch's thread pool does not survive a fork
    with mp.get_context("spawn").Pool(workers) as pool:
        res = pool.map(_e4m3_chunk, starts)
    total = sum(n for n, _ in res)
    first = [b for n, b in res if n]
    assert total == 0, f"{total} mismatches, first pattern {first[0]:#010x}"


def test_e4m3_encode_saturates_at_448():
    big = np.array([448.0, 448.5, 463.9, 464.0, 479.0, 480.0, 1e6, 3.0e38, np.inf], np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert oracle.e4m3_encode(np.array([447.9], np.float32))[0] == 0x7E  # nearest is 448
    assert oracle.e4m3_encode(np.array([431.9], np.float32))[0] == 0x7D  # nearest is 416


# ------------------------------------------------------------------------------------------------
# E2M1 encoder vs the closed-form threshold rule
# ------------------------------------------------------------------------------------------------


def _threshold_rule(y):
    y = np.asarray(y, dtype=np.float64)
    return ((y > 0.25).astype(int) + (y >= 0.75) + (y > 1.25) + (y >= 1.75) + (y > 2.5)
            + (y >= 3.5) + (y > 5.0))


def _check_e2m1(y):
    got = oracle.e2m1_encode_magnitude(y)
    ref = _threshold_rule(y)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first y={y[bad[0]]!r} got={got[bad[0]]} ref={ref[bad[0]]}"


def test_e2m1_all_bf16_patterns():
    _check_e2m1(_nonneg_bf16_patterns())


def test_e2m1_windows_around_every_threshold():
    _check_e2m1(_windows([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6], half=8192))


def test_e2m1_random_patterns():
    _check_e2m1(_random_nonneg_f32(2_000_000, 13, 8.0))
    _check_e2m1(_random_nonneg_f32(200_000, 14, 3.0e38))


def _e2m1_chunk(start: int) -> tuple[int, int]:
    """Mismatches of the oracle against the threshold rule on patterns [start, start + 2^24)."""
    stop = min(start + (1 << 24), 0x7F800001)
    y = _f32(np.arange(start, stop, dtype=np.uint32))
    bad = np.nonzero(oracle.e2m1_encode_magnitude(y) != _threshold_rule(y))[0]
    return int(bad.size), (int(start + bad[0]) if bad.size else -1)


def test_e2m1_every_nonnegative_binary32_pattern():
    # exhaustive: +0 through +inf, every pattern (2^31 - 2^23 + 1 of them), in 2^24-pattern chunks
    # over the host's cores (about two minutes of single-core work)
    import multiprocessing as mp
    import os

    starts = list(range(0, 0x7F800001, 1 << 24))
    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with mp.get_context("fork").Pool(workers) as pool:
        res = pool.map(_e2m1_chunk, starts)
    total = sum(n for n, _ in res)
    first = [b for n, b in res if n]
    assert total == 0, f"{total} mismatches, first pattern {first[0]:#010x}"


def _brute_force_e2m1(y: Fraction) -> int:
    """Exact argmin |y - V_i| with ties to the even index, saturating at 6."""
    vals = [Fraction(v).limit_denominator() for v in [0, 0.5, 1, 1.5, 2, 3, 4, 6]]
    if y >= vals[-1]:
        return 7
    d = [abs(y - v) for v in vals]
    best = min(d)
    cands = [i for i, di in enumerate(d) if di == best]
    if len(cands) == 1:
        return cands[0]
    return [i for i in cands if i % 2 == 0][0]


def test_e2m1_brute_force_on_ties_and_neighbours():
    pts = []
    for t in [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]:
        f = np.float32(t)
        pts += [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(10))]
    pts += [0.0, 0.5, 1.0, 6.0, 6.5, 100.0]
    y = np.array(pts, dtype=np.float32)
    got = oracle.e2m1_encode_magnitude(y)
    ref = [_brute_force_e2m1(Fraction(float(v))) for v in y]
    assert got.tolist() == ref
    # the ties themselves, spelled out: 0.25->0, 0.75->2 (1.0), 1.25->2, 1.75->4 (2.0), 2.5->4,
    # 3.5->6 (4.0), 5->6
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    assert oracle.e2m1_encode_magnitude(ties).tolist() == [0, 2, 2, 4, 4, 6, 6]
