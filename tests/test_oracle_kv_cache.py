"""Pins of the FP8 E4M3 KV-cache oracle (oracle/kv_cache.py).

* Codes against torch's float8_e4m3fn cast (a library routine) wherever that cast is defined
  (|y| below the saturation threshold; torch has no saturating mode) and saturation above it.
* Brute force: every finite magnitude code decodes and re-encodes to itself, for scale 1 and
  power-of-two scales (exact products).
* Sign symmetry, signed zero, round-trip error at most half a grid step for scaled values in the
  normal range, and the calibrated scale mapping the calibration amax to exactly 448.
"""

import numpy as np
import torch

import oracle


def _torch_codes(y):
    t = torch.from_numpy(np.asarray(y, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_matches_torch_cast_below_saturation():
    rng = np.random.default_rng(61)
    x = (rng.normal(0, 1, 200000) * np.exp2(rng.integers(-14, 9, 200000))).astype(np.float32)
    for scale in (1.0, 0.0371, 3.5, 2.0 ** -5):
        y = x * (np.float32(1.0) / np.float32(scale))
        ok = np.abs(y) < 464.0  # beyond the rounding threshold of 448 torch gives NaN
        got = oracle.kv_fp8_encode(x, scale)
        assert np.array_equal(got[ok], _torch_codes(y[ok])), scale
        assert np.all((got[~ok] & 0x7F) == 0x7E)


def test_every_code_round_trips():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for scale in (1.0, 0.25, 8.0):
        v = oracle.kv_fp8_decode(codes, scale)
        again = oracle.kv_fp8_encode(v, scale)
        assert np.array_equal(again, codes)


def test_sign_zero_and_saturation():
    x = np.array([0.0, -0.0, 1e-12, -1e-12, 1e6, -1e6, 448.0, 464.0, 463.9], dtype=np.float32)
    c = oracle.kv_fp8_encode(x, 1.0)
    assert list(c) == [0x00, 0x80, 0x00, 0x80, 0x7E, 0xFE, 0x7E, 0x7E, 0x7E]
    rng = np.random.default_rng(62)
    y = rng.normal(0, 30, 10000).astype(np.float32)
    assert np.array_equal(oracle.kv_fp8_encode(-y, 0.7) ^ 0x80, oracle.kv_fp8_encode(y, 0.7))


def test_round_trip_error_half_step():
    rng = np.random.default_rng(63)
    x = rng.normal(0, 2.0, 100000).astype(np.float32)
    scale = oracle.kv_calibrated_scale(x)
    y = np.abs(x) / scale
    normal = (y >= 2.0 ** -6) & (y <= 448.0)
    xhat = oracle.kv_fp8_decode(oracle.kv_fp8_encode(x, scale), scale)
    # grid step of a normal E4M3 value v is 2^(floor(log2 v) - 3); half of it, times the scale
    step = np.exp2(np.floor(np.log2(y[normal])) - 3) * scale
    assert np.all(np.abs(xhat[normal] - x[normal]) <= 0.5 * step * (1 + 1e-6))


def test_calibrated_scale_maps_amax_to_448():
    rng = np.random.default_rng(64)
    x = rng.normal(0, 5, 5000).astype(np.float32)
    s = oracle.kv_calibrated_scale(x)
    i = np.argmax(np.abs(x))
    assert oracle.kv_fp8_encode(x[i:i + 1], s)[0] & 0x7F == 0x7E
    assert oracle.kv_calibrated_scale(np.zeros(8, np.float32)) == 1.0


def test_bf16_decode_rounds_once():
    codes = np.arange(0, 127, dtype=np.uint8)
    scale = np.float32(0.0371)
    f = oracle.kv_fp8_decode(codes, scale)
    b = oracle.kv_fp8_decode(codes, scale, "bf16")
    ref = torch.from_numpy(f).to(torch.bfloat16).float().numpy()  # one rounding from binary32
    assert np.array_equal(b, ref)
