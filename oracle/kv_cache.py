"""CPU oracle for the FP8 E4M3 KV-cache quantizer with static per-tensor scales (test
infrastructure only).

This module is test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import it, and it imports nothing from the product path.

Source: ai.info summary, "Main Findings" (calibrated FP8 KV-cache scales: one static per-tensor
scale for each K and V tensor of the attention layers; an FP8 KV cache without them is the
uncalibrated baseline), "Key Contributions" (the KV-cache recipe: calibrated per-layer scales) and
"Real-world applications" (FP8 KV cache sizing).  The pages name the
format (FP8) and the granularity (per tensor, static); the rules below are readings:

K1  the scale is decode-direction: a stored code c represents ``E4M3(c) * scale``; the
    uncalibrated cache is ``scale = 1``.  A calibrated scale is ``amax / 448`` of calibration data.
K2  encode: ``y = fl32(x * fl32(1 / scale))`` (one reciprocal per tensor), then E4M3 nearest with
    ties to the even code, saturating at 448 (code 0x7E), subnormals kept; the sign bit is copied
    (bit 7), so -0.0 and negatives that round to zero give 0x80.
K3  decode: ``fl32(E4M3(c) * scale)``, optionally rounded to bfloat16 (nearest-even).

Parity status: pinned in ``tests/test_oracle_kv_cache.py`` (torch's float8_e4m3fn cast, brute
force through the 127 finite magnitudes, saturation, sign symmetry, round-trip error bound).
"""

from __future__ import annotations

import numpy as np

from .nvfp4_oracle import e4m3_decode, e4m3_encode


def kv_fp8_encode(x, scale) -> np.ndarray:
    """E4M3 codes (uint8) of ``x`` (float32 values) under the decode-direction ``scale``."""
    x = np.asarray(x, dtype=np.float32)
    inv = np.float32(1.0) / np.float32(scale)
    with np.errstate(over="ignore"):
        y = x * inv  # binary32 product, one rounding (an overflow to inf saturates below)
    mag = e4m3_encode(np.abs(y)).astype(np.uint8)
    sign = (np.signbit(y).astype(np.uint8) << 7).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def kv_fp8_decode(codes, scale, out_dtype: str = "f32") -> np.ndarray:
    """``fl32(E4M3(c) * scale)`` as float32 (``out_dtype='bf16'``: rounded to bfloat16, nearest
    even, returned as the float32 holding it)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = e4m3_decode(c & 0x7F).astype(np.float32)
    v = np.where((c & 0x80) != 0, -mag, mag).astype(np.float32) * np.float32(scale)
    if out_dtype == "bf16":
        from .activation import round_to_bf16

        return round_to_bf16(v.astype(np.float64))
    return v.astype(np.float32)


def kv_calibrated_scale(x) -> np.float32:
    """Static per-tensor scale from calibration data: ``amax / 448`` (1 for an all-zero tensor)."""
    amax = np.float32(np.max(np.abs(np.asarray(x, dtype=np.float32)))) if np.size(x) else 0
    return np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(448.0)
