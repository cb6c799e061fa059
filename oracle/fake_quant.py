"""CPU oracle for NVFP4 fake quantization, its error statistics, and the checkpoint-side
harmonization of fused global scales (test infrastructure only).

This module is test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import it, and it imports nothing from the product path.

Sources (ai.info summary of arXiv 2609.04098):

* "Methodology in Plain English": the authors inject exactly the 4-bit rounding error by fake
  quantization -- quantize, dequantize, continue in high precision -- and repaired the serving
  pipeline by harmonizing the fused modules' global scales on the checkpoint side.
* "Main Findings": the statistics they report at NVFP4 granularity -- per-token activation (A4)
  error 7.5-9.2 %, weight error 10.5-11.9 %, 10-32 % of 16-element blocks dominated by a single
  value.

Readings (the pages give no formulas):

F1  dequantized value ``xh = fl32(V * sd / g)``: the exact product ``V * sd`` (it has at most six
    significant bits) divided once by the FP32 global scale in binary32, correctly rounded; the
    sign bit is copied (code 0x8 gives -0.0).  Fake quantization of ``x`` is this value of
    ``quantize(x, g)``; the codes are never stored.
F2  per-row statistics: ``err2 = sum_k (xh - x)^2`` and ``norm2 = sum_k x^2``, in binary64 (each
    difference is exact in binary64); the per-token relative error is ``sqrt(err2 / norm2)`` and a
    tensor's error ``sqrt(sum err2 / sum norm2)``.
F3  a block is dominated by a single value when its largest magnitude holds more than half of the
    block's energy: ``2 * amax^2 > sum of the 16 squares``, both sides in binary64, the sum taken in
    element order (the decision is then identical wherever it is taken in this order).  An
    all-zero block is not dominated.
F4  harmonization (repair on the checkpoint side): every module j of a fused weight, stored as
    codes, scales and its own global scale g_j, is re-encoded under one shared scale
    ``g* = min_j g_j``: ``requantize = quantize(dequantize(codes_j, scales_j, g_j), g*)``.  The
    smallest encode-direction scale belongs to the module with the largest calibrated range, so no
    block scale of any module can saturate; the fused product may then use g* for every segment.

Parity status: pinned in ``tests/test_oracle_fake_quant.py`` (exact rational rounding of the
dequantized values, a hand-worked example, idempotence, closed-form statistics on constructed rows,
power-of-two harmonization being lossless, the harmonized fused product against per-segment
products).
"""

from __future__ import annotations

import numpy as np

from .nvfp4_oracle import BLOCK, decode_values, quantize


def dequantize_f32(codes, scales, g) -> np.ndarray:
    """Reading F1: ``fl32(V * sd / g)`` as float32 ``[R, K]``."""
    q = decode_values(codes, scales).astype(np.float32)  # exact: at most 6 significant bits
    with np.errstate(divide="ignore", over="ignore"):
        return (q / np.float32(g)).astype(np.float32)  # one binary32 division per element


def fake_quantize(x, g=None):
    """``(xh, g)``: the dequantized NVFP4 encoding of ``x`` (dynamic g when ``g`` is None)."""
    codes, scales, gg = quantize(np.asarray(x, dtype=np.float32), g)
    return dequantize_f32(codes, scales, gg), gg


def dominated_blocks(x) -> np.ndarray:
    """Reading F3: number of dominated 16-element blocks per row (int64)."""
    x = np.asarray(x, dtype=np.float32)
    R, K = x.shape
    xb = x.reshape(R, K // BLOCK, BLOCK).astype(np.float64)
    total = np.zeros(xb.shape[:2], dtype=np.float64)
    for i in range(BLOCK):  # element order, one binary64 rounding per addition
        total = total + xb[:, :, i] * xb[:, :, i]
    amax = np.abs(xb).max(axis=2)
    dom = (2.0 * amax * amax > total) & (amax > 0)
    return dom.sum(axis=1).astype(np.int64)


def quant_error_stats(x, g=None):
    """Reading F2/F3 per row: ``(err2 f64[R], norm2 f64[R], dominated int64[R], g)``."""
    x = np.asarray(x, dtype=np.float32)
    xh, gg = fake_quantize(x, g)
    d = xh.astype(np.float64) - x.astype(np.float64)
    err2 = (d * d).sum(axis=1)
    x64 = x.astype(np.float64)
    norm2 = (x64 * x64).sum(axis=1)
    return err2, norm2, dominated_blocks(x), gg


def requantize(codes, scales, g_in, g_out):
    """Re-encode an NVFP4 tensor from global scale ``g_in`` to ``g_out`` (reading F4)."""
    return quantize(dequantize_f32(codes, scales, g_in), g_out)[:2]


def harmonize_segments(codes, scales, seg_g, seg_offsets):
    """Reading F4 for a fused weight ``[N, K]`` whose rows ``[o_j, o_j+1)`` form module j with
    global scale ``seg_g[j]``: ``(codes', scales', g*)`` with every module re-encoded under
    ``g* = min_j seg_g[j]``."""
    seg_g = np.asarray(seg_g, dtype=np.float32)
    gs = np.float32(seg_g.min())
    c_out = np.array(codes, dtype=np.uint8, copy=True)
    s_out = np.array(scales, dtype=np.uint8, copy=True)
    off = [int(o) for o in seg_offsets]
    for j in range(len(off) - 1):
        r0, r1 = off[j], off[j + 1]
        c, s = requantize(codes[r0:r1], scales[r0:r1], seg_g[j], gs)
        c_out[r0:r1], s_out[r0:r1] = c, s
    return c_out, s_out, gs
