"""CPU oracle for the NVFP4 W4A4 linear layer (test infrastructure only).

This module is test infrastructure.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and this module imports nothing from
the product path.

It is a plain, slow, obviously checkable NumPy implementation of what the hot path computes:

* NVFP4 encoding of a tensor: 4-bit E2M1 element codes, one FP8 E4M3 scale per 16 consecutive
  elements of a row, one FP32 global scale per tensor (or per calibrated module);
* the W4A4 product of two encoded operands, computed exactly in integers and rounded once;
* the fused-module form in which the output columns are split into segments, each carrying the
  global scale of the module it came from, and the defective form that applies the largest of
  those global scales to every segment.

Sources.  Pages are cited by site and section.  All five pages summarise the paper
"Why Gated DeltaNet Survives 4-Bit Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B
LLM" (arXiv 2609.04098):

* [ai.info, Methodology]  -- ai.info "AI summary" page, section "Methodology in Plain English":
  NVFP4 pairs 4-bit E2M1 values with an E4M3 scale per 16-element block, and the block's largest
  value fixes that scale.
* [ai.info, Main Findings] -- same page, section "Main Findings": one FP32 global scale per linear
  module from calibration; fused serving GEMMs (in_proj_qkv+z, in_proj_b+a) apply the maximum of
  the constituent global scales without rescaling the block scales; the paired scales differ by
  1.82x and 2.75x.
* [chatpaper.ai, abstract] -- the English abstract: 16-element block scaling localises outliers;
  the repair of the global-scale mismatch of fused GEMMs.

The pages name the formats but print no encoding procedure.  The E2M1 and E4M3 value sets below are
the public OCP definitions of those format names.  Where the pages leave a step open, the reading
taken here is stated at the step; every reading is also listed in the design notes.

Readings (the pages are silent on all of these):

R1  global scale ``g`` is an encode-direction multiplier; dequantisation divides by it.  The
    dynamic choice is ``g = 2688 / amax(tensor)`` (2688 = 6 * 448, the largest E2M1 magnitude
    times the largest E4M3 value), ``g = 1`` for an all-zero tensor.
R2  block scale ``s = amax_block * fl(g / 6)``, rounded to E4M3 to nearest, ties to the even
    code, saturating at 448; subnormal E4M3 values are kept; values below half the smallest
    subnormal round to zero.
R3  element ``y = fl(|x| * fl(g / sd))`` with ``sd`` the decoded block scale, rounded to E2M1 to
    nearest, ties to the even code, saturating at 6.  A block whose scale decodes to 0 encodes
    every element with magnitude 0.
R4  the sign bit is copied from the input, so -0.0 and negative values that round to zero give
    code 0x8.
R5  two codes per byte, the even-indexed element in the low nibble; scales row-major
    ``[rows, cols/16]`` with no swizzle; blocks run along the contraction axis K for both
    operands.
R6  every operation of the encoding is an IEEE binary32 operation in the order written here.

Parity status: every public function here is pinned by tests under ``tests/`` (see the test
module docstrings for which pin covers which function).  No function is "parity unpinned".
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

# ----------------------------------------------------------------------------------------------
# Codebooks from the format names ([ai.info, Methodology]) and the public OCP definitions.
# ----------------------------------------------------------------------------------------------


def _e2m1_value(index: int) -> float:
    """Magnitude of E2M1 code ``index`` (0..7): 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    e, m = index >> 1, index & 1
    if e == 0:
        return m * 0.5  # subnormal: m * 2^(1-1) * 2^-1
    return (1.0 + m / 2.0) * 2.0 ** (e - 1)


def _e4m3_value(code: int) -> float:
    """Value of non-negative OCP E4M3 (e4m3fn) code 0x00..0x7E: bias 7, no infinities."""
    e, m = code >> 3, code & 7
    if e == 0:
        return m * 2.0 ** -9  # subnormal: (m/8) * 2^(1-7)
    return (1.0 + m / 8.0) * 2.0 ** (e - 7)


#: E2M1 magnitudes by index, {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
E2M1_VALUES = np.array([_e2m1_value(i) for i in range(8)], dtype=np.float64)
#: E4M3 finite non-negative values by code 0x00..0x7E (0x7F is NaN and never produced).
E4M3_VALUES = np.array([_e4m3_value(c) for c in range(0x7F)], dtype=np.float64)
E4M3_MAX = 448.0
E2M1_MAX = 6.0
#: dynamic global-scale numerator (reading R1)
GLOBAL_SCALE_NUMERATOR = np.float32(E2M1_MAX * E4M3_MAX)  # 2688
BLOCK = 16


def _round_to_grid_nearest_even(y: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid point nearest to each ``y >= 0``; a tie goes to the even index; values
    at or above the last grid point take the last index (saturation).

    ``grid`` is ascending and the index equals the format's code, so an even index is an even
    mantissa LSB.  Midpoints of consecutive grid points are exact in float64 (the grids hold at
    most 4 significant bits), and ``y`` converts exactly from float32, so every comparison below
    is exact.
    """
    y = np.asarray(y, dtype=np.float64)
    last = len(grid) - 1
    j = np.searchsorted(grid, y, side="right") - 1  # grid[j] <= y < grid[j+1]
    j = np.clip(j, 0, last)
    inner = j < last
    jn = np.minimum(j + 1, last)
    mid = (grid[j] + grid[jn]) / 2.0
    up = inner & (y > mid)
    tie = inner & (y == mid)
    idx = np.where(up, jn, j)
    even = np.where(j % 2 == 0, j, jn)
    idx = np.where(tie, even, idx)
    return idx.astype(np.int64)


def e4m3_encode(s: np.ndarray) -> np.ndarray:
    """Round non-negative float32 scale values to E4M3 codes (reading R2): nearest, ties to even
    code, 448 and above saturate to 0x7E, subnormals kept."""
    s = np.asarray(s, dtype=np.float32)
    if np.any(np.isnan(s)) or np.any(s < 0):
        raise ValueError("e4m3_encode: scale must be non-negative and not NaN")
    return _round_to_grid_nearest_even(s, E4M3_VALUES).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """E4M3 codes 0x00..0x7E to their exact values (float64; every value is exact in float32)."""
    code = np.asarray(code, dtype=np.int64)
    if np.any(code > 0x7E) or np.any(code < 0):
        raise ValueError("e4m3_decode: only non-negative finite codes are produced")
    return E4M3_VALUES[code]


def e2m1_encode_magnitude(y: np.ndarray) -> np.ndarray:
    """Round non-negative float32 magnitudes to E2M1 indices 0..7 (reading R3): nearest, ties to
    even index, saturating at 6."""
    return _round_to_grid_nearest_even(np.asarray(y, dtype=np.float32), E2M1_VALUES)


# ----------------------------------------------------------------------------------------------
# Encoding of a tensor ([ai.info, Methodology]; readings R1-R6).
# ----------------------------------------------------------------------------------------------


def dynamic_global_scale(x: np.ndarray) -> np.float32:
    """Reading R1: ``g = fl(2688 / amax)`` over the whole tensor, ``g = 1`` if the tensor is all
    zeros.  The max of absolute values is exact in any order."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0:
        return np.float32(1.0)
    return np.float32(GLOBAL_SCALE_NUMERATOR / amax)


def quantize(x: np.ndarray, g: float | None = None):
    """Encode a 2-D float32 tensor ``x[R, K]`` (K a multiple of 16) as NVFP4.

    ``g`` is the FP32 global scale (static, e.g. calibrated); ``None`` selects the dynamic scale of
    reading R1.  Returns ``(codes uint8[R, K/2], scales uint8[R, K/16], g float32)``.

    Steps (readings R1-R6), each an IEEE binary32 operation:
      1. ``gs6 = fl(g / 6)`` once per tensor;
      2. per block of 16 consecutive elements of a row, ``amax_b = max |x|`` and
         ``s = fl(amax_b * gs6)``: the block's largest value fixes its scale
         ([ai.info, Methodology]);
      3. ``sb = E4M3(s)``, ``sd`` its exact value;
      4. ``r = fl(g / sd)`` per block; per element ``y = fl(|x| * r)`` and ``i = E2M1(y)``;
         a block with ``sd == 0`` gets ``i = 0`` everywhere;
      5. ``code = signbit(x) << 3 | i``; two codes per byte, even element in the low nibble.
    """
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("quantize expects float32 values (bf16/f16 inputs widen exactly)")
    if x.ndim != 2 or x.shape[1] % BLOCK != 0:
        raise ValueError("quantize expects a 2-D tensor whose row length is a multiple of 16")
    R, K = x.shape
    g = dynamic_global_scale(x) if g is None else np.float32(g)
    if not (np.isfinite(g) and g > 0):
        raise ValueError("global scale must be positive and finite")

    gs6 = np.float32(g / np.float32(6.0))
    xb = x.reshape(R, K // BLOCK, BLOCK)
    ax = np.abs(xb)
    amax_b = ax.max(axis=2) if K else np.zeros((R, 0), np.float32)
    with np.errstate(over="ignore"):
        s = (amax_b * gs6).astype(np.float32)
    sb = e4m3_encode(s)
    sd = e4m3_decode(sb).astype(np.float32)
    nz = sd > 0
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        r = np.where(nz, g / np.where(nz, sd, np.float32(1.0)), np.float32(0.0)).astype(np.float32)
        y = (ax * r[:, :, None]).astype(np.float32)
    idx = e2m1_encode_magnitude(y)
    idx = np.where(nz[:, :, None], idx, 0)
    sign = np.signbit(xb).astype(np.int64)
    code = (sign << 3) | idx
    code = code.reshape(R, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, sb.reshape(R, K // BLOCK).astype(np.uint8), np.float32(g)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    """Packed bytes ``[R, K/2]`` to 4-bit codes ``[R, K]`` (even element from the low nibble)."""
    codes = np.asarray(codes, dtype=np.uint8)
    R, H = codes.shape
    out = np.empty((R, 2 * H), dtype=np.int64)
    out[:, 0::2] = codes & 0xF
    out[:, 1::2] = codes >> 4
    return out


def decode_values(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decoded element values ``V(code) * sd`` (without the global scale), float64 and exact."""
    c = unpack_codes(codes)
    mag = E2M1_VALUES[c & 7]
    sgn = np.where(c & 8, -1.0, 1.0)
    sd = e4m3_decode(np.repeat(np.asarray(scales, dtype=np.int64), BLOCK, axis=1))
    return sgn * mag * sd


def dequantize(codes: np.ndarray, scales: np.ndarray, g: float) -> np.ndarray:
    """Dequantised tensor ``V(code) * sd / g`` in float64 (reading R1: decode divides by g)."""
    return decode_values(codes, scales) / np.float64(np.float32(g))


def decode_integers(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decoded elements as exact integers ``2*V * 512*sd`` = ``V * sd * 2^10`` (int64).

    ``2*V`` is in {0, 1, 2, 3, 4, 6, 8, 12} and ``512*sd`` is an integer up to 229376, so each is
    below 2^22 and a product of two is below 2^44."""
    c = unpack_codes(codes)
    c2 = np.rint(2.0 * E2M1_VALUES[c & 7]).astype(np.int64)
    c2 = np.where(c & 8, -c2, c2)
    si = np.rint(e4m3_decode(np.asarray(scales, dtype=np.int64)) * 512.0).astype(np.int64)
    return c2 * np.repeat(si, BLOCK, axis=1)


# ----------------------------------------------------------------------------------------------
# W4A4 product ([ai.info, Main Findings]: one global scale per module; fused GEMMs).
# ----------------------------------------------------------------------------------------------


def _check_segments(seg_offsets, N: int):
    off = [int(o) for o in seg_offsets]
    if len(off) < 2 or off[0] != 0 or off[-1] != N or any(b <= a for a, b in zip(off, off[1:])):
        raise ValueError("segment offsets must rise strictly from 0 to N")
    return off


def gemm_exact(a_codes, a_scales, a_g, w_codes, w_scales, seg_g, seg_offsets=None):
    """``C[m, n] = sum_k a[m,k] * w[n,k] / (gA * gW[seg(n)])`` for NVFP4 operands.

    ``a`` is ``[M, K]``, ``w`` is ``[N, K]`` (the linear layer's weight layout); both are encoded
    along K.  ``seg_g`` holds one global scale per segment, ``seg_offsets`` the column boundaries
    ``0 = o_0 < ... < o_S = N`` (default: one segment).  The sum is formed exactly in int64 from
    the integer decodings (|sum| < 2^44 * K < 2^63 for K < 2^19) and converted to float64 once;
    the division by the product of the two global scales happens in float64 (the product of two
    float32 values is exact in float64).
    """
    A = decode_integers(a_codes, a_scales)
    W = decode_integers(w_codes, w_scales)
    M, K = A.shape
    N, K2 = W.shape
    if K != K2:
        raise ValueError("A and W disagree on K")
    if K >= 1 << 19:
        raise ValueError("K too large for the exact int64 sum")
    seg_g = np.asarray(seg_g, dtype=np.float32).reshape(-1)
    off = _check_segments([0, N] if seg_offsets is None else seg_offsets, N)
    if len(seg_g) != len(off) - 1:
        raise ValueError("one global scale per segment")
    S = A @ W.T  # int64, exact
    C = np.empty((M, N), dtype=np.float64)
    ga = np.float64(np.asarray(a_g, dtype=np.float32).item())
    for j in range(len(seg_g)):
        lo, hi = off[j], off[j + 1]
        denom = ga * np.float64(seg_g[j])
        C[:, lo:hi] = S[:, lo:hi].astype(np.float64) * 2.0 ** -20 / denom
    return C


def gemm_abs_bound(a_codes, a_scales, a_g, w_codes, w_scales, seg_g, seg_offsets=None):
    """``sum_k |a[m,k] * w[n,k]| / (gA * gW[seg(n)])``: the scale of the per-element tolerance."""
    A = np.abs(decode_integers(a_codes, a_scales))
    W = np.abs(decode_integers(w_codes, w_scales))
    N = W.shape[0]
    seg_g = np.asarray(seg_g, dtype=np.float32).reshape(-1)
    off = _check_segments([0, N] if seg_offsets is None else seg_offsets, N)
    S = A @ W.T
    B = np.empty(S.shape, dtype=np.float64)
    ga = np.float64(np.asarray(a_g, dtype=np.float32).item())
    for j in range(len(seg_g)):
        lo, hi = off[j], off[j + 1]
        B[:, lo:hi] = S[:, lo:hi].astype(np.float64) * 2.0 ** -20 / (ga * np.float64(seg_g[j]))
    return B


def gemm_dequant_f64(a_codes, a_scales, a_g, w_codes, w_scales, seg_g, seg_offsets=None):
    """Second, independent route: dequantise both operands in float64 and call ``np.matmul``."""
    Af = dequantize(a_codes, a_scales, a_g)
    N = np.asarray(w_codes).shape[0]
    seg_g = np.asarray(seg_g, dtype=np.float32).reshape(-1)
    off = _check_segments([0, N] if seg_offsets is None else seg_offsets, N)
    Wf = decode_values(w_codes, w_scales)
    for j in range(len(seg_g)):
        Wf[off[j]:off[j + 1]] /= np.float64(seg_g[j])
    return np.matmul(Af, Wf.T)


def fused_scale_defect(seg_g) -> np.ndarray:
    """The defective fused serving path of [ai.info, Main Findings]: every segment takes the
    largest of the constituent modules' global scales, block scales untouched."""
    seg_g = np.asarray(seg_g, dtype=np.float32).reshape(-1)
    return np.full_like(seg_g, seg_g.max())


def quantize_segments(w: np.ndarray, seg_offsets, seg_g=None):
    """Offline weight encoding of a fused module: each row range ``[o_j, o_{j+1})`` is one
    calibrated module with its own global scale (dynamic per segment if ``seg_g`` is None).
    Returns ``(codes, scales, gW[S])`` with the segments concatenated along N."""
    N = w.shape[0]
    off = _check_segments(seg_offsets, N)
    cs, ss, gs = [], [], []
    for j in range(len(off) - 1):
        c, s, g = quantize(w[off[j]:off[j + 1]], None if seg_g is None else seg_g[j])
        cs.append(c)
        ss.append(s)
        gs.append(g)
    return np.concatenate(cs), np.concatenate(ss), np.array(gs, dtype=np.float32)


# ----------------------------------------------------------------------------------------------
# Exact scalar forms, for brute force on tiny inputs.
# ----------------------------------------------------------------------------------------------


def element_value_exact(codes, scales, row: int, k: int) -> Fraction:
    """The decoded value ``V * sd`` of one element as an exact rational, read straight from the
    packed bytes (low nibble = even element) and the row-major block scales."""
    byte = int(codes[row][k // 2])
    nib = byte & 0xF if k % 2 == 0 else byte >> 4
    mag = Fraction(_e2m1_value(nib & 7))
    sd = Fraction(_e4m3_value(int(scales[row][k // BLOCK])))
    v = mag * sd
    return -v if nib & 8 else v
