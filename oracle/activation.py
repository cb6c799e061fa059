"""CPU oracle for the fused SiLU(g) * u -> NVFP4 encoding (test infrastructure only).

This module is test infrastructure: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import it, and it imports nothing from the product path.

What is computed.  The pages quantize all 496 linear layers, 192 of them MLP projections
([ai.info, Methodology]); the input of an MLP's down projection is the gated activation of its
gate and up projections.  Reading (the pages name no activation function): the gate is SiLU,
``act = SiLU(g) * u`` with ``SiLU(x) = x / (1 + exp(-x))``, the activation the down projection
consumes is held in bfloat16 (the model's activation type), and the fused step produces exactly the
NVFP4 encoding of that bfloat16 tensor:

    a = RNE_bf16( SiLU(g) * u )              (one rounding, from the exact real value)
    codes, scales = quantize(a, g_A)          (the encoder of ``nvfp4_oracle``)

The real value is evaluated in binary64 (its error, a few units of 2^-53, decides a bfloat16
rounding only when the value lies that close to a bfloat16 midpoint) and rounded straight from
binary64 to bfloat16 -- never through binary32, which would round twice.

Parity status: ``silu`` and ``round_to_bf16`` are pinned in ``tests/test_oracle_activation.py``
(a library SiLU, an exact identity, brute force over every bfloat16 value); ``silu_mul_quantize``
is their composition with the pinned encoder.
"""

from __future__ import annotations

import numpy as np

from .nvfp4_oracle import quantize


def silu(x) -> np.ndarray:
    """SiLU in binary64: ``x / (1 + exp(-x))``."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value of each binary64 ``x`` (ties to the even significand), as float32.

    bfloat16 keeps 8 significant bits and binary32's exponent range: a value with leading bit
    2^(e-1) (``frexp`` exponent e) lies on the grid of multiples of 2^(e-8); below the normal range
    (2^-126) the grid is the multiples of 2^-133.  Dividing by the grid step (a power of two) is
    exact, ``rint`` rounds half to even, and multiplying back is exact.  Magnitudes at or beyond
    2^128 (after rounding) become infinities; NaN stays NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)
    step_exp = np.maximum(e, -125) - 8
    q = np.ldexp(np.ones_like(xf), step_exp)
    out[fin] = np.rint(xf / q) * q
    out[~fin] = x[~fin]
    with np.errstate(over="ignore"):
        return out.astype(np.float32)


def silu_mul_activation(g, u) -> np.ndarray:
    """``RNE_bf16(SiLU(g) * u)`` elementwise, evaluated in binary64, as float32 (exact)."""
    return round_to_bf16(silu(g) * np.asarray(u, dtype=np.float64))


def silu_mul_quantize(g, u, global_scale=None):
    """NVFP4 encoding of ``silu_mul_activation(g, u)``: ``(codes, scales, g_A)`` exactly as
    ``quantize`` gives for that tensor (dynamic global scale if ``global_scale`` is None)."""
    return quantize(silu_mul_activation(g, u), global_scale)
