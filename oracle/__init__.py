"""CPU oracle for the NVFP4 W4A4 linear layer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import this
package.  The product path never imports it, and it imports nothing from the product path.
"""

from .nvfp4_oracle import (  # noqa: F401
    BLOCK,
    E2M1_VALUES,
    E4M3_VALUES,
    GLOBAL_SCALE_NUMERATOR,
    decode_integers,
    decode_values,
    dequantize,
    dynamic_global_scale,
    e2m1_encode_magnitude,
    e4m3_decode,
    e4m3_encode,
    element_value_exact,
    fused_scale_defect,
    gemm_abs_bound,
    gemm_dequant_f64,
    gemm_exact,
    quantize,
    quantize_segments,
    unpack_codes,
)
from .activation import round_to_bf16, silu, silu_mul_activation, silu_mul_quantize  # noqa: F401
from .kv_cache import kv_calibrated_scale, kv_fp8_decode, kv_fp8_encode  # noqa: F401
from .fake_quant import (  # noqa: F401
    dequantize_f32,
    dominated_blocks,
    fake_quantize,
    harmonize_segments,
    quant_error_stats,
    requantize,
)
