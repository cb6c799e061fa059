"""Python binding of libnvfp4 (NVFP4 W4A4 linear layer on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of libnvfp4.so,
reached through the C ABI declared in ``include/nvfp4.h``.  PyTorch provides device memory and the
current HIP stream.  If the library has not been built, importing works but every call raises; the
library is never replaced by a CPU or PyTorch fallback.

Entry points (same names as the C ABI):

* ``nvfp4_quantize(x, global_scale=None)`` -> ``(codes, scales, global_scale)``
* ``nvfp4_silu_mul_quantize(gate, up, global_scale=None)`` -> ``(codes, scales, global_scale)``
* ``nvfp4_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_dtype)`` -> ``C``
* ``fused_nvfp4_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale, seg_offsets,
  out_dtype)`` -> ``C``
* ``nvfp4_linear(x, a_gscale, w_codes, w_scales, seg_gscale, seg_offsets, out_dtype)`` ->
  ``(C, a_codes, a_scales)``
* ``nvfp4_fake_quantize(x, global_scale=None, out_dtype=None)`` -> ``(xh, global_scale)``
* ``nvfp4_quant_error_stats(x, global_scale=None)`` -> ``(err2, norm2, dominated, global_scale)``
* ``nvfp4_requantize(codes, scales, g_in, g_out)`` -> ``(codes, scales)``
* ``nvfp4_harmonize_segments(codes, scales, seg_gscale, seg_offsets)`` -> ``(codes, scales, g)``
* ``nvfp4_kv_fp8_store(key, value, key_scale, value_scale, key_cache, value_cache, slot_mapping)``
* ``nvfp4_kv_fp8_load(cache, scale, slot_mapping, out_dtype)`` -> decoded rows
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libnvfp4.so")

NVFP4_OK, NVFP4_EINVAL, NVFP4_ESHAPE, NVFP4_EALIGN, NVFP4_EDEVICE = range(5)
NVFP4_F32, NVFP4_BF16, NVFP4_F16 = 0, 1, 2
NVFP4_MAX_SEGMENTS = 16

#: every symbol include/nvfp4.h declares
EXPORTED_SYMBOLS = ("nvfp4_quantize", "nvfp4_silu_mul_quantize", "nvfp4_gemm", "fused_nvfp4_gemm",
                    "nvfp4_linear", "nvfp4_fake_quantize", "nvfp4_quant_error_stats", "nvfp4_requantize",
                    "nvfp4_harmonize_segments", "nvfp4_kv_fp8_store", "nvfp4_kv_fp8_load",
                    "nvfp4_status_string", "nvfp4_version")

_lib = None


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libnvfp4.so (once) and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"libnvfp4.so not found at {p}: build it with `python -m bit_block_scaled_nvfp4_amd.build`"
            " (there is no fallback implementation)")
    lib = ctypes.CDLL(p)
    c_i64, c_int, c_vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.nvfp4_quantize.argtypes = [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_int, c_vp, c_vp, c_vp]
    lib.nvfp4_quantize.restype = c_int
    lib.nvfp4_silu_mul_quantize.argtypes = [c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_i64, c_vp,
                                            c_int, c_vp, c_vp, c_vp]
    lib.nvfp4_silu_mul_quantize.restype = c_int
    lib.nvfp4_fake_quantize.argtypes = [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_int, c_vp, c_int,
                                        c_i64, c_vp]
    lib.nvfp4_fake_quantize.restype = c_int
    lib.nvfp4_quant_error_stats.argtypes = [c_vp, c_int, c_i64, c_i64, c_i64, c_vp, c_int, c_vp,
                                            c_vp, c_vp, c_vp]
    lib.nvfp4_quant_error_stats.restype = c_int
    lib.nvfp4_requantize.argtypes = [c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]
    lib.nvfp4_requantize.restype = c_int
    lib.nvfp4_harmonize_segments.argtypes = [c_vp, c_vp, c_vp, ctypes.POINTER(c_i64), c_int, c_i64,
                                             c_i64, c_vp, c_vp, c_vp, c_vp]
    lib.nvfp4_harmonize_segments.restype = c_int
    lib.nvfp4_kv_fp8_store.argtypes = [c_vp, c_vp, c_int, c_i64, c_i64, c_i64, c_i64, c_vp, c_vp,
                                       c_vp, c_vp, c_vp, c_i64, c_i64, c_vp]
    lib.nvfp4_kv_fp8_store.restype = c_int
    lib.nvfp4_kv_fp8_load.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_vp, c_int,
                                      c_i64, c_vp]
    lib.nvfp4_kv_fp8_load.restype = c_int
    lib.nvfp4_gemm.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_int,
                               c_i64, c_vp]
    lib.nvfp4_gemm.restype = c_int
    lib.fused_nvfp4_gemm.argtypes = [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.POINTER(c_i64),
                                     c_int, c_i64, c_i64, c_i64, c_vp, c_int, c_i64, c_vp]
    lib.fused_nvfp4_gemm.restype = c_int
    lib.nvfp4_linear.argtypes = [c_vp, c_int, c_i64, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                 ctypes.POINTER(c_i64), c_int, c_i64, c_i64, c_i64, c_vp, c_int,
                                 c_i64, c_vp]
    lib.nvfp4_linear.restype = c_int
    lib.nvfp4_status_string.argtypes = [c_int]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_version.argtypes = []
    lib.nvfp4_version.restype = c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().nvfp4_status_string(status).decode()


def _check(status: int):
    if status != NVFP4_OK:
        msg = status_string(status)
        if status == NVFP4_EDEVICE:
            raise Nvfp4Error(status, msg)
        raise Nvfp4Error(status, msg)


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t == torch.float32:
        return NVFP4_F32
    if t == torch.bfloat16:
        return NVFP4_BF16
    if t == torch.float16:
        return NVFP4_F16
    raise ValueError(f"unsupported dtype {t}")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _require_cuda(*ts):
    devs = set()
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            devs.add(t.device)
    if len(devs) > 1:
        raise ValueError("tensors must live on one GPU")


# Shape, dtype and layout checks, made before any tensor reaches the library: the C ABI takes bare
# pointers, so a wrongly sized or strided tensor would otherwise be read or written out of bounds.

def _packed(t, rows: int, width: int, name: str):
    """``t`` must be uint8 ``[rows, width]`` with rows packed back to back (row pitch = width)."""
    torch = _torch()
    if t.dtype != torch.uint8:
        raise ValueError(f"{name} must be uint8, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != (rows, width):
        raise ValueError(f"{name} must have shape [{rows}, {width}], got {list(t.shape)}")
    if rows > 0 and width > 0 and (t.stride(1) != 1 or (rows > 1 and t.stride(0) != width)):
        raise ValueError(f"{name} must be row-contiguous with row pitch {width}, "
                         f"got strides {t.stride()}")


def _scales_f32(t, n: int, name: str):
    """``t`` must hold at least ``n`` contiguous float32 values."""
    torch = _torch()
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if t.numel() < n or (n > 1 and (t.dim() != 1 or t.stride(0) != 1)):
        raise ValueError(f"{name} must hold {n} contiguous float32 value(s)")


def _matrix_out(t, rows: int, cols: int, name: str, dtypes):
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype in {dtypes}, got {t.dtype}")
    if t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError(f"{name} must have shape [{rows}, {cols}], got {list(t.shape)}")
    if rows > 0 and cols > 0 and t.stride(1) != 1:
        raise ValueError(f"{name} must have contiguous rows (stride(1) == 1)")


def _input_matrix(x, name: str):
    torch = _torch()
    if x.dim() != 2 or (x.numel() > 0 and x.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with contiguous rows")
    if x.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        raise ValueError(f"{name} must be float32, bfloat16 or float16, got {x.dtype}")
    if x.shape[1] % 16 != 0:
        raise ValueError(f"{name} must have a multiple of 16 columns, got {x.shape[1]}")


def _gemm_operands(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale, nseg):
    """Check the encoded operands of a product; returns (M, N, K)."""
    if a_codes.dim() != 2 or w_codes.dim() != 2:
        raise ValueError("a_codes and w_codes must be 2-D")
    M, K = a_codes.shape[0], a_codes.shape[1] * 2
    N = w_codes.shape[0]
    if w_codes.shape[1] * 2 != K:
        raise ValueError("A and W disagree on K")
    if K % 16 != 0:
        raise ValueError(f"K = {K} is not a multiple of 16")
    _packed(a_codes, M, K // 2, "a_codes")
    _packed(a_scales, M, K // 16, "a_scales")
    _packed(w_codes, N, K // 2, "w_codes")
    _packed(w_scales, N, K // 16, "w_scales")
    _scales_f32(a_gscale, 1, "a_gscale")
    _scales_f32(seg_gscale, nseg, "segment global scales")
    return M, N, K


def nvfp4_quantize(x, global_scale=None, codes=None, scales=None):
    """Encode ``x[rows, cols]`` (f32/bf16/f16, row-contiguous) as NVFP4 on the GPU.

    ``global_scale``: a 1-element float32 device tensor holding a static scale, or None for the
    dynamic scale, which is then returned in a new 1-element tensor.  Returns
    ``(codes uint8[rows, cols/2], scales uint8[rows, cols/16], global_scale)``."""
    torch = _torch()
    lib = load_library()
    _input_matrix(x, "x")
    rows, cols = x.shape
    if global_scale is not None:
        _scales_f32(global_scale, 1, "global_scale")
    if codes is not None:
        _packed(codes, rows, cols // 2, "codes")
    if scales is not None:
        _packed(scales, rows, cols // 16, "scales")
    _require_cuda(x, global_scale, codes, scales)
    dynamic = global_scale is None
    if dynamic:
        global_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    _check(lib.nvfp4_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0),
                              _ptr(global_scale), int(dynamic), _ptr(codes), _ptr(scales),
                              _stream(x.device)))
    return codes, scales, global_scale


def nvfp4_silu_mul_quantize(gate, up, global_scale=None, codes=None, scales=None):
    """Encode ``bf16(SiLU(gate) * up)`` as NVFP4 on the GPU in one pass (the activation itself is
    never written).  ``gate`` and ``up``: 2-D, same shape and dtype (f32/bf16/f16), contiguous
    rows.  ``global_scale`` as for :func:`nvfp4_quantize`.  Returns ``(codes, scales,
    global_scale)``."""
    torch = _torch()
    lib = load_library()
    _input_matrix(gate, "gate")
    _input_matrix(up, "up")
    if gate.shape != up.shape or gate.dtype != up.dtype:
        raise ValueError("gate and up must have the same shape and dtype")
    rows, cols = gate.shape
    if global_scale is not None:
        _scales_f32(global_scale, 1, "global_scale")
    if codes is not None:
        _packed(codes, rows, cols // 2, "codes")
    if scales is not None:
        _packed(scales, rows, cols // 16, "scales")
    _require_cuda(gate, up, global_scale, codes, scales)
    dynamic = global_scale is None
    if dynamic:
        global_scale = torch.empty(1, dtype=torch.float32, device=gate.device)
    if codes is None:
        codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=gate.device)
    if scales is None:
        scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=gate.device)
    _check(lib.nvfp4_silu_mul_quantize(_ptr(gate), _ptr(up), _dtype_code(gate.dtype), rows, cols,
                                       gate.stride(0), up.stride(0), _ptr(global_scale),
                                       int(dynamic), _ptr(codes), _ptr(scales),
                                       _stream(gate.device)))
    return codes, scales, global_scale


def _out(M, N, out_dtype, device):
    torch = _torch()
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    return torch.empty((M, N), dtype=out_dtype, device=device)


def nvfp4_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out_dtype=None, out=None):
    """``C = A @ W^T / (gA * gW)`` for NVFP4 ``A[M, K]`` and ``W[N, K]``."""
    torch = _torch()
    lib = load_library()
    M, N, K = _gemm_operands(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, 1)
    if out is not None:
        _matrix_out(out, M, N, "out", (torch.float32, torch.bfloat16))
    _require_cuda(a_codes, a_scales, a_gscale, w_codes, w_scales, w_gscale, out)
    if out is None:
        out = _out(M, N, out_dtype or torch.float32, a_codes.device)
    _check(lib.nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_gscale), _ptr(w_codes),
                          _ptr(w_scales), _ptr(w_gscale), M, N, K, _ptr(out),
                          _dtype_code(out.dtype), out.stride(0), _stream(a_codes.device)))
    return out


def fused_nvfp4_gemm(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale, seg_offsets,
                     out_dtype=None, out=None):
    """Product with a fused weight of ``len(seg_offsets) - 1`` calibrated modules; columns
    ``[seg_offsets[j], seg_offsets[j+1])`` are divided by ``gA * seg_gscale[j]``."""
    torch = _torch()
    lib = load_library()
    offs = [int(o) for o in seg_offsets]
    nseg = len(offs) - 1
    if not 1 <= nseg <= NVFP4_MAX_SEGMENTS:
        raise ValueError(f"between 1 and {NVFP4_MAX_SEGMENTS} segments, got {nseg}")
    M, N, K = _gemm_operands(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale, nseg)
    if out is not None:
        _matrix_out(out, M, N, "out", (torch.float32, torch.bfloat16))
    _require_cuda(a_codes, a_scales, a_gscale, w_codes, w_scales, seg_gscale, out)
    arr = (ctypes.c_int64 * len(offs))(*offs)
    if out is None:
        out = _out(M, N, out_dtype or torch.float32, a_codes.device)
    _check(lib.fused_nvfp4_gemm(_ptr(a_codes), _ptr(a_scales), _ptr(a_gscale), _ptr(w_codes),
                                _ptr(w_scales), _ptr(seg_gscale), arr, nseg, M, N, K, _ptr(out),
                                _dtype_code(out.dtype), out.stride(0), _stream(a_codes.device)))
    return out


def nvfp4_linear(x, a_gscale, w_codes, w_scales, seg_gscale, seg_offsets=None, out_dtype=None,
                 out=None, a_codes=None, a_scales=None):
    """The linear layer on a raw activation ``x[M, K]`` (f32/bf16/f16, contiguous rows): encode it
    with the static scale ``a_gscale`` (bit-identical to :func:`nvfp4_quantize`) and form the fused
    product with the weight's modules (``seg_offsets``; None: one module), in one launch for decode
    shapes.  Returns ``(C, a_codes, a_scales)``."""
    torch = _torch()
    lib = load_library()
    _input_matrix(x, "x")
    M, K = x.shape
    if w_codes.dim() != 2:
        raise ValueError("w_codes must be 2-D")
    N = w_codes.shape[0]
    offs = [0, N] if seg_offsets is None else [int(o) for o in seg_offsets]
    nseg = len(offs) - 1
    if not 1 <= nseg <= NVFP4_MAX_SEGMENTS:
        raise ValueError(f"between 1 and {NVFP4_MAX_SEGMENTS} segments, got {nseg}")
    if w_codes.shape[1] * 2 != K:
        raise ValueError("x and W disagree on K")
    _packed(w_codes, N, K // 2, "w_codes")
    _packed(w_scales, N, K // 16, "w_scales")
    _scales_f32(a_gscale, 1, "a_gscale")
    _scales_f32(seg_gscale, nseg, "segment global scales")
    if a_codes is not None:
        _packed(a_codes, M, K // 2, "a_codes")
    if a_scales is not None:
        _packed(a_scales, M, K // 16, "a_scales")
    if out is not None:
        _matrix_out(out, M, N, "out", (torch.float32, torch.bfloat16))
    _require_cuda(x, a_gscale, w_codes, w_scales, seg_gscale, out, a_codes, a_scales)
    if a_codes is None:
        a_codes = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if a_scales is None:
        a_scales = torch.empty((M, K // 16), dtype=torch.uint8, device=x.device)
    if out is None:
        out = _out(M, N, out_dtype or torch.float32, x.device)
    arr = (ctypes.c_int64 * len(offs))(*offs)
    _check(lib.nvfp4_linear(_ptr(x), _dtype_code(x.dtype), x.stride(0), _ptr(a_gscale),
                            _ptr(a_codes), _ptr(a_scales), _ptr(w_codes), _ptr(w_scales),
                            _ptr(seg_gscale), arr, nseg, M, N, K, _ptr(out), _dtype_code(out.dtype),
                            out.stride(0), _stream(x.device)))
    return out, a_codes, a_scales


def nvfp4_fake_quantize(x, global_scale=None, out_dtype=None, out=None):
    """``dequantize(quantize(x))`` on the GPU: ``x[rows, cols]`` (f32/bf16/f16, contiguous rows)
    with its NVFP4 rounding error, as float32 (default) or bfloat16.  ``global_scale`` as for
    :func:`nvfp4_quantize`.  Returns ``(xh, global_scale)``."""
    torch = _torch()
    lib = load_library()
    _input_matrix(x, "x")
    rows, cols = x.shape
    if global_scale is not None:
        _scales_f32(global_scale, 1, "global_scale")
    if out is not None:
        _matrix_out(out, rows, cols, "out", (torch.float32, torch.bfloat16))
    _require_cuda(x, global_scale, out)
    dynamic = global_scale is None
    if dynamic:
        global_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    if out is None:
        out = _out(rows, cols, out_dtype or torch.float32, x.device)
    _check(lib.nvfp4_fake_quantize(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                   _ptr(global_scale), int(dynamic), _ptr(out),
                                   _dtype_code(out.dtype), out.stride(0), _stream(x.device)))
    return out, global_scale


def nvfp4_quant_error_stats(x, global_scale=None):
    """Per-row NVFP4 quantization-error statistics of ``x``: ``(err2 f64[rows], norm2 f64[rows],
    dominated int32[rows], global_scale)``."""
    torch = _torch()
    lib = load_library()
    _input_matrix(x, "x")
    rows, cols = x.shape
    if global_scale is not None:
        _scales_f32(global_scale, 1, "global_scale")
    _require_cuda(x, global_scale)
    dynamic = global_scale is None
    if dynamic:
        global_scale = torch.empty(1, dtype=torch.float32, device=x.device)
    err2 = torch.zeros(rows, dtype=torch.float64, device=x.device)
    norm2 = torch.zeros(rows, dtype=torch.float64, device=x.device)
    dom = torch.zeros(rows, dtype=torch.int32, device=x.device)
    _check(lib.nvfp4_quant_error_stats(_ptr(x), _dtype_code(x.dtype), rows, cols, x.stride(0),
                                       _ptr(global_scale), int(dynamic), _ptr(err2), _ptr(norm2),
                                       _ptr(dom), _stream(x.device)))
    return err2, norm2, dom, global_scale


def nvfp4_requantize(codes, scales, g_in, g_out, codes_out=None, scales_out=None):
    """Re-encode NVFP4 ``(codes [rows, cols/2], scales [rows, cols/16])`` from global scale
    ``g_in`` to ``g_out`` (1-element float32 device tensors).  The outputs may be the inputs."""
    lib = load_library()
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D")
    rows, cols = codes.shape[0], codes.shape[1] * 2
    if cols % 16 != 0:
        raise ValueError(f"{cols} columns is not a multiple of 16")
    _packed(codes, rows, cols // 2, "codes")
    _packed(scales, rows, cols // 16, "scales")
    _scales_f32(g_in, 1, "g_in")
    _scales_f32(g_out, 1, "g_out")
    if codes_out is not None:
        _packed(codes_out, rows, cols // 2, "codes_out")
    if scales_out is not None:
        _packed(scales_out, rows, cols // 16, "scales_out")
    _require_cuda(codes, scales, g_in, g_out, codes_out, scales_out)
    if codes_out is None:
        codes_out = codes.new_empty(codes.shape)
    if scales_out is None:
        scales_out = scales.new_empty(scales.shape)
    _check(lib.nvfp4_requantize(_ptr(codes), _ptr(scales), _ptr(g_in), _ptr(g_out), rows, cols,
                                _ptr(codes_out), _ptr(scales_out), _stream(codes.device)))
    return codes_out, scales_out


def nvfp4_harmonize_segments(codes, scales, seg_gscale, seg_offsets, codes_out=None,
                             scales_out=None, shared_gscale=None):
    """Re-encode every module of a fused NVFP4 weight under the smallest module scale.  Returns
    ``(codes, scales, shared_gscale)``; the outputs may be the inputs."""
    torch = _torch()
    lib = load_library()
    if codes.dim() != 2:
        raise ValueError("codes must be 2-D")
    N, K = codes.shape[0], codes.shape[1] * 2
    if K % 16 != 0:
        raise ValueError(f"K = {K} is not a multiple of 16")
    offs = [int(o) for o in seg_offsets]
    if not 1 <= len(offs) - 1 <= NVFP4_MAX_SEGMENTS:
        raise ValueError(f"between 1 and {NVFP4_MAX_SEGMENTS} segments, got {len(offs) - 1}")
    _packed(codes, N, K // 2, "codes")
    _packed(scales, N, K // 16, "scales")
    _scales_f32(seg_gscale, len(offs) - 1, "seg_gscale")
    if codes_out is not None:
        _packed(codes_out, N, K // 2, "codes_out")
    if scales_out is not None:
        _packed(scales_out, N, K // 16, "scales_out")
    if shared_gscale is not None:
        _scales_f32(shared_gscale, 1, "shared_gscale")
    _require_cuda(codes, scales, seg_gscale, codes_out, scales_out, shared_gscale)
    arr = (ctypes.c_int64 * len(offs))(*offs)
    if codes_out is None:
        codes_out = codes.new_empty(codes.shape)
    if scales_out is None:
        scales_out = scales.new_empty(scales.shape)
    if shared_gscale is None:
        shared_gscale = torch.empty(1, dtype=torch.float32, device=codes.device)
    _check(lib.nvfp4_harmonize_segments(_ptr(codes), _ptr(scales), _ptr(seg_gscale), arr,
                                        len(offs) - 1, N, K, _ptr(shared_gscale), _ptr(codes_out),
                                        _ptr(scales_out), _stream(codes.device)))
    return codes_out, scales_out, shared_gscale


def nvfp4_kv_fp8_store(key, value, key_scale, value_scale, key_cache, value_cache,
                       slot_mapping=None):
    """Encode ``key`` (and ``value``, or None) ``[tokens, width]`` to FP8 E4M3 under the static
    decode-direction scales (1-element float32 device tensors) and write token t's row into row
    ``slot_mapping[t]`` (int64 device tensor, or None for row t) of the uint8 caches
    ``[num_slots, width]`` (``value_cache`` None with ``value``).  Slots outside the cache are
    skipped."""
    torch = _torch()
    lib = load_library()
    _input_matrix(key, "key")
    tokens, width = key.shape
    _scales_f32(key_scale, 1, "key_scale")
    if value is not None:
        if value_scale is None or value_cache is None:
            raise ValueError("value needs value_scale and value_cache")
        _scales_f32(value_scale, 1, "value_scale")
    elif value_scale is not None or value_cache is not None:
        raise ValueError("value_scale and value_cache come with value")
    if key_cache.dtype != torch.uint8:
        raise ValueError("key_cache must be uint8")
    ts = [key, key_scale, key_cache]
    if value is not None:
        if value.shape != key.shape or value.dtype != key.dtype or value.stride(1) != 1:
            raise ValueError("value must match key's shape and dtype, with contiguous rows")
        ts += [value, value_scale, value_cache]
    if slot_mapping is not None:
        ts.append(slot_mapping)
        if slot_mapping.dtype.itemsize != 8 or slot_mapping.numel() != tokens:
            raise ValueError("slot_mapping must hold one int64 per token")
    _require_cuda(*ts)
    if key_cache.dim() != 2 or key_cache.stride(1) != 1 or key_cache.shape[1] < width:
        raise ValueError("key_cache must be 2-D [num_slots, >= width] with contiguous rows")
    if value_cache is not None and (value_cache.shape != key_cache.shape or
                                    value_cache.stride() != key_cache.stride()):
        raise ValueError("value_cache must have key_cache's shape and strides")
    _check(lib.nvfp4_kv_fp8_store(_ptr(key), _ptr(value), _dtype_code(key.dtype), tokens, width,
                                  key.stride(0), value.stride(0) if value is not None else 0,
                                  _ptr(key_scale), _ptr(value_scale), _ptr(slot_mapping),
                                  _ptr(key_cache), _ptr(value_cache), key_cache.shape[0],
                                  key_cache.stride(0), _stream(key.device)))


def nvfp4_kv_fp8_load(cache, scale, slot_mapping=None, out_dtype=None, width=None, out=None):
    """Gather rows ``slot_mapping[t]`` (int64 device tensor; None: every row in order) of the FP8
    cache ``[num_slots, >= width]`` and decode them with ``scale``; returns ``[tokens, width]``
    float32 or bfloat16.  Slots outside the cache give rows of zeros."""
    torch = _torch()
    lib = load_library()
    if cache.dim() != 2 or cache.stride(1) != 1 or cache.dtype != torch.uint8:
        raise ValueError("cache must be 2-D uint8 with contiguous rows")
    width = cache.shape[1] if width is None else int(width)
    if not 0 <= width <= cache.shape[1]:
        raise ValueError(f"width {width} exceeds the cache row of {cache.shape[1]}")
    _scales_f32(scale, 1, "scale")
    tokens = cache.shape[0] if slot_mapping is None else slot_mapping.numel()
    if out is not None:
        _matrix_out(out, tokens, width, "out", (torch.float32, torch.bfloat16))
    ts = [cache, scale]
    if slot_mapping is not None:
        ts.append(slot_mapping)
        if slot_mapping.dtype.itemsize != 8:
            raise ValueError("slot_mapping must be int64")
    _require_cuda(*ts)
    if out is None:
        out = _out(tokens, width, out_dtype or torch.float32, cache.device)
    _check(lib.nvfp4_kv_fp8_load(_ptr(cache), cache.shape[0], cache.stride(0), width, _ptr(scale),
                                 _ptr(slot_mapping), tokens, _ptr(out), _dtype_code(out.dtype),
                                 out.stride(0), _stream(cache.device)))
    return out
