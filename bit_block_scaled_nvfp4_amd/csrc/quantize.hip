// NVFP4 encoder for gfx950: one FP32 global scale per tensor, one E4M3 scale per 16 consecutive
// elements of a row, E2M1 element codes packed two per byte.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Methodology in Plain English" (E2M1 values with an E4M3 scale per 16-element block; the block's
// largest value fixes the scale) and "Main Findings" (one FP32 global scale per module).  The
// rounding rules the pages leave open are the ones stated in include/nvfp4.h; every operation
// below is one IEEE binary32 operation in that order (this file is built with -ffp-contract=off
// and correctly rounded division), so the codes are bit-exact with the CPU reference encoder.
//
// Work split: one thread encodes one 16-element block (32 bytes of bf16/f16 or 64 bytes of f32 in,
// 8 code bytes and 1 scale byte out).  Consecutive threads take consecutive blocks of a row, so
// loads and stores of a wavefront are contiguous.  The kernel is bound by HBM bandwidth.
#include "codec.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace codec;

constexpr int kThreads = 256;

// ---- SiLU(g) * u rounded once to bfloat16 ---------------------------------------------------

// Nearest bfloat16 value of a binary64 x (ties to the even significand), returned as the
// binary32 holding it.  bfloat16 keeps 8 significant bits and binary32's exponent range: in the
// normal range the binary64 pattern is rounded to 7 explicit mantissa bits (nearest-even on the 45
// dropped bits; a carry into the exponent is the correct binade change, up to +inf); below 2^-126
// the grid is the multiples of 2^-133, reached by an exact power-of-two scaling and rint.
__device__ __forceinline__ float bf16_round_from_f64(double x) {
  const uint64_t bits = (uint64_t)__double_as_longlong(x);
  const uint64_t sign = bits & 0x8000000000000000ull;
  const uint64_t mag = bits ^ sign;
  if (mag >= 0x47F0000000000000ull) return (float)x;  // |x| >= 2^128, inf, NaN
  if (mag < 0x3810000000000000ull)                    // |x| < 2^-126
    return (float)(__builtin_rint(x * 0x1p133) * 0x1p-133);
  const uint64_t r = (mag + ((1ull << 44) - 1ull) + ((mag >> 45) & 1ull)) & ~((1ull << 45) - 1ull);
  return (float)__longlong_as_double((long long)(r | sign));
}

// bfloat16 value of SiLU(g) * u = g / (1 + e^-g) * u, rounded once from the exact value.
// Fast path (|g| <= 16): binary32 with the hardware 2^x and reciprocal.  Its relative error is
// below 40 units in the last place of the binary32 result (argument rounding of -g log2(e) with
// |g| <= 16 contributes at most 16 ulp through 2^x, the 2^x and reciprocal instructions about one
// ulp each, four roundings half an ulp each), so rounding it to bfloat16 gives the same result as
// rounding the exact value unless it lies within 64 ulps of a bfloat16 midpoint (low 16 bits
// 0x8000).  Those cases, |g| > 16 and results that are zero, subnormal or not finite are
// evaluated in binary64 (g / (1 + exp(-g)) * u, in that order) and rounded from there.
__device__ __forceinline__ float silu_mul_bf16(float g, float u) {
  if (fabsf(g) <= 16.0f) {
    const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
    const float s = g * __builtin_amdgcn_rcpf(1.0f + e);
    const float y = s * u;
    const uint32_t yb = __float_as_uint(y);
    const uint32_t ex = (yb >> 23) & 0xFFu;
    const uint32_t low = yb & 0xFFFFu;
    if (ex != 0u && ex != 0xFFu && (low < 0x8000u - 64u || low > 0x8000u + 64u))
      return __uint_as_float((yb + 0x7FFFu + ((yb >> 16) & 1u)) & 0xFFFF0000u);
  }
  const double gd = g, ud = u;
  return bf16_round_from_f64(gd / (1.0 + exp(-gd)) * ud);
}

template <nvfp4_dtype DT>
__global__ void __launch_bounds__(kThreads)
quantize_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t nb, uint32_t total,
                const float* __restrict__ gptr, int dynamic, uint8_t* __restrict__ codes,
                uint8_t* __restrict__ scales) {
  const uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= total) return;
  const float g = read_global_scale(gptr, dynamic);
  const float gs6 = g / 6.0f;
  const uint32_t row = b / nb;
  const uint32_t j = b - row * nb;

  float v[16];
  load_block<DT>(x + (int64_t)row * ldx_bytes + (int64_t)j * 16 * elem_bytes<DT>(), v);

  encode_block(v, g, gs6, b, codes, scales);
}

// Tensor-wide max |x| (exact, order-free) into *out as a binary32 bit pattern: for non-negative
// floats the unsigned integer order of the bit patterns is the numeric order, so atomicMax on the
// pattern is the float max.  *out must hold +0.0 before the launch.
template <nvfp4_dtype DT>
__global__ void __launch_bounds__(kThreads)
amax_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t nb, uint32_t total,
            float* out) {
  float m = 0.0f;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t row = b / nb;
    const uint32_t j = b - row * nb;
    float v[16];
    load_block<DT>(x + (int64_t)row * ldx_bytes + (int64_t)j * 16 * elem_bytes<DT>(), v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0 && m > 0.0f)
    atomicMax(reinterpret_cast<unsigned int*>(out), __float_as_uint(m));
}

// Fused SiLU(g) * u -> NVFP4: block b of the activation is formed from blocks b of gate and up
// (each element rounded once to bfloat16) and encoded exactly like quantize_kernel's blocks.
template <nvfp4_dtype DT>
__global__ void __launch_bounds__(kThreads)
silu_mul_quantize_kernel(const uint8_t* __restrict__ gate, int64_t ldg_bytes,
                         const uint8_t* __restrict__ up, int64_t ldu_bytes, uint32_t nb,
                         uint32_t total, const float* __restrict__ gptr, int dynamic,
                         uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= total) return;
  const float g = read_global_scale(gptr, dynamic);
  const float gs6 = g / 6.0f;
  const uint32_t row = b / nb;
  const uint32_t j = b - row * nb;
  float gv[16], uv[16], v[16];
  load_block<DT>(gate + (int64_t)row * ldg_bytes + (int64_t)j * 16 * elem_bytes<DT>(), gv);
  load_block<DT>(up + (int64_t)row * ldu_bytes + (int64_t)j * 16 * elem_bytes<DT>(), uv);
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = silu_mul_bf16(gv[i], uv[i]);
  encode_block(v, g, gs6, b, codes, scales);
}

// max |SiLU(g) * u| (each element rounded to bfloat16) into *out, as amax_kernel.
template <nvfp4_dtype DT>
__global__ void __launch_bounds__(kThreads)
silu_mul_amax_kernel(const uint8_t* __restrict__ gate, int64_t ldg_bytes,
                     const uint8_t* __restrict__ up, int64_t ldu_bytes, uint32_t nb,
                     uint32_t total, float* out) {
  float m = 0.0f;
  for (uint32_t b = blockIdx.x * kThreads + threadIdx.x; b < total; b += gridDim.x * kThreads) {
    const uint32_t row = b / nb;
    const uint32_t j = b - row * nb;
    float gv[16], uv[16];
    load_block<DT>(gate + (int64_t)row * ldg_bytes + (int64_t)j * 16 * elem_bytes<DT>(), gv);
    load_block<DT>(up + (int64_t)row * ldu_bytes + (int64_t)j * 16 * elem_bytes<DT>(), uv);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(silu_mul_bf16(gv[i], uv[i])));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0 && m > 0.0f)
    atomicMax(reinterpret_cast<unsigned int*>(out), __float_as_uint(m));
}

__global__ void fill_zero_kernel(float* p) { *p = 0.0f; }

__global__ void finalize_dynamic_scale_kernel(float* p) {
  const float amax = *p;
  *p = amax == 0.0f ? 1.0f : 2688.0f / amax;
}

template <nvfp4_dtype DT>
hipError_t launch_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, float* g,
                        int dynamic, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const uint32_t total = (uint32_t)(rows * (cols / 16));
  const int64_t ldx_bytes = ldx * elem_bytes<DT>();
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  if (dynamic) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(1), 0, stream, g);
    if (total > 0) {
      uint32_t grid = (total + kThreads - 1) / kThreads;
      grid = grid > 4096u ? 4096u : grid;
      hipLaunchKernelGGL(amax_kernel<DT>, dim3(grid), dim3(kThreads), 0, stream, xb, ldx_bytes, nb,
                         total, g);
    }
  }
  if (total > 0) {
    const uint32_t grid = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(quantize_kernel<DT>, dim3(grid), dim3(kThreads), 0, stream, xb, ldx_bytes,
                       nb, total, g, dynamic, codes, scales);
  }
  if (dynamic) hipLaunchKernelGGL(finalize_dynamic_scale_kernel, dim3(1), dim3(1), 0, stream, g);
  return hipGetLastError();
}

template <nvfp4_dtype DT>
hipError_t launch_silu_typed(const void* gate, const void* up, int64_t rows, int64_t cols,
                             int64_t ldg, int64_t ldu, float* g, int dynamic, uint8_t* codes,
                             uint8_t* scales, hipStream_t stream) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const uint32_t total = (uint32_t)(rows * (cols / 16));
  const int64_t ldg_bytes = ldg * elem_bytes<DT>(), ldu_bytes = ldu * elem_bytes<DT>();
  const uint8_t* gb = reinterpret_cast<const uint8_t*>(gate);
  const uint8_t* ub = reinterpret_cast<const uint8_t*>(up);
  if (dynamic) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(1), 0, stream, g);
    if (total > 0) {
      uint32_t grid = (total + kThreads - 1) / kThreads;
      grid = grid > 4096u ? 4096u : grid;
      hipLaunchKernelGGL(silu_mul_amax_kernel<DT>, dim3(grid), dim3(kThreads), 0, stream, gb,
                         ldg_bytes, ub, ldu_bytes, nb, total, g);
    }
  }
  if (total > 0) {
    const uint32_t grid = (total + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(silu_mul_quantize_kernel<DT>, dim3(grid), dim3(kThreads), 0, stream, gb,
                       ldg_bytes, ub, ldu_bytes, nb, total, g, dynamic, codes, scales);
  }
  if (dynamic) hipLaunchKernelGGL(finalize_dynamic_scale_kernel, dim3(1), dim3(1), 0, stream, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_silu_mul_quantize(const void* gate, const void* up, nvfp4_dtype dt,
                                    int64_t rows, int64_t cols, int64_t ldg, int64_t ldu,
                                    float* g, int dynamic, uint8_t* codes, uint8_t* scales,
                                    hipStream_t stream) {
  switch (dt) {
    case NVFP4_F32:
      return launch_silu_typed<NVFP4_F32>(gate, up, rows, cols, ldg, ldu, g, dynamic, codes,
                                          scales, stream);
    case NVFP4_BF16:
      return launch_silu_typed<NVFP4_BF16>(gate, up, rows, cols, ldg, ldu, g, dynamic, codes,
                                           scales, stream);
    case NVFP4_F16:
      return launch_silu_typed<NVFP4_F16>(gate, up, rows, cols, ldg, ldu, g, dynamic, codes,
                                          scales, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dynamic_amax(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                               int64_t ldx, float* cell, hipStream_t stream) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const uint32_t total = (uint32_t)(rows * (cols / 16));
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(1), 0, stream, cell);
  if (total > 0) {
    uint32_t grid = (total + kThreads - 1) / kThreads;
    grid = grid > 4096u ? 4096u : grid;
    switch (dt) {
      case NVFP4_F32:
        hipLaunchKernelGGL(amax_kernel<NVFP4_F32>, dim3(grid), dim3(kThreads), 0, stream, xb,
                           ldx * 4, nb, total, cell);
        break;
      case NVFP4_BF16:
        hipLaunchKernelGGL(amax_kernel<NVFP4_BF16>, dim3(grid), dim3(kThreads), 0, stream, xb,
                           ldx * 2, nb, total, cell);
        break;
      case NVFP4_F16:
        hipLaunchKernelGGL(amax_kernel<NVFP4_F16>, dim3(grid), dim3(kThreads), 0, stream, xb,
                           ldx * 2, nb, total, cell);
        break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_finalize_dynamic(float* cell, hipStream_t stream) {
  hipLaunchKernelGGL(finalize_dynamic_scale_kernel, dim3(1), dim3(1), 0, stream, cell);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols, int64_t ldx,
                           float* g, int dynamic, uint8_t* codes, uint8_t* scales,
                           hipStream_t stream) {
  switch (dt) {
    case NVFP4_F32:
      return launch_typed<NVFP4_F32>(x, rows, cols, ldx, g, dynamic, codes, scales, stream);
    case NVFP4_BF16:
      return launch_typed<NVFP4_BF16>(x, rows, cols, ldx, g, dynamic, codes, scales, stream);
    case NVFP4_F16:
      return launch_typed<NVFP4_F16>(x, rows, cols, ldx, g, dynamic, codes, scales, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace nvfp4
