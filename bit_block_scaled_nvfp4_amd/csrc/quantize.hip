// NVFP4 encoder for gfx950: one FP32 global scale per tensor, one E4M3 scale per 16 consecutive
// elements of a row, E2M1 element codes packed two per byte.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Methodology in Plain English" (E2M1 values with an E4M3 scale per 16-element block; the block's
// largest value fixes the scale) and "Main Findings" (one FP32 global scale per module).  The
// rounding rules the pages leave open are the ones stated in include/nvfp4.h; every arithmetic
// operation below is one IEEE binary32 operation in that order (this file is built with
// -ffp-contract=off and correctly rounded division) and the E2M1 and bfloat16 roundings are gfx950
// conversions that round to nearest-even, so the codes are bit-exact with the CPU reference
// encoder.
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
//
// Fast path: y = fl(fl(g * rcp(fl(1 + exp2(fl(g * c))))) * u) in binary32, c = fl(-log2 e), with
// the hardware 2^x and reciprocal (each within one ulp).  Rounding g * c moves the argument of 2^x
// by at most 2|g| units of 2^-24 relative to e^-g; that error reaches 1 + e^-g scaled by
// e^-g / (1 + e^-g) < 1.  With the two instruction errors and four roundings, y is within
// (2|g| + 7) units of 2^-24 relative to the exact value, i.e. under 40 ulps for |g| <= 16.  So when
// y is a normal number whose low 16 bits are more than 64 away from 0x8000 (a bfloat16 midpoint),
// its nearest-even bfloat16 (v_cvt_pk_bf16_f32, two values at a time) is the rounding of the exact
// value.  Every other case (|g| > 16; y zero, subnormal, infinite or NaN; y near a midpoint) is
// evaluated in binary64 as g / (1 + exp(-g)) * u, in that order, and rounded from there.
//
// Each element's check is a single predicate and the binary64 path a single branch per element:
// with the fast values formed without branches the compiler interleaves the elements, which nested
// per-element branches prevent.
__device__ __forceinline__ float silu_mul_bf16_exact(float g, float u) {
  const double gd = g, ud = u;
  return bf16_round_from_f64(gd / (1.0 + exp(-gd)) * ud);
}

// The binary32 fast value y and whether its bfloat16 rounding is certified.
__device__ __forceinline__ float silu_mul_f32(float g, float u, bool& ok) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  const float s = g * __builtin_amdgcn_rcpf(1.0f + e);
  const float y = s * u;
  const uint32_t yb = __float_as_uint(y);
  const bool normal = __builtin_amdgcn_classf(y, (1 << 3) | (1 << 8));  // -normal, +normal
  const bool off_mid = ((yb - (0x8000u - 64u)) & 0xFFFFu) > 128u;
  ok = (fabsf(g) <= 16.0f) & normal & off_mid;
  return y;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bfloat16 values (as binary32) of SiLU(g0) * u0 and SiLU(g1) * u1.
__device__ __forceinline__ void silu_mul_pair(float g0, float u0, float g1, float u1, float& r0,
                                              float& r1) {
  bool ok0, ok1;
  const float y0 = silu_mul_f32(g0, u0, ok0);
  const float y1 = silu_mul_f32(g1, u1, ok1);
  const bf16x2_t b = __builtin_convertvector((f32x2_t){y0, y1}, bf16x2_t);
  const uint32_t w = __builtin_bit_cast(uint32_t, b);
  r0 = ok0 ? __uint_as_float(w << 16) : silu_mul_bf16_exact(g0, u0);
  r1 = ok1 ? __uint_as_float(w & 0xFFFF0000u) : silu_mul_bf16_exact(g1, u1);
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

// Raise *out to the workgroup's largest per-thread value m >= 0.  For non-negative floats the
// unsigned order of the bit patterns is the numeric order, so atomicMax on the pattern is the
// float max (exact and order-free).  The workgroup first reduces through shuffles and one LDS slot
// per wavefront, and its one atomic is skipped when the cell already holds at least m: every
// workgroup updating one address would otherwise serialise thousands of atomics.  A stale read of
// the cell can only cost an extra atomic.  Called by every thread of the workgroup.
__device__ __forceinline__ void publish_max(float m, float* out) {
  __shared__ float wave_max[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, wave_max[w]);
    unsigned int* cell = reinterpret_cast<unsigned int*>(out);
    const unsigned int cur = __hip_atomic_load(cell, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(m) > cur) atomicMax(cell, __float_as_uint(m));
  }
}

// Tensor-wide max |x| into *out (as publish_max).  *out must hold +0.0 before the launch.
template <nvfp4_dtype DT>
__global__ void __launch_bounds__(kThreads)
amax_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t nb, uint32_t total,
            float* out) {
  float m = 0.0f;
  const uint32_t stride = gridDim.x * kThreads;
  uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  // four blocks in flight per thread (the grid is one workgroup per compute unit)
  const uint32_t unrolled_end = total > 3u * stride ? total - 3u * stride : 0u;
  for (; b < unrolled_end; b += 4u * stride) {
    float v[4][16];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t bu = b + (uint32_t)u * stride;
      const uint32_t row = bu / nb;
      const uint32_t j = bu - row * nb;
      load_block<DT>(x + (int64_t)row * ldx_bytes + (int64_t)j * 16 * elem_bytes<DT>(), v[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[u][i]));
  }
  for (; b < total; b += stride) {
    const uint32_t row = b / nb;
    const uint32_t j = b - row * nb;
    float v[16];
    load_block<DT>(x + (int64_t)row * ldx_bytes + (int64_t)j * 16 * elem_bytes<DT>(), v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  publish_max(m, out);
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
  for (int i = 0; i < 16; i += 2) silu_mul_pair(gv[i], uv[i], gv[i + 1], uv[i + 1], v[i], v[i + 1]);
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
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; i += 2) silu_mul_pair(gv[i], uv[i], gv[i + 1], uv[i + 1], v[i], v[i + 1]);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  publish_max(m, out);
}

__global__ void fill_zero_kernel(float* p) { *p = 0.0f; }

__global__ void finalize_dynamic_scale_kernel(float* p) {
  const float amax = *p;
  *p = amax == 0.0f ? 1.0f : 2688.0f / amax;
}

// Workgroups of the max pass over `total` blocks: one per compute unit (fewer workgroups mean
// fewer atomics on the one cell; each thread keeps four blocks of loads in flight instead).
hipError_t amax_grid(uint32_t total, uint32_t* grid) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const uint32_t need = (total + kThreads - 1) / kThreads;
  *grid = need < (uint32_t)(cus > 0 ? cus : 1) ? need : (uint32_t)(cus > 0 ? cus : 1);
  return hipSuccess;
}

template <nvfp4_dtype DT>
hipError_t launch_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, float* g,
                        int dynamic, uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const uint32_t total = (uint32_t)(rows * (cols / 16));
  const int64_t ldx_bytes = ldx * elem_bytes<DT>();
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  if (dynamic) {
    uint32_t grid = 0;
    if (total > 0) {
      const hipError_t e = amax_grid(total, &grid);  // before any launch
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(1), 0, stream, g);
    if (total > 0)
      hipLaunchKernelGGL(amax_kernel<DT>, dim3(grid), dim3(kThreads), 0, stream, xb, ldx_bytes, nb,
                         total, g);
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
  uint32_t grid = 0;
  if (total > 0) {
    const hipError_t e = amax_grid(total, &grid);  // before any launch
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(1), 0, stream, cell);
  if (total > 0) {
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
