// Device helpers shared by the W4A4 product kernels (gfx950).
//
// Exact decode.  An NVFP4 element is V * sd with V an E2M1 value (at most 2 significant bits) and
// sd an E4M3 block scale (at most 4 significant bits, 2^-9 .. 448).  The product has at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in binary16 (normal range), and the
// product of two decoded elements (<= 12 significant bits) is exact in binary32.  The MFMA
// therefore sees the exact NVFP4 values and only its FP32 accumulation rounds.  The hardware's
// scaled FP4 matrix instructions take E8M0 (power-of-two) scales per 32 elements, which cannot
// express E4M3 scales per 16 elements, so the f16 matrix instructions are used.
#pragma once

#include "nvfp4_internal.h"

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// E4M3 code (0x00..0x7E) -> exact binary16 value, via its exact binary32 value.
__device__ __forceinline__ _Float16 e4m3_to_half(uint32_t c) {
  const float f = c < 8u ? (float)c * 0.001953125f : __uint_as_float((c + 960u) << 20);
  return (_Float16)f;
}

// Eight E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i) times the block scale
// -> eight exact binary16 values.  The hardware FP4->F16 conversion runs with a unit scale and the
// block scale is applied with a packed f16 multiply (exact, see above).  Element order inside the
// result is the order the conversion produces for each byte; both operands of a product go
// through this same function, so their contraction slots match.
__device__ __forceinline__ half8_t decode8(uint32_t q, _Float16 s) {
  const half2_t ss = {s, s};
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 0) * ss;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 1) * ss;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 2) * ss;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(q, 1.0f, 3) * ss;
  half8_t r;
  r[0] = p0[0];
  r[1] = p0[1];
  r[2] = p1[0];
  r[3] = p1[1];
  r[4] = p2[0];
  r[5] = p2[1];
  r[6] = p3[0];
  r[7] = p3[1];
  return r;
}

// Segment (calibrated module) of output column n.
__device__ __forceinline__ int column_segment(const SegTable& seg, int n) {
  int j = 0;
#pragma unroll 1
  for (int t = 1; t < seg.nseg; ++t) j += (n >= seg.off[t]) ? 1 : 0;
  return j;
}

// Epilogue factor of output column n: 1 / (gA * gW[seg(n)]).
__device__ __forceinline__ float column_alpha(const SegTable& seg, const float* seg_g, float ga,
                                              int n) {
  return 1.0f / (ga * seg_g[column_segment(seg, n)]);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Store one FP32 value of C (bounds already checked by the caller).
__device__ __forceinline__ void store_c(void* c, int c_bf16, int64_t ldc, int m, int n, float v) {
  if (c_bf16)
    reinterpret_cast<uint16_t*>(c)[(int64_t)m * ldc + n] = f32_to_bf16_rne(v);
  else
    reinterpret_cast<float*>(c)[(int64_t)m * ldc + n] = v;
}

}  // namespace nvfp4
