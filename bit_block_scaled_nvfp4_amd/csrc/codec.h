// NVFP4 codec helpers shared by the encoding kernels (gfx950): element loading, the E4M3 and E2M1
// roundings, block encoding and decoding.  The rounding rules are the ones stated in
// include/nvfp4.h.  Every arithmetic operation is one IEEE binary32 operation in the order written
// (the library is built with -ffp-contract=off and correctly rounded division).  The E2M1 element
// rounding of a block goes through the gfx950 fp4 conversion, which rounds exactly as e2m1_index
// below.  So results are bit-exact with the CPU reference encoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {
namespace codec {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---- element loading: 16 consecutive elements widened exactly to f32 --------------------------

template <nvfp4_dtype DT>
__device__ __forceinline__ void load_block(const void* base, float (&v)[16]);

template <>
__device__ __forceinline__ void load_block<NVFP4_F32>(const void* base, float (&v)[16]) {
  const f32x4* p = reinterpret_cast<const f32x4*>(base);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f32x4 q = __builtin_nontemporal_load(p + i);
    v[4 * i + 0] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
}

template <>
__device__ __forceinline__ void load_block<NVFP4_BF16>(const void* base, float (&v)[16]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    u32x4 q = __builtin_nontemporal_load(p + i);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
      v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
  }
}

template <>
__device__ __forceinline__ void load_block<NVFP4_F16>(const void* base, float (&v)[16]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(base);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    u32x4 q = __builtin_nontemporal_load(p + i);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFFu));
      _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
      v[8 * i + 2 * j + 0] = (float)lo;
      v[8 * i + 2 * j + 1] = (float)hi;
    }
  }
}

template <nvfp4_dtype DT>
constexpr int elem_bytes() {
  return DT == NVFP4_F32 ? 4 : 2;
}

// ---- the two codecs ------------------------------------------------------------------------

// Non-negative binary32 -> OCP E4M3 code: nearest, ties to the even code, >= 448 saturates to
// 0x7E, subnormal codes kept.  Below 2^-6 the E4M3 grid is the multiples of 2^-9, so the code is
// round-to-nearest-even of s * 512 (exact product).  In the normal range the code is the binary32
// pattern rounded to 3 mantissa bits (nearest-even on the 20 dropped bits, carries into the
// exponent are the correct binade change) and rebiased: code = (bits >> 20) - ((127 - 7) << 3).
// Both candidates are formed and one is selected, so the code has no branches (a per-element
// branch costs a divergent exec-mask sequence on this target).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  const uint32_t sub = (uint32_t)__builtin_rintf(s * 512.0f);
  const uint32_t u = __float_as_uint(s);
  const uint32_t nrm = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - 960u;
  const uint32_t c = s < 0.015625f ? sub : nrm;
  return s < 448.0f ? c : 0x7Eu;
}

// Exact binary32 value of an E4M3 code 0x00..0x7E.
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const float sub = (float)c * 0.001953125f;
  const float nrm = __uint_as_float((c + 960u) << 20);
  return c < 8u ? sub : nrm;
}

// Non-negative binary32 (or +inf) -> E2M1 magnitude index: nearest, ties to the even index,
// saturating at 6.  Below 1 the grid is {0, 0.5, 1}: round-to-nearest-even of 2y.  From 1 up the
// grid keeps one mantissa bit: round the pattern to 1 mantissa bit (nearest-even on 22 dropped
// bits) and read exponent and that bit as the index, (bits >> 22) - 252, clamped at 7.
// Branch-free as e4m3_encode.
__device__ __forceinline__ uint32_t e2m1_index(float y) {
  const uint32_t lo = (uint32_t)__builtin_rintf(y * 2.0f);
  const uint32_t u = __float_as_uint(y);
  const uint32_t hi = min(((u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22) - 252u, 7u);
  return y < 1.0f ? lo : hi;
}

// Signed E2M1 codes of fl(v[i] * r) for 16 values, packed two per byte with the even element in
// the low nibble.  Each pair goes through the gfx950 conversion v_cvt_scalef32_pk_fp4_f32 at unit
// scale (the byte it fills is the last operand).  For every binary32 input other than NaN that
// conversion gives exactly e2m1_index(|y|) with the sign bit of y on top, zeros and subnormals
// included; RNE is symmetric, so fl(x * r) carries the sign of x and the magnitude fl(|x| * r).
// A NaN product (0 * inf, only when r is infinite) is the caller's to avoid.
__device__ __forceinline__ void e2m1_pack16(const float (&v)[16], float r, uint32_t (&word)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float* p = v + 8 * h;
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[0] * r, p[1] * r, 1.0f, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[2] * r, p[3] * r, 1.0f, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[4] * r, p[5] * r, 1.0f, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, p[6] * r, p[7] * r, 1.0f, 3);
    word[h] = w;
  }
}

// Scale code and packed element codes of a block: amax, the E4M3 code of fl(amax * gs6), its
// value sd, the element factor r = fl(g / sd) (0 if sd is 0), then the codes of fl(x * r).
// r overflows to +inf only for global scales above about 2^119; there 0 * r is NaN, so such
// blocks take the element-by-element path, whose e2m1_index maps NaN to index 7 as the reference
// encoder does.
__device__ __forceinline__ uint32_t encode_codes(const float (&v)[16], float g, float gs6,
                                                 uint32_t (&word)[2]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sc = e4m3_encode(amax * gs6);
  const float sd = e4m3_value(sc);
  // sd == 0: r = 0 makes every magnitude 0 (finite inputs)
  const float r = sd > 0.0f ? g / sd : 0.0f;
  if (r < __builtin_inff()) {
    e2m1_pack16(v, r, word);
  } else {
    word[0] = 0u;
    word[1] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t code = e2m1_index(fabsf(v[i]) * r) | ((__float_as_uint(v[i]) >> 31) << 3);
      word[i >> 3] |= code << (4 * (i & 7));
    }
  }
  return sc;
}

// Encode 16 binary32 values as block b: one E4M3 scale byte and 8 code bytes.
__device__ __forceinline__ void encode_block(const float (&v)[16], float g, float gs6, uint32_t b,
                                             uint8_t* __restrict__ codes,
                                             uint8_t* __restrict__ scales) {
  uint32_t word[2];
  const uint32_t sc = encode_codes(v, g, gs6, word);
  uint2 out;
  out.x = word[0];
  out.y = word[1];
  *reinterpret_cast<uint2*>(codes + (int64_t)b * 8) = out;
  scales[b] = (uint8_t)sc;
}

// Exact binary32 value of an E2M1 magnitude index 0..7: {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
__device__ __forceinline__ float e2m1_value(uint32_t i) {
  const float lo = 0.5f * (float)i;
  const float hi = __uint_as_float((((i >> 1) + 126u) << 23) | ((i & 1u) << 22));
  return i < 2u ? lo : hi;
}

__device__ __forceinline__ float read_global_scale(const float* g, int dynamic) {
  float v = __builtin_nontemporal_load(g);
  if (!dynamic) return v;
  // dynamic: *g holds amax(|x|) at this point (written by amax_kernel)
  return v == 0.0f ? 1.0f : 2688.0f / v;
}

}  // namespace codec
}  // namespace nvfp4
