// NVFP4 fake quantization, quantization-error statistics and re-encoding under another global
// scale (checkpoint-side harmonization of fused modules), gfx950.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Methodology in Plain English" (exactly the 4-bit rounding error is injected by quantizing,
// dequantizing and continuing in high precision; the fused modules' global scales are harmonized
// on the checkpoint side) and "Main Findings" (per-token activation error, weight error and the
// share of 16-element blocks dominated by one value).  The readings the pages leave open are
// stated in include/nvfp4.h:
//   dequantized value  fl32(V * sd / g)  -- the exact product V * sd divided once by g;
//   dominated block    2 * amax^2 > sum of the 16 squares, in binary64, summed in element order.
//
// Work split.  Fake quantization and re-encoding: one thread per 16-element block, consecutive
// threads on consecutive blocks of a row (as the encoder), bound by HBM.  The fake-quantized
// output (64 or 32 bytes per thread) leaves through LDS so that every store instruction of a
// wavefront writes 1 KiB of consecutive memory; a lane writing its own 64 bytes in four 16-byte
// stores runs at less than half the rate.  Statistics: one wavefront
// per row, lane l taking blocks l, l + 64, ... and accumulating in binary64; the lanes' sums meet in
// a fixed butterfly, so the result is deterministic.
#include "codec.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace codec;

constexpr int kThreads = 256;

// Dequantized values fl(V * sd / g) of the 16 E2M1 codes c[i] (sign in bit 3) of a block with
// decoded scale sd under global scale g.  Every E2M1 magnitude is 2^k * m with m in {1, 1.5} and
// k in {-1, 0, 1, 2}, and in the binary32 normal range rounding commutes with scaling by a power
// of two, so fl(2^k * m * sd / g) = 2^k * fl(m * sd / g): two correctly rounded divisions per
// block (t1 = fl(sd / g), t15 = fl(1.5 sd / g)) and an exact ldexp per element.  When t1 / 2 or
// 4 * t15 would leave the normal range (then some scaled value might), every element is divided
// on its own instead.
__device__ __forceinline__ void dequant_block(const uint32_t (&c)[16], float sd, float g,
                                              float (&xh)[16]) {
  const float t1 = sd / g;
  const float t15 = (1.5f * sd) / g;  // 1.5 * sd is exact
  if (t1 >= 0x1p-125f && t15 <= 0x1p125f) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t i = c[k] & 7u;
      const float base = (i & 1u) && i >= 2u ? t15 : t1;
      const int e = i >= 2u ? (int)(i >> 1) - 1 : -1;
      const float v = i == 0u ? 0.0f : __builtin_ldexpf(base, e);
      xh[k] = __uint_as_float(__float_as_uint(v) | ((c[k] & 8u) << 28));
    }
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float v = (e2m1_value(c[k] & 7u) * sd) / g;  // V * sd is exact
      xh[k] = __uint_as_float(__float_as_uint(v) | ((c[k] & 8u) << 28));
    }
  }
}

// Encode the 16 values of a block (as the encoder does) and return their dequantized values.
__device__ __forceinline__ void fake_quantize_block(const float (&v)[16], float g, float gs6,
                                                    float (&xh)[16]) {
  uint32_t word[2];
  const float sd = e4m3_value(encode_codes(v, g, gs6, word));
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = (word[i >> 3] >> (4 * (i & 7))) & 0xFu;
  dequant_block(c, sd, g, xh);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <nvfp4_dtype DT, bool BF16_OUT>
__global__ void __launch_bounds__(kThreads)
fake_quantize_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t nb, uint32_t total,
                     const float* __restrict__ gptr, int dynamic, uint8_t* __restrict__ out,
                     int64_t ldo_bytes) {
  // per-thread output: 64 bytes (f32) or 32 bytes (bf16), staged in LDS so that each store
  // instruction of a wavefront writes 64 consecutive 16-byte pieces
  constexpr int kOutBytes = BF16_OUT ? 32 : 64;
  constexpr int kPieces = kOutBytes / 16;
  __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads * kOutBytes];
  const uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = threadIdx.x >> 6;
  uint8_t* ws = stage + wave * 64 * kOutBytes;
  const float g = read_global_scale(gptr, dynamic);
  const float gs6 = g / 6.0f;
  const uint32_t bb = b < total ? b : total - 1;
  const uint32_t row = bb / nb;
  const uint32_t j = bb - row * nb;
  float v[16], xh[16];
  load_block<DT>(x + (int64_t)row * ldx_bytes + (int64_t)j * 16 * elem_bytes<DT>(), v);
  fake_quantize_block(v, g, gs6, xh);
  if constexpr (BF16_OUT) {
    u32x4* d = reinterpret_cast<u32x4*>(ws + lane * 32);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 o;
      o.x = bf16_rne(xh[8 * i + 0]) | (bf16_rne(xh[8 * i + 1]) << 16);
      o.y = bf16_rne(xh[8 * i + 2]) | (bf16_rne(xh[8 * i + 3]) << 16);
      o.z = bf16_rne(xh[8 * i + 4]) | (bf16_rne(xh[8 * i + 5]) << 16);
      o.w = bf16_rne(xh[8 * i + 6]) | (bf16_rne(xh[8 * i + 7]) << 16);
      d[i] = o;
    }
  } else {
    f32x4* d = reinterpret_cast<f32x4*>(ws + lane * 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 o;
      o.x = xh[4 * i + 0];
      o.y = xh[4 * i + 1];
      o.z = xh[4 * i + 2];
      o.w = xh[4 * i + 3];
      d[i] = o;
    }
  }
  // LDS accesses of one wavefront complete in order; the stage rows belong to this wavefront
  const uint32_t wb = blockIdx.x * kThreads + wave * 64;  // first block of the wavefront
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const uint32_t q = i * 64 + lane;           // piece index within the wavefront's output
    const uint32_t t = q / kPieces;             // owning lane
    const uint32_t ob = wb + t;
    if (ob < total) {
      const uint32_t orow = ob / nb;
      const uint32_t oj = ob - orow * nb;
      const u32x4 val = *reinterpret_cast<const u32x4*>(ws + q * 16);
      __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(
          out + (int64_t)orow * ldo_bytes + (int64_t)oj * kOutBytes + (q % kPieces) * 16));
    }
  }
}

// One wavefront per row: squared error of the fake quantization, squared norm, dominated blocks.
template <nvfp4_dtype DT>
__global__ void __launch_bounds__(kThreads)
quant_error_stats_kernel(const uint8_t* __restrict__ x, int64_t ldx_bytes, uint32_t nb,
                         uint32_t rows, const float* __restrict__ gptr, int dynamic,
                         double* __restrict__ err2, double* __restrict__ norm2,
                         int32_t* __restrict__ dominated) {
  const uint32_t row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const uint32_t lane = threadIdx.x & 63;
  if (row >= rows) return;  // the whole wavefront leaves together
  const float g = read_global_scale(gptr, dynamic);
  const float gs6 = g / 6.0f;
  double e = 0.0, n = 0.0;
  int dom = 0;
  for (uint32_t j = lane; j < nb; j += 64) {
    float v[16], xh[16];
    load_block<DT>(x + (int64_t)row * ldx_bytes + (int64_t)j * 16 * elem_bytes<DT>(), v);
    fake_quantize_block(v, g, gs6, xh);
    double bt = 0.0;
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const double xd = (double)v[i];
      const double d = (double)xh[i] - xd;  // exact unless the two are 2^29 apart in size
      e += d * d;
      bt = bt + xd * xd;  // element order: the dominance decision uses this exact sequence
      amax = fmaxf(amax, fabsf(v[i]));
    }
    n += bt;
    const double a = (double)amax;
    dom += (amax > 0.0f && 2.0 * a * a > bt) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    e += __shfl_xor(e, o, 64);
    n += __shfl_xor(n, o, 64);
    dom += __shfl_xor(dom, o, 64);
  }
  if (lane == 0) {
    err2[row] = e;
    norm2[row] = n;
    dominated[row] = dom;
  }
}

// Re-encode block b of an NVFP4 tensor from the global scale of its row's segment to g_out (or to
// the smallest segment scale).  A thread reads its block whole before writing it, so the output may
// be the input itself.
__global__ void __launch_bounds__(kThreads)
requantize_kernel(const uint8_t* codes, const uint8_t* scales, uint32_t nb, uint32_t total,
                  SegTable seg, const float* __restrict__ g_in, const float* __restrict__ g_out,
                  float* g_shared, uint8_t* codes_out, uint8_t* scales_out) {
  const uint32_t b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= total) return;
  const int32_t row = (int32_t)(b / nb);
  int s = 0;
  float gmin = g_in[0];
  for (int k = 1; k < seg.nseg; ++k) {
    if (row >= seg.off[k]) s = k;
    gmin = fminf(gmin, g_in[k]);
  }
  const float gi = g_in[s];
  const float go = g_out ? *g_out : gmin;
  if (g_shared && b == 0) *g_shared = go;
  const uint2 cw = *reinterpret_cast<const uint2*>(codes + (int64_t)b * 8);
  const uint32_t w[2] = {cw.x, cw.y};
  uint32_t c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = (w[i >> 3] >> (4 * (i & 7))) & 0xFu;
  float xh[16];
  dequant_block(c, e4m3_value(scales[b]), gi, xh);
  encode_block(xh, go, go / 6.0f, b, codes_out, scales_out);
}

template <nvfp4_dtype DT>
hipError_t launch_fake_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, float* g,
                             int dynamic, void* out, nvfp4_dtype out_dt, int64_t ldo,
                             hipStream_t stream) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const uint32_t total = (uint32_t)(rows * (cols / 16));
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  uint8_t* ob = reinterpret_cast<uint8_t*>(out);
  if (dynamic) {
    const hipError_t e = launch_dynamic_amax(x, DT, rows, cols, ldx, g, stream);
    if (e != hipSuccess) return e;
  }
  if (total > 0) {
    const uint32_t grid = (total + kThreads - 1) / kThreads;
    if (out_dt == NVFP4_BF16)
      hipLaunchKernelGGL((fake_quantize_kernel<DT, true>), dim3(grid), dim3(kThreads), 0, stream,
                         xb, ldx * elem_bytes<DT>(), nb, total, g, dynamic, ob, ldo * 2);
    else
      hipLaunchKernelGGL((fake_quantize_kernel<DT, false>), dim3(grid), dim3(kThreads), 0, stream,
                         xb, ldx * elem_bytes<DT>(), nb, total, g, dynamic, ob, ldo * 4);
  }
  if (dynamic) return launch_finalize_dynamic(g, stream);
  return hipGetLastError();
}

template <nvfp4_dtype DT>
hipError_t launch_stats_typed(const void* x, int64_t rows, int64_t cols, int64_t ldx, float* g,
                              int dynamic, double* err2, double* norm2, int32_t* dominated,
                              hipStream_t stream) {
  const uint32_t nb = (uint32_t)(cols / 16);
  if (dynamic) {
    const hipError_t e = launch_dynamic_amax(x, DT, rows, cols, ldx, g, stream);
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    const uint32_t grid = (uint32_t)((rows + kThreads / 64 - 1) / (kThreads / 64));
    hipLaunchKernelGGL(quant_error_stats_kernel<DT>, dim3(grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint8_t*>(x), ldx * elem_bytes<DT>(), nb,
                       (uint32_t)rows, g, dynamic, err2, norm2, dominated);
  }
  if (dynamic) return launch_finalize_dynamic(g, stream);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fake_quantize(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                int64_t ldx, float* g, int dynamic, void* out, nvfp4_dtype out_dt,
                                int64_t ldo, hipStream_t stream) {
  switch (dt) {
    case NVFP4_F32:
      return launch_fake_typed<NVFP4_F32>(x, rows, cols, ldx, g, dynamic, out, out_dt, ldo, stream);
    case NVFP4_BF16:
      return launch_fake_typed<NVFP4_BF16>(x, rows, cols, ldx, g, dynamic, out, out_dt, ldo, stream);
    case NVFP4_F16:
      return launch_fake_typed<NVFP4_F16>(x, rows, cols, ldx, g, dynamic, out, out_dt, ldo, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_quant_error_stats(const void* x, nvfp4_dtype dt, int64_t rows, int64_t cols,
                                    int64_t ldx, float* g, int dynamic, double* err2,
                                    double* norm2, int32_t* dominated, hipStream_t stream) {
  switch (dt) {
    case NVFP4_F32:
      return launch_stats_typed<NVFP4_F32>(x, rows, cols, ldx, g, dynamic, err2, norm2, dominated,
                                           stream);
    case NVFP4_BF16:
      return launch_stats_typed<NVFP4_BF16>(x, rows, cols, ldx, g, dynamic, err2, norm2, dominated,
                                            stream);
    case NVFP4_F16:
      return launch_stats_typed<NVFP4_F16>(x, rows, cols, ldx, g, dynamic, err2, norm2, dominated,
                                           stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_requantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, const SegTable& seg, const float* g_in,
                             const float* g_out, float* g_shared, uint8_t* codes_out,
                             uint8_t* scales_out, hipStream_t stream) {
  const uint32_t nb = (uint32_t)(cols / 16);
  const uint32_t total = (uint32_t)(rows * (cols / 16));
  if (total == 0) return hipSuccess;
  const uint32_t grid = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(requantize_kernel, dim3(grid), dim3(kThreads), 0, stream, codes, scales, nb,
                     total, seg, g_in, g_out, g_shared, codes_out, scales_out);
  return hipGetLastError();
}

}  // namespace nvfp4
