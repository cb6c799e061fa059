// W4A4 NVFP4 product for decode-shaped problems (M <= 16 activation rows), gfx950.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Main Findings": decode is weight-bandwidth-bound, so the work here is streaming the NVFP4
// weights once at HBM rate while the few activation rows ride along.
//
// Layout of the work: a workgroup owns 16 output columns (16 weight rows) and all M <= 16 rows;
// its 8 wavefronts split K into equal runs of 128-element chunks.  Each wavefront issues every
// global load of its run up front (weights 16 B per lane per chunk, activations likewise), then
// decodes and contracts with v_mfma_f32_16x16x32_f16 (A = activations padded to 16 rows with
// zeros, B = weights).  The 8 partial 16x16 tiles are summed through LDS in a fixed order (so the
// result is deterministic), scaled per column by 1 / (gA * gW[seg(n)]) and stored.
//
// K-slot permutation: in a 16x16x32 MFMA, lane l supplies row/column (l % 16) and 8 of the 32
// k-slots (group g = l / 16).  Within a chunk of 128, lane group g reads the 16 bytes holding
// elements [32g, 32g + 32) of its row and uses 32-bit word j of them in MFMA step j (j = 0..3);
// word j covers elements 32g + 8j .. +7, inside 16-block 2g + j/2.  Both operands use this map.
#include "gemm_common.h"

namespace nvfp4 {
namespace {

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyBatch = 8;  // chunks whose loads are in flight together, per wavefront

typedef float floatx4_t __attribute__((ext_vector_type(4)));

// One wavefront's loads for up to kSkinnyBatch chunks: code words and the two scale bytes each.
struct SkinnyBatch {
  uint4 w[kSkinnyBatch];
  uint4 a[kSkinnyBatch];
  uint32_t ws[kSkinnyBatch];
  uint32_t as[kSkinnyBatch];
};

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

__global__ void __launch_bounds__(kSkinnyWaves * 64)
gemm_skinny_kernel(GemmArgs p) {
  __shared__ floatx4_t partial[kSkinnyWaves][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;  // weight row (output column) and activation row of this lane
  const int g = lane >> 4;  // k group
  const int n0 = blockIdx.x * 16;
  const int nchunks = p.K / 128;
  const int per_wave = (nchunks + kSkinnyWaves - 1) / kSkinnyWaves;
  const int c_begin = min(wave * per_wave, nchunks);
  const int c_end = min(c_begin + per_wave, nchunks);
  const int64_t kb = p.K / 2, ks = p.K / 16;

  const int wrow = min(n0 + r, p.N - 1);
  const bool arow_valid = r < p.M;
  const uint8_t* wc = p.w_codes + wrow * kb + g * 16;
  const uint8_t* wsc = p.w_scales + wrow * ks + g * 2;
  const uint8_t* ac = p.a_codes + (int64_t)min(r, p.M - 1) * kb + g * 16;
  const uint8_t* asc = p.a_scales + (int64_t)min(r, p.M - 1) * ks + g * 2;

  floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c0 = c_begin; c0 < c_end; c0 += kSkinnyBatch) {
    SkinnyBatch b;
    const int nb = min(kSkinnyBatch, c_end - c0);
#pragma unroll
    for (int i = 0; i < kSkinnyBatch; ++i) {
      if (i < nb) {
        const int c = c0 + i;
        b.w[i] = *reinterpret_cast<const uint4*>(wc + c * 64);
        b.ws[i] = load_u16(wsc + c * 8);
        if (arow_valid) {
          b.a[i] = *reinterpret_cast<const uint4*>(ac + c * 64);
          b.as[i] = load_u16(asc + c * 8);
        } else {
          b.a[i] = uint4{0u, 0u, 0u, 0u};
          b.as[i] = 0u;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kSkinnyBatch; ++i) {
      if (i < nb) {
        const half2_t sw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.ws[i], 1.0f, false);
        const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b.as[i], 1.0f, false);
        const uint32_t wq[4] = {b.w[i].x, b.w[i].y, b.w[i].z, b.w[i].w};
        const uint32_t aq[4] = {b.a[i].x, b.a[i].y, b.a[i].z, b.a[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const half8_t bv = decode8(wq[j], j < 2 ? sw[0] : sw[1]);
          const half8_t av = decode8(aq[j], j < 2 ? sa[0] : sa[1]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
        }
      }
    }
  }

  // deterministic reduction of the 8 partial tiles: wave 0 adds waves 1..7 in order
  partial[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kSkinnyWaves; ++w) acc += partial[w][lane];

  // output tile: lane holds column n0 + (l % 16), rows 4 * (l / 16) + e
  const int n = n0 + r;
  if (n >= p.N) return;
  const float alpha = column_alpha(p.seg, p.seg_g, *p.a_g, n);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * g + e;
    if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, acc[e] * alpha);
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  const uint32_t blocks = (a.N + 15) / 16;
  hipLaunchKernelGGL(gemm_skinny_kernel, dim3(blocks), dim3(kSkinnyWaves * 64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
