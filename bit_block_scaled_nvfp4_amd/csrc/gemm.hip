// W4A4 NVFP4 product kernels for gfx950 with the per-segment global-scale epilogue.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Main Findings": both operands NVFP4 (W4A4), one FP32 global scale per calibrated module, and
// fused serving GEMMs whose output segments need their own module's global scale.
//
// C[m, n] = (sum_k a[m,k] * w[n,k]) * alpha[seg(n)],  alpha[j] = 1 / (gA * gW[j]),
// the sum over exactly decoded elements accumulated in FP32 by v_mfma_f32_32x32x16_f16.
//
// Two kernels:
//  * gemm_general_kernel: any K that is a multiple of 16.  One wavefront per 32x32 output tile,
//    operands read straight from global memory 4 bytes (8 codes) per lane per K step.
//  * gemm_tiled_kernel: K a multiple of 64.  A workgroup owns a BM x BN output tile; each K chunk of
//    64 is staged in LDS as raw 4-bit codes plus E4M3 bytes (9/16 byte per element instead of 2 for
//    f16, so staging costs a quarter of the LDS space and bandwidth of an f16 GEMM), then every
//    wavefront decodes its own fragments in registers right before the MFMAs.
//
// K-slot permutation.  In a 32x32x16 MFMA, lane l supplies row (l % 32) and 8 of the 16 k-slots
// (half h = l / 32).  Within a K chunk of 64, lane half h reads the 16 contiguous bytes holding
// elements [32h, 32h + 32) of its row and uses 32-bit word j of them in MFMA step j (j = 0..3).
// A and W use the same map, so after 4 steps every k of the chunk has been contracted once.  Word
// j covers elements 32h + 8j .. +7, which lie in 16-block 2h + j/2 of the chunk.
#include "gemm_common.h"

namespace nvfp4 {
namespace {

// ------------------------------------------------------------------------------------------------
// general kernel
// ------------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(256) gemm_general_kernel(GemmArgs p, uint32_t tiles_n) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t tile = blockIdx.x;
  const int tm = (int)(tile / tiles_n) * 64 + (wave >> 1) * 32;
  const int tn = (int)(tile % tiles_n) * 64 + (wave & 1) * 32;
  if (tm >= p.M || tn >= p.N) return;
  const int r = lane & 31;
  const int h = lane >> 5;
  const int am = min(tm + r, p.M - 1);
  const int wn = min(tn + r, p.N - 1);
  const int64_t kb = p.K / 2, ks = p.K / 16;
  const uint8_t* ac = p.a_codes + am * kb + h * 4;
  const uint8_t* wc = p.w_codes + wn * kb + h * 4;
  const uint8_t* as = p.a_scales + am * ks;
  const uint8_t* ws = p.w_scales + wn * ks;

  floatx16 acc = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    const uint32_t qa = *reinterpret_cast<const uint32_t*>(ac + k0 / 2);
    const uint32_t qw = *reinterpret_cast<const uint32_t*>(wc + k0 / 2);
    const _Float16 sa = e4m3_to_half(as[k0 / 16]);
    const _Float16 sw = e4m3_to_half(ws[k0 / 16]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(decode8(qa, sa), decode8(qw, sw), acc, 0, 0, 0);
  }

  const int n = tn + r;
  if (n >= p.N) return;
  const float alpha = column_alpha(p.seg, p.seg_g, *p.a_g, n);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = tm + 8 * (i / 4) + 4 * h + (i % 4);
    if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, acc[i] * alpha);
  }
}

// ------------------------------------------------------------------------------------------------
// tiled kernel
// ------------------------------------------------------------------------------------------------

template <int WAVES_M, int WAVES_N, int FM, int FN>
struct TileCfg {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int BM = WAVES_M * FM * 32;
  static constexpr int BN = WAVES_N * FN * 32;
  // one stage: codes of BM + BN rows (32 bytes each per K chunk) and their 4 scale bytes
  static constexpr int kCodesA = BM * 32;
  static constexpr int kCodesB = BN * 32;
  static constexpr int kScalesA = BM * 4;
  static constexpr int kScalesB = BN * 4;
  static constexpr int kStage = kCodesA + kCodesB + kScalesA + kScalesB;
  static constexpr int kPiecesA = BM * 2 / kThreads;  // 16-byte pieces per thread
  static constexpr int kPiecesB = BN * 2 / kThreads;
  static constexpr int kScaleWords = (BM + BN) / kThreads;  // 4-byte scale words per thread
  static_assert(BM * 2 % kThreads == 0 && BN * 2 % kThreads == 0, "piece split");
  static_assert((BM + BN) % kThreads == 0, "scale split");
};

template <class Cfg>
struct Prefetch {
  uint4 a[Cfg::kPiecesA];
  uint4 b[Cfg::kPiecesB];
  uint32_t s[Cfg::kScaleWords];
};

// Global -> registers for K chunk `kc` of the tile.  Piece p of an operand holds row
// (p / 64) * 32 + (p % 32), bytes [16 * ((p % 64) / 32), +16) of the chunk, and is stored at LDS
// offset 16 p: each 32-row group becomes 1 KiB laid out [half][row][16 B], which is exactly the
// order in which the 64 lanes of a fragment read it (lane l at 16 l), so fragment reads are
// contiguous and free of bank conflicts.
template <class Cfg>
__device__ __forceinline__ void load_chunk(const GemmArgs& p, int m0, int n0, int kc,
                                           Prefetch<Cfg>& f) {
  const int64_t kb = p.K / 2, ks = p.K / 16;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesA; ++i) {
    const int pc = tid + i * Cfg::kThreads;
    const int row = (pc >> 6) * 32 + (pc & 31);
    const int gm = min(m0 + row, p.M - 1);
    f.a[i] = *reinterpret_cast<const uint4*>(p.a_codes + gm * kb + kc * 32 + ((pc >> 5) & 1) * 16);
  }
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesB; ++i) {
    const int pc = tid + i * Cfg::kThreads;
    const int row = (pc >> 6) * 32 + (pc & 31);
    const int gn = min(n0 + row, p.N - 1);
    f.b[i] = *reinterpret_cast<const uint4*>(p.w_codes + gn * kb + kc * 32 + ((pc >> 5) & 1) * 16);
  }
#pragma unroll
  for (int i = 0; i < Cfg::kScaleWords; ++i) {
    const int w = tid + i * Cfg::kThreads;
    if (w < Cfg::BM) {
      const int gm = min(m0 + w, p.M - 1);
      f.s[i] = *reinterpret_cast<const uint32_t*>(p.a_scales + gm * ks + kc * 4);
    } else {
      const int gn = min(n0 + (w - Cfg::BM), p.N - 1);
      f.s[i] = *reinterpret_cast<const uint32_t*>(p.w_scales + gn * ks + kc * 4);
    }
  }
}

template <class Cfg>
__device__ __forceinline__ void store_chunk(uint8_t* stage, const Prefetch<Cfg>& f) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesA; ++i)
    *reinterpret_cast<uint4*>(stage + (tid + i * Cfg::kThreads) * 16) = f.a[i];
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesB; ++i)
    *reinterpret_cast<uint4*>(stage + Cfg::kCodesA + (tid + i * Cfg::kThreads) * 16) = f.b[i];
#pragma unroll
  for (int i = 0; i < Cfg::kScaleWords; ++i)
    *reinterpret_cast<uint32_t*>(stage + Cfg::kCodesA + Cfg::kCodesB +
                                 (tid + i * Cfg::kThreads) * 4) = f.s[i];
}

template <int WAVES_M, int WAVES_N, int FM, int FN>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64)
gemm_tiled_kernel(GemmArgs p, uint32_t tiles_n) {
  using Cfg = TileCfg<WAVES_M, WAVES_N, FM, FN>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int h = lane >> 5;
  const int r = lane & 31;
  const uint32_t tile = blockIdx.x;
  const int m0 = (int)(tile / tiles_n) * Cfg::BM;
  const int n0 = (int)(tile % tiles_n) * Cfg::BN;
  const int nchunks = p.K / 64;

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

  Prefetch<Cfg> f;
  load_chunk<Cfg>(p, m0, n0, 0, f);
  store_chunk<Cfg>(lds, f);
  __syncthreads();

  for (int kc = 0; kc < nchunks; ++kc) {
    uint8_t* stage = lds + (kc & 1) * Cfg::kStage;
    if (kc + 1 < nchunks) load_chunk<Cfg>(p, m0, n0, kc + 1, f);

    uint4 qa[FM], qb[FN];
    uint32_t sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int g = wm * FM + i;
      qa[i] = *reinterpret_cast<const uint4*>(stage + g * 1024 + lane * 16);
      sa[i] = *reinterpret_cast<const uint16_t*>(stage + Cfg::kCodesA + Cfg::kCodesB +
                                                 (g * 32 + r) * 4 + h * 2);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int g = wn * FN + j;
      qb[j] = *reinterpret_cast<const uint4*>(stage + Cfg::kCodesA + g * 1024 + lane * 16);
      sb[j] = *reinterpret_cast<const uint16_t*>(stage + Cfg::kCodesA + Cfg::kCodesB +
                                                 Cfg::kScalesA + (g * 32 + r) * 4 + h * 2);
    }
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      half8_t av[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t q = step == 0 ? qa[i].x : step == 1 ? qa[i].y : step == 2 ? qa[i].z : qa[i].w;
        av[i] = decode8(q, e4m3_to_half(step < 2 ? (sa[i] & 0xFFu) : (sa[i] >> 8)));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint32_t q = step == 0 ? qb[j].x : step == 1 ? qb[j].y : step == 2 ? qb[j].z : qb[j].w;
        bv[j] = decode8(q, e4m3_to_half(step < 2 ? (sb[j] & 0xFFu) : (sb[j] >> 8)));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
    }

    if (kc + 1 < nchunks) store_chunk<Cfg>(lds + ((kc + 1) & 1) * Cfg::kStage, f);
    __syncthreads();
  }

  // epilogue: lane holds column n = tile col + r of each FN fragment, rows 8*(i/4) + 4h + i%4
  const float ga = *p.a_g;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * FN * 32 + j * 32 + r;
    if (n >= p.N) continue;
    const float alpha = column_alpha(p.seg, p.seg_g, ga, n);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int mb = m0 + wm * FM * 32 + i * 32 + 4 * h;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int m = mb + 8 * (e / 4) + (e % 4);
        if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, acc[i][j][e] * alpha);
      }
    }
  }
}

template <int WAVES_M, int WAVES_N, int FM, int FN>
hipError_t launch_tiled_cfg(const GemmArgs& a, hipStream_t stream) {
  using Cfg = TileCfg<WAVES_M, WAVES_N, FM, FN>;
  const uint32_t tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM;
  const uint32_t tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
  auto kern = gemm_tiled_kernel<WAVES_M, WAVES_N, FM, FN>;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(Cfg::kThreads), 2 * Cfg::kStage, stream,
                     a, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_general(const GemmArgs& a, hipStream_t stream) {
  const uint32_t tiles_m = (a.M + 63) / 64;
  const uint32_t tiles_n = (a.N + 63) / 64;
  hipLaunchKernelGGL(gemm_general_kernel, dim3(tiles_m * tiles_n), dim3(256), 0, stream, a,
                     tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  return launch_tiled_cfg<2, 2, 2, 2>(a, stream);
}

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  return launch_gemm_general(a, stream);
}

GemmPath choose_gemm_path(int64_t M, int64_t K) {
  if (K % 64 != 0) return GemmPath::General;
  (void)M;
  return GemmPath::Tiled;
}

}  // namespace nvfp4
