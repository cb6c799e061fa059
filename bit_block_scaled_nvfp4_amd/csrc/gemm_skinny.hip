// W4A4 NVFP4 product for decode-shaped problems (M <= 16 activation rows), gfx950.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Main Findings": decode is weight-bandwidth-bound, so the work here is streaming the NVFP4
// weights once at HBM rate while the few activation rows ride along.
//
// A workgroup owns 16 output columns (16 weight rows, all of K) and all M <= 16 activation rows.
// Its 8 wavefronts first copy the 16 weight rows (codes and scales) into LDS with direct
// global->LDS copies in which each wavefront instruction moves 1 KiB of contiguous memory, so the
// weight stream is fully coalesced.  Each wavefront then takes one eighth of K: it reads the
// weight fragments from LDS and the activation fragments from global memory (L2-resident: every
// workgroup reads the same few rows), decodes both exactly to f16 and contracts with
// v_mfma_f32_16x16x32_f16 (A = activations padded to 16 rows with zeros, B = weights).  The 8
// partial 16x16 tiles are summed through LDS in a fixed order (deterministic), scaled per column
// by 1 / (gA * gW[seg(n)]) and stored.
//
// K-slot permutation: in a 16x16x32 MFMA, lane l supplies row/column (l % 16) and 8 of the 32
// k-slots (group g = l / 16).  Within a chunk of 128, lane group g uses the 16 bytes holding
// elements [32g, 32g + 32) of its row, 32-bit word j of them in MFMA step j (j = 0..3); word j
// covers elements 32g + 8j .. +7, inside 16-block 2g + j/2.  Both operands use this map.
//
// LDS layout of the codes: row r, 16-byte piece j (bytes [16j, 16j+16) of the row) sits at slot
// r * P + ((j & ~15) | ((j ^ r) & 15)), P = K/32 pieces per row.  The XOR swizzle spreads the 16
// rows a fragment read touches over all LDS banks; the copy realises it by choosing, for each
// destination slot, which global piece to fetch (a permutation inside 256-byte groups, so each
// copy instruction still reads 1 KiB of contiguous memory).
#include "gemm_common.h"

namespace nvfp4 {
namespace {

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyThreads = kSkinnyWaves * 64;
constexpr int kSkinnyMaxChunks = (int)(kSkinnyMaxK / 128 / kSkinnyWaves);  // per wavefront

typedef float floatx4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t load_u16_global(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ floatx4_t partial[kSkinnyWaves][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;  // weight row (output column) and activation row of this lane
  const int g = lane >> 4;  // k group
  const int n0 = blockIdx.x * 16;
  const int kb = p.K / 2, ks = p.K / 16;
  const int P = p.K / 32;                  // 16-byte code pieces per row
  const int code_slots = 16 * P;
  const int scale_slots = 16 * (ks / 16);  // 16-byte scale pieces of the 16 rows
  uint8_t* const lds_codes = lds;
  uint8_t* const lds_scales = lds + code_slots * 16;

  // 1. coalesced copy of the 16 weight rows into LDS (rows past N are clamped to the last row)
  for (int s0 = wave * 64; s0 < code_slots; s0 += kSkinnyThreads) {
    const int s = s0 + lane;
    if (s < code_slots) {
      const int row = s / P;
      const int jl = s - row * P;
      const int j = (jl & ~15) | ((jl ^ row) & 15);
      const int grow = min(n0 + row, p.N - 1);
      __builtin_amdgcn_global_load_lds(p.w_codes + (int64_t)grow * kb + j * 16,
                                       lds_codes + s0 * 16, 16, 0, 0);
    }
  }
  for (int s0 = wave * 64; s0 < scale_slots; s0 += kSkinnyThreads) {
    const int s = s0 + lane;
    if (s < scale_slots) {
      const int per_row = ks / 16;
      const int row = s / per_row;
      const int grow = min(n0 + row, p.N - 1);
      __builtin_amdgcn_global_load_lds(p.w_scales + (int64_t)grow * ks + (s - row * per_row) * 16,
                                       lds_scales + s0 * 16, 16, 0, 0);
    }
  }

  // 2. this wavefront's share of K; its activation fragments (rows >= M are zero) are loaded now,
  //    so their latency overlaps the weight copies
  const int nchunks = p.K / 128;
  const int per_wave = (nchunks + kSkinnyWaves - 1) / kSkinnyWaves;
  const int c_begin = min(wave * per_wave, nchunks);
  const int count = min(c_begin + per_wave, nchunks) - c_begin;
  const bool arow_valid = r < p.M;
  const uint8_t* ac = p.a_codes + (int64_t)min(r, p.M - 1) * kb + g * 16 + c_begin * 64;
  const uint8_t* asc = p.a_scales + (int64_t)min(r, p.M - 1) * ks + g * 2 + c_begin * 8;
  uint4 aw[kSkinnyMaxChunks];
  uint32_t as2[kSkinnyMaxChunks];
#pragma unroll
  for (int i = 0; i < kSkinnyMaxChunks; ++i) {
    aw[i] = uint4{0u, 0u, 0u, 0u};
    as2[i] = 0u;
    if (i < count && arow_valid) {
      aw[i] = *reinterpret_cast<const uint4*>(ac + i * 64);
      as2[i] = load_u16_global(asc + i * 8);
    }
  }

  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this wavefront's copies and loads have landed
  __syncthreads();                      // ... and every other wavefront's copies

  floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kSkinnyMaxChunks; ++i) {
    if (i < count) {
      const int c = c_begin + i;
      const int j = c * 4 + g;
      const uint4 ww = *reinterpret_cast<const uint4*>(
          lds_codes + (r * P + ((j & ~15) | ((j ^ r) & 15))) * 16);
      const uint32_t ws2 =
          *reinterpret_cast<const uint16_t*>(lds_scales + r * ks + c * 8 + g * 2);
      const half2_t sw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws2, 1.0f, false);
      const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as2[i], 1.0f, false);
      const uint32_t wq[4] = {ww.x, ww.y, ww.z, ww.w};
      const uint32_t aq[4] = {aw[i].x, aw[i].y, aw[i].z, aw[i].w};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) {
        const half8_t bv = decode8(wq[s2], s2 < 2 ? sw[0] : sw[1]);
        const half8_t av = decode8(aq[s2], s2 < 2 ? sa[0] : sa[1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
      }
    }
  }

  // 3. deterministic reduction of the 8 partial tiles: wave 0 adds waves 1..7 in order
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

size_t skinny_lds_bytes(int64_t K) { return (size_t)(16 * (K / 2) + 16 * (K / 16)); }

hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  const uint32_t blocks = (a.N + 15) / 16;
  const size_t lds = skinny_lds_bytes(a.K);
  static bool attr_set = false;  // idempotent; a race between threads is benign
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_skinny_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)skinny_lds_bytes(kSkinnyMaxK));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(gemm_skinny_kernel, dim3(blocks), dim3(kSkinnyThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
