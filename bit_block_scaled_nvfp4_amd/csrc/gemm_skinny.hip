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
constexpr int kPhaseK = 1024;                    // K elements per phase (8 chunks of 128)
constexpr int kPhasePieces = kPhaseK / 32;       // 16-byte code pieces per row per phase (32)
constexpr int kPhaseCodes = 16 * kPhasePieces;   // code slots per phase (512 = one per thread)
constexpr int kPhaseScaleBytes = kPhaseK / 16;   // scale bytes per row per phase (64)
constexpr int kPhaseBytes = kPhaseCodes * 16;   // 8 KiB of codes per phase
constexpr int kVmemPerPhase = 2;  // per wavefront: weight-code copy, activation-code load

typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// Issue phase P's copy (weight codes of the 16 rows into `buf`) and this lane's activation-code
// load for its chunk of the phase.  Every wavefront issues exactly kVmemPerPhase vector memory
// instructions per phase, so the wait for phase P is a compile-time vmcnt.
template <int P>
__device__ __forceinline__ void issue_phase(const GemmArgs& p, int n0, int wave, int lane, int r,
                                            int g, uint8_t* buf, uint4& aw) {
  const int kb = p.K / 2;
  // codes: slot t = wave * 64 + lane holds row t / 32, phase piece (t % 32) ^ row within 16s
  {
    const int t = wave * 64 + lane;
    const int row = t / kPhasePieces;
    const int jl = t - row * kPhasePieces;
    const int j = (jl & ~15) | ((jl ^ row) & 15);
    const int grow = min(n0 + row, p.N - 1);
    __builtin_amdgcn_global_load_lds(p.w_codes + (int64_t)grow * kb + P * (kPhaseK / 2) + j * 16,
                                     buf + wave * 64 * 16, 16, 0, 0);
  }
  // this lane's activation fragment for chunk `wave` of the phase; rows >= M load the last row
  // (unconditionally, so no register merge forces an early wait) and are zeroed at use
  {
    const int c = P * (kPhaseK / 128) + wave;
    const int arow = min(r, p.M - 1);
    aw = *reinterpret_cast<const uint4*>(p.a_codes + (int64_t)arow * kb + c * 64 + g * 16);
  }
  // keep the phases' memory instructions in phase order (the waits count on it)
  __builtin_amdgcn_sched_barrier(0);
}

// Contract this wavefront's chunk of phase data in `buf` (chunk `wave` of the phase).
__device__ __forceinline__ void compute_phase(const uint8_t* buf, const uint8_t* wsc,
                                              const uint8_t* asc, int ks, int c, int wave, int r,
                                              int g, bool arow_valid, const uint4& aw_in,
                                              floatx4_t& acc) {
  const uint32_t keep = arow_valid ? 0xFFFFFFFFu : 0u;  // padded rows contribute zeros
  const uint4 aw = {aw_in.x & keep, aw_in.y & keep, aw_in.z & keep, aw_in.w & keep};
  const uint32_t as2 = *reinterpret_cast<const uint16_t*>(asc + r * ks + c * 8 + g * 2) & keep;
  const int j = wave * 4 + g;
  const uint4 ww = *reinterpret_cast<const uint4*>(
      buf + (r * kPhasePieces + ((j & ~15) | ((j ^ r) & 15))) * 16);
  const uint32_t ws2 = *reinterpret_cast<const uint16_t*>(wsc + r * ks + c * 8 + g * 2);
  const half2_t sw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws2, 1.0f, false);
  const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as2, 1.0f, false);
  const uint32_t wq[4] = {ww.x, ww.y, ww.z, ww.w};
  const uint32_t aq[4] = {aw.x, aw.y, aw.z, aw.w};
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const half8_t bv = decode8(wq[s2], s2 < 2 ? sw[0] : sw[1]);
    const half8_t av = decode8(aq[s2], s2 < 2 ? sa[0] : sa[1]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc, 0, 0, 0);
  }
}

// K = NPH * 1024.  Every phase has its own statically named LDS buffer, and all copies are issued
// before any phase is computed: the compiler sees which buffer each read depends on, so phase P is
// computed as soon as its own copies (and activation loads) have landed while later phases are
// still streaming in.
template <int NPH>
__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_kernel(GemmArgs p) {
  __shared__ floatx4_t partial[kSkinnyWaves][64];
  // block scales of the 16 weight rows and of up to 16 activation rows, [16][K/16] each (sized
  // for the largest K: a template-dependent size here is miscompiled by the host pass)
  __shared__ __attribute__((aligned(16))) uint8_t wsc[16 * (kSkinnyMaxK / 16)];
  __shared__ __attribute__((aligned(16))) uint8_t asc[16 * (kSkinnyMaxK / 16)];
  __shared__ __attribute__((aligned(16))) uint8_t b0[kPhaseBytes];
  __shared__ __attribute__((aligned(16))) uint8_t b1[NPH > 1 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b2[NPH > 2 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b3[NPH > 3 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b4[NPH > 4 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b5[NPH > 5 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b6[NPH > 6 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b7[NPH > 7 ? kPhaseBytes : 16];
  uint8_t* const bufs[8] = {b0, b1, b2, b3, b4, b5, b6, b7};

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;  // weight row (output column) and activation row of this lane
  const int g = lane >> 4;  // k group
  const int n0 = blockIdx.x * 16;
  const bool arow_valid = r < p.M;

  // all block scales of the 16 weight rows and of the M activation rows, copied once (coalesced:
  // 16-byte pieces of consecutive rows); older than every phase's instructions, so each phase's
  // wait covers them
  {
    const int ks = p.K / 16, per_row = ks / 16;
    const int s = threadIdx.x;
    if (s < 16 * per_row) {
      const int row = s / per_row;
      const int grow = min(n0 + row, p.N - 1);
      __builtin_amdgcn_global_load_lds(p.w_scales + (int64_t)grow * ks + (s - row * per_row) * 16,
                                       wsc + (s & ~63) * 16, 16, 0, 0);
    }
    if (s < p.M * per_row) {
      const int row = s / per_row;
      __builtin_amdgcn_global_load_lds(p.a_scales + (int64_t)row * ks + (s - row * per_row) * 16,
                                       asc + (s & ~63) * 16, 16, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  uint4 aw[8];  // entries >= NPH are never touched
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    const int ph = q;
    switch (ph) {  // compile-time after unrolling
      case 0: issue_phase<0>(p, n0, wave, lane, r, g, bufs[0], aw[0]); break;
      case 1: issue_phase<1>(p, n0, wave, lane, r, g, bufs[1], aw[1]); break;
      case 2: issue_phase<2>(p, n0, wave, lane, r, g, bufs[2], aw[2]); break;
      case 3: issue_phase<3>(p, n0, wave, lane, r, g, bufs[3], aw[3]); break;
      case 4: issue_phase<4>(p, n0, wave, lane, r, g, bufs[4], aw[4]); break;
      case 5: issue_phase<5>(p, n0, wave, lane, r, g, bufs[5], aw[5]); break;
      case 6: issue_phase<6>(p, n0, wave, lane, r, g, bufs[6], aw[6]); break;
      default: issue_phase<7>(p, n0, wave, lane, r, g, bufs[7], aw[7]); break;
    }
  }

  floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    const int ph = q;
    // phase ph has landed once only the later phases' instructions are outstanding
    __builtin_amdgcn_sched_barrier(0);
    switch (NPH - 1 - q) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<1 * kVmemPerPhase>(); break;
      case 2: wait_vmcnt<2 * kVmemPerPhase>(); break;
      case 3: wait_vmcnt<3 * kVmemPerPhase>(); break;
      case 4: wait_vmcnt<4 * kVmemPerPhase>(); break;
      case 5: wait_vmcnt<5 * kVmemPerPhase>(); break;
      case 6: wait_vmcnt<6 * kVmemPerPhase>(); break;
      default: wait_vmcnt<7 * kVmemPerPhase>(); break;
    }
    __builtin_amdgcn_s_barrier();  // every wavefront's copies of phase ph have landed
    __builtin_amdgcn_sched_barrier(0);
    compute_phase(bufs[ph], wsc, asc, p.K / 16, ph * (kPhaseK / 128) + wave, wave, r, g,
                  arow_valid, aw[ph], acc);
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
  const dim3 grid(blocks), block(kSkinnyThreads);
  switch (a.K / kPhaseK) {
    case 1: hipLaunchKernelGGL(gemm_skinny_kernel<1>, grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL(gemm_skinny_kernel<2>, grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL(gemm_skinny_kernel<3>, grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL(gemm_skinny_kernel<4>, grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL(gemm_skinny_kernel<5>, grid, block, 0, stream, a); break;
    case 6: hipLaunchKernelGGL(gemm_skinny_kernel<6>, grid, block, 0, stream, a); break;
    case 7: hipLaunchKernelGGL(gemm_skinny_kernel<7>, grid, block, 0, stream, a); break;
    case 8: hipLaunchKernelGGL(gemm_skinny_kernel<8>, grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nvfp4
