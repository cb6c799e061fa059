// W4A4 NVFP4 product for decode-shaped problems (M <= 16 activation rows), gfx950.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Main Findings": decode is weight-bandwidth-bound, so the work here is streaming the NVFP4
// weights once at HBM rate while the few activation rows ride along.
//
// Work split.  One workgroup per compute unit: workgroup b owns the `ncols` output columns
// [b * ncols, (b + 1) * ncols) -- ncols = ceil(N / compute units), so every compute unit streams the
// same number of weight bytes -- as T = 1 or 2 MFMA tiles of 16 columns (the second tile may be
// partly empty), plus all M <= 16 activation rows.  Its 8 wavefronts first copy the tiles' weight
// rows (codes and scales) into LDS with direct global->LDS copies in which each wavefront
// instruction moves 1 KiB of contiguous memory, so the weight stream is fully coalesced.  Each
// wavefront then takes one eighth of every K phase: it reads the weight fragments from LDS and the
// activation fragments from global memory (L2-resident: every workgroup reads the same few rows),
// decodes the activation fragment once and the weight fragments of each tile exactly to f16, and
// contracts with v_mfma_f32_16x16x32_f16 (A = activations padded to 16 rows with zeros, B =
// weights).  The 8 partial 16x16 tiles of each tile are summed through LDS in a fixed order
// (deterministic), scaled per column by 1 / (gA * gW[seg(n)]) and stored.  Every output element
// is accumulated the same way whichever workgroup and tile slot its column falls in.
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
// per wavefront and phase: one weight-code copy per tile and the activation-code load
template <int T>
constexpr int kVmemPerPhase = T + 1;

typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// Issue phase P's copies (weight codes of each tile's 16 rows into its buffer) and this lane's
// activation-code load for its chunk of the phase.  Every wavefront issues exactly
// kVmemPerPhase<T> vector memory instructions per phase, so the wait for phase P is a compile-time
// vmcnt.  Rows past the workgroup's columns load its last column instead (never stored).
template <int P, int T>
__device__ __forceinline__ void issue_phase(const GemmArgs& p, int c0, int clast, int wave,
                                            int lane, int r, int g, uint8_t* buf0, uint8_t* buf1,
                                            uint4& aw) {
  const int kb = p.k_pitch / 2;
  // codes: slot t = wave * 64 + lane holds row t / 32, phase piece (t % 32) ^ row within 16s
  const int t = wave * 64 + lane;
  const int row = t / kPhasePieces;
  const int jl = t - row * kPhasePieces;
  const int j = (jl & ~15) | ((jl ^ row) & 15);
#pragma unroll
  for (int tile = 0; tile < T; ++tile) {
    const int grow = min(c0 + tile * 16 + row, clast);
    __builtin_amdgcn_global_load_lds(p.w_codes + (int64_t)grow * kb + P * (kPhaseK / 2) + j * 16,
                                     (tile == 0 ? buf0 : buf1) + wave * 64 * 16, 16, 0, 0);
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

// Contract this wavefront's chunk of phase data (chunk `wave` of the phase) for each tile: the
// activation fragment is decoded once per MFMA step and used by every tile.
template <int T>
__device__ __forceinline__ void compute_phase(const uint8_t* buf0, const uint8_t* buf1,
                                              const uint8_t* wsc, const uint8_t* asc, int ks,
                                              int c, int wave, int r, int g, bool arow_valid,
                                              const uint4& aw_in, floatx4_t (&acc)[T]) {
  const uint32_t keep = arow_valid ? 0xFFFFFFFFu : 0u;  // padded rows contribute zeros
  const uint4 aw = {aw_in.x & keep, aw_in.y & keep, aw_in.z & keep, aw_in.w & keep};
  const uint32_t as2 = *reinterpret_cast<const uint16_t*>(asc + r * ks + c * 8 + g * 2) & keep;
  const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as2, 1.0f, false);
  const int j = wave * 4 + g;
  const int slot = (r * kPhasePieces + ((j & ~15) | ((j ^ r) & 15))) * 16;
  uint4 ww[T];
  half2_t sw[T];
#pragma unroll
  for (int tile = 0; tile < T; ++tile) {
    ww[tile] = *reinterpret_cast<const uint4*>((tile == 0 ? buf0 : buf1) + slot);
    const uint32_t ws2 =
        *reinterpret_cast<const uint16_t*>(wsc + (tile * 16 + r) * ks + c * 8 + g * 2);
    sw[tile] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws2, 1.0f, false);
  }
  const uint32_t aq[4] = {aw.x, aw.y, aw.z, aw.w};
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const half8_t av = decode8(aq[s2], s2 < 2 ? sa[0] : sa[1]);
#pragma unroll
    for (int tile = 0; tile < T; ++tile) {
      const uint32_t wq = s2 == 0 ? ww[tile].x : s2 == 1 ? ww[tile].y : s2 == 2 ? ww[tile].z
                                                                                   : ww[tile].w;
      const half8_t bv = decode8(wq, s2 < 2 ? sw[tile][0] : sw[tile][1]);
      acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[tile], 0, 0, 0);
    }
  }
}

// K = NPH * 1024.  Every phase of every tile has its own statically named LDS buffer, and all
// copies are issued before any phase is computed: the compiler sees which buffer each read depends
// on, so phase P is computed as soon as its own copies (and activation loads) have landed while
// later phases are still streaming in.
template <int NPH, int T>
__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_kernel(GemmArgs p, int ncols) {
  __shared__ floatx4_t partial[T > 1 ? 2 : 1][kSkinnyWaves][64];
  // block scales of the (up to) 32 weight rows and of up to 16 activation rows, [rows][K/16]
  // (sized for the largest K: a template-dependent size here is miscompiled by the host pass)
  __shared__ __attribute__((aligned(16))) uint8_t wsc[32 * (kSkinnyMaxK / 16)];
  __shared__ __attribute__((aligned(16))) uint8_t asc[16 * (kSkinnyMaxK / 16)];
  __shared__ __attribute__((aligned(16))) uint8_t b0[kPhaseBytes];
  __shared__ __attribute__((aligned(16))) uint8_t b1[NPH > 1 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b2[NPH > 2 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b3[NPH > 3 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b4[NPH > 4 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b5[NPH > 5 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b6[NPH > 6 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t b7[NPH > 7 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c0b[T > 1 ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c1b[(T > 1 && NPH > 1) ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c2b[(T > 1 && NPH > 2) ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c3b[(T > 1 && NPH > 3) ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c4b[(T > 1 && NPH > 4) ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c5b[(T > 1 && NPH > 5) ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c6b[(T > 1 && NPH > 6) ? kPhaseBytes : 16];
  __shared__ __attribute__((aligned(16))) uint8_t c7b[(T > 1 && NPH > 7) ? kPhaseBytes : 16];
  uint8_t* const bufs0[8] = {b0, b1, b2, b3, b4, b5, b6, b7};
  uint8_t* const bufs1[8] = {c0b, c1b, c2b, c3b, c4b, c5b, c6b, c7b};

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;  // weight row (output column) and activation row of this lane
  const int g = lane >> 4;  // k group
  const int c0 = blockIdx.x * ncols;
  const int cend = min(c0 + ncols, p.N);
  const int clast = cend - 1;
  const bool arow_valid = r < p.M;

  // all block scales of the weight rows and of the M activation rows, copied once (coalesced:
  // 16-byte pieces of consecutive rows); older than every phase's instructions, so each phase's
  // wait covers them
  {
    const int ks = p.k_pitch / 16, per_row = p.K / 256;  // row pitch; 16-byte pieces per row
#pragma unroll
    for (int s = threadIdx.x; s < T * 16 * per_row; s += kSkinnyThreads) {
      const int row = s / per_row;
      const int grow = min(c0 + row, clast);
      __builtin_amdgcn_global_load_lds(p.w_scales + (int64_t)grow * ks + (s - row * per_row) * 16,
                                       wsc + (s & ~63) * 16, 16, 0, 0);
    }
    const int s = threadIdx.x;
    if (s < p.M * per_row) {
      const int row = s / per_row;
      __builtin_amdgcn_global_load_lds(p.a_scales + (int64_t)row * ks + (s - row * per_row) * 16,
                                       asc + (s & ~63) * 16, 16, 0, 0);
    }
  }
  // global scales for the epilogue factors 1 / (gA * gW[seg(n)]) of this lane's columns: issued
  // here as vector loads, older than every phase's copies (so the phase waits cover them), and
  // used only at the end -- nothing waits on them before the weight stream is under way
  int zero = 0;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(zero));  // a lane-varying index keeps the gA load a vector load
#endif
  const float ga = p.a_g[zero];
  float gw[T];
#pragma unroll
  for (int tile = 0; tile < T; ++tile)
    gw[tile] = p.seg_g[column_segment(p.seg, min(c0 + tile * 16 + r, clast))];
  __builtin_amdgcn_sched_barrier(0);

  uint4 aw[8];  // entries >= NPH are never touched
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    switch (q) {  // compile-time after unrolling
      case 0: issue_phase<0, T>(p, c0, clast, wave, lane, r, g, bufs0[0], bufs1[0], aw[0]); break;
      case 1: issue_phase<1, T>(p, c0, clast, wave, lane, r, g, bufs0[1], bufs1[1], aw[1]); break;
      case 2: issue_phase<2, T>(p, c0, clast, wave, lane, r, g, bufs0[2], bufs1[2], aw[2]); break;
      case 3: issue_phase<3, T>(p, c0, clast, wave, lane, r, g, bufs0[3], bufs1[3], aw[3]); break;
      case 4: issue_phase<4, T>(p, c0, clast, wave, lane, r, g, bufs0[4], bufs1[4], aw[4]); break;
      case 5: issue_phase<5, T>(p, c0, clast, wave, lane, r, g, bufs0[5], bufs1[5], aw[5]); break;
      case 6: issue_phase<6, T>(p, c0, clast, wave, lane, r, g, bufs0[6], bufs1[6], aw[6]); break;
      default: issue_phase<7, T>(p, c0, clast, wave, lane, r, g, bufs0[7], bufs1[7], aw[7]); break;
    }
  }

  floatx4_t acc[T];
#pragma unroll
  for (int tile = 0; tile < T; ++tile) acc[tile] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  constexpr int V = kVmemPerPhase<T>;
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    // phase q has landed once only the later phases' instructions are outstanding
    __builtin_amdgcn_sched_barrier(0);
    switch (NPH - 1 - q) {
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<1 * V>(); break;
      case 2: wait_vmcnt<2 * V>(); break;
      case 3: wait_vmcnt<3 * V>(); break;
      case 4: wait_vmcnt<4 * V>(); break;
      case 5: wait_vmcnt<5 * V>(); break;
      case 6: wait_vmcnt<6 * V>(); break;
      default: wait_vmcnt<7 * V>(); break;
    }
    __builtin_amdgcn_s_barrier();  // every wavefront's copies of phase q have landed
    __builtin_amdgcn_sched_barrier(0);
    compute_phase<T>(bufs0[q], bufs1[q], wsc, asc, p.K / 16, q * (kPhaseK / 128) + wave, wave, r,
                     g, arow_valid, aw[q], acc);
  }

  // deterministic reduction of the 8 partial tiles of each tile: wavefront `tile` adds the 8 in
  // order
#pragma unroll
  for (int tile = 0; tile < T; ++tile) partial[tile][wave][lane] = acc[tile];
  __syncthreads();
  if (wave >= T) return;
  floatx4_t sum = partial[wave][0][lane];
#pragma unroll
  for (int w = 1; w < kSkinnyWaves; ++w) sum += partial[wave][w][lane];

  // output tile `wave`: lane holds column c0 + 16 * wave + (l % 16), rows 4 * (l / 16) + e
  const int n = c0 + wave * 16 + r;
  if (n >= cend) return;
  const float al = 1.0f / (ga * (wave == 0 ? gw[0] : gw[T - 1]));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int m = 4 * g + e;
    if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, sum[e] * al);
  }
}

}  // namespace

// One workgroup per compute unit when two tiles per workgroup suffice and fit in LDS (K up to
// 7168): ncols = ceil(N / compute units) columns each, so every compute unit streams the same
// number of weight bytes.  Otherwise tiles of 16 columns, one per workgroup.
template <int NPH>
hipError_t launch_skinny_nph(const GemmArgs& a, int cus, hipStream_t stream) {
  const dim3 block(kSkinnyThreads);
  const int per_cu = (a.N + cus - 1) / cus;
  if (NPH <= 7 && per_cu > 16) {
    const int ncols = per_cu <= 32 ? per_cu : 32;
    const dim3 grid((a.N + ncols - 1) / ncols);
    hipLaunchKernelGGL((gemm_skinny_kernel<NPH, (NPH <= 7 ? 2 : 1)>), grid, block, 0, stream, a,
                       ncols);
  } else {
    const dim3 grid((a.N + 15) / 16);
    hipLaunchKernelGGL((gemm_skinny_kernel<NPH, 1>), grid, block, 0, stream, a, 16);
  }
  return hipGetLastError();
}

static hipError_t launch_skinny_piece(const GemmArgs& a, int cus, hipStream_t stream) {
  switch (a.K / kPhaseK) {
    case 1: return launch_skinny_nph<1>(a, cus, stream);
    case 2: return launch_skinny_nph<2>(a, cus, stream);
    case 3: return launch_skinny_nph<3>(a, cus, stream);
    case 4: return launch_skinny_nph<4>(a, cus, stream);
    case 5: return launch_skinny_nph<5>(a, cus, stream);
    case 6: return launch_skinny_nph<6>(a, cus, stream);
    case 7: return launch_skinny_nph<7>(a, cus, stream);
    case 8: return launch_skinny_nph<8>(a, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

// Decode-shaped products.  Up to 32 columns per compute unit and K up to kSkinnyMaxK: this
// kernel, in one pass.  More columns, or K up to kStreamMaxK: the streaming kernels
// (gemm_stream.hip), which keep their weight copies always in flight.  K beyond that
// (f32 output only): the streaming kernel on the fewest pieces of K of at most 8 phases, as equal
// as possible; the first piece writes C and each later one, launched after it on the same stream,
// adds its scaled partial product: C = fl(...fl(acc_0 a) + acc_1 a ...).  (Pieces are slower than
// one pass at K = 17408, N = 5120: every piece meets the uneven share of 320 tiles among the
// compute units again.)
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  cus = cus > 0 ? cus : 1;
  const int per_cu = (a.N + cus - 1) / cus;
  if (a.K <= kSkinnyMaxK && per_cu <= 32) return launch_skinny_piece(a, cus, stream);
  if (a.K <= kStreamMaxK) return launch_gemm_stream(a, stream);
  const int phases = a.K / kPhaseK;
  const int pieces = (phases + 7) / 8;
  int k0 = 0;
  for (int i = 0; i < pieces; ++i) {
    const int nph = phases / pieces + (i < phases % pieces ? 1 : 0);
    GemmArgs b = a;
    b.a_codes = a.a_codes + k0 / 2;
    b.a_scales = a.a_scales + k0 / 16;
    b.w_codes = a.w_codes + k0 / 2;
    b.w_scales = a.w_scales + k0 / 16;
    b.K = nph * kPhaseK;
    b.k_pitch = a.K;
    b.c_accumulate = i > 0 ? 1 : 0;
    e = launch_gemm_stream(b, stream);
    if (e != hipSuccess) return e;
    k0 += b.K;
  }
  return hipSuccess;
}

}  // namespace nvfp4
